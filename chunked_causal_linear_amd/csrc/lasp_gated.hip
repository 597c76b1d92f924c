// HIP kernels (gfx950 / MI355X) for the gated form: a per-token, per-key-channel
// decay (LASP Appendix A.4, Eq. 24 with the GLA / GateLoop row of Table 5):
//   kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p,   o_p = q_p kv_p.
//
// The gates arrive as log-gates.  Inside a chunk of C = 64 tokens every kernel
// works with b, the inclusive running sum of the chunk's log-gates in base-2
// units (b_r = log2(g_0 ... g_r) per channel).  With m a reference row,
//   o_s = sum_{i<=s} (q_s 2^(b_s - b_m)) . (k_i 2^(b_m - b_i)) v_i + (q_s 2^(b_s)) P_t
// where P_t is the state entering the chunk.  The intra-chunk score products
// run on MFMA over 32x32 tiles with m the first row of the query tile: for a
// key tile left of the query tile both factors are at most 1, so nothing
// overflows whatever the gates.  On a diagonal tile the key factor grows up to
// 2^(b_m - b_(m+31)); a tile whose log-gate drop stays within SPAN2 bits uses
// the same products, any other tile sums its pairs one by one with the exact
// factor 2^(b_s - b_i) <= 1.  The chunk state and its reverse are
//   P_{t+1} = Diag(gam_t) P_t + (K_t 2^(b_last - b))^T V_t,   gam_t = 2^(b_last)
//   R_{t-1} = Diag(gam_t) R_t + (Q_t 2^b)^T dO_t
// carried over segments of G chunks (local kernels) and across segments by a
// scan, as in the decayed form.  The log-gate gradient uses that the map
// depends on the running log-gate B through 2^(B_s - B_i) and 2^(B_s) only:
// dl/dB_u = q_u dq_u - k_u dk_u per channel, and the log-gate of token p enters
// every B_u with u >= p, so dlog_g_p is a suffix sum of these; the part of the
// suffix beyond the chunk is rowsum(R_t . P_{t+1}).
#include "lasp_device.h"

namespace lasp {

constexpr int GC = 64;            // chunk length of the gated kernels

// Workgroups per CU the local-state, output and gradient kernels are built
// for (their LDS allows two, except for float32 at d = 128).
template <typename T, int D> struct WgPerCu {
    static constexpr int N = (sizeof(T) == 4 && D == 128) ? 1 : 2;
};
constexpr float SPAN2 = 80.f;     // largest log2-gate drop inside a factorised diagonal tile

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// bS[r][c] = log2(g_0 ... g_r) for channel c of the chunk whose first log-gate
// row is lg; rows at or past Ct repeat the last valid one (gate 1).  All
// threads take part: NTHR / D parts of the rows per channel, each summed in
// registers, then offset by the totals of the parts before it.  The caller
// synchronizes before anyone reads bS and after anyone last read it.
template <int D> struct LogRows {
    static constexpr int NP = NTHR / D, RP = GC / NP;
    float x[RP];
};

template <int D>
__device__ __forceinline__ void cumlog_load(LogRows<D> &lr, const float *lg, int Ct) {
    constexpr int RP = LogRows<D>::RP;
    const int c = threadIdx.x % D, r0 = (threadIdx.x / D) * RP;
    // the thread's offset, opaque to the compiler: the loads' addresses are
    // then formed here, not hoisted out of the caller's loop into registers
    int off = r0 * D + c;
    asm volatile("" : "+v"(off));
    const float *src = lg + off;
#pragma unroll
    for (int j = 0; j < RP; ++j) lr.x[j] = r0 + j < Ct ? src[j * D] : 0.f;
}

template <int D>
__device__ __forceinline__ void cumlog_scan(float *bS, const LogRows<D> &lr) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int RP = LogRows<D>::RP;
    const int c = threadIdx.x % D, r0 = (threadIdx.x / D) * RP;
    float x[RP];
    x[0] = lr.x[0] * LOG2E;
#pragma unroll
    for (int j = 1; j < RP; ++j) x[j] = x[j - 1] + lr.x[j] * LOG2E;
    bS[(r0 + RP - 1) * D + c] = x[RP - 1];
    __syncthreads();
    float off = 0.f;
    for (int q = RP - 1; q < r0; q += RP) off += bS[q * D + c];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RP; ++j) bS[(r0 + j) * D + c] = x[j] + off;
}

// The same in blocks of 16 rows (fewer registers live; the kernels that use
// it keep their other tiles in registers meanwhile).
template <int D>
__device__ __forceinline__ void chunk_cumlog(float *bS, const float *lg, int Ct) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int RP = LogRows<D>::RP, B = RP < 16 ? RP : 16;
    const int c = threadIdx.x % D, r0 = (threadIdx.x / D) * RP;
    float run = 0.f;
#pragma unroll
    for (int b0 = 0; b0 < RP; b0 += B) {
        float x[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int r = r0 + b0 + j;
            x[j] = r < Ct ? lg[(int64_t)r * D + c] * LOG2E : 0.f;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            run += x[j];
            bS[(r0 + b0 + j) * D + c] = run;
        }
    }
    __syncthreads();
    float off = 0.f;
    for (int q = RP - 1; q < r0; q += RP) off += bS[q * D + c];
    __syncthreads();
    if (off != 0.f) {
#pragma unroll 8
        for (int j = 0; j < RP; ++j) bS[(r0 + j) * D + c] += off;
    }
}

// 16 bytes of V converted values at p.
template <typename T>
__device__ __forceinline__ void store_vec(T *p, const float *f) {
#pragma unroll
    for (int j = 0; j < Tr<T>::VEC; j += 4) store4(p + j, f[j], f[j + 1], f[j + 2], f[j + 3]);
}

struct RowId {
    __device__ int operator()(int j) const { return j; }
};

// Staging of token tiles into LDS, split in two halves so that the loads of
// several tiles (and of the states) are in flight together: raw_load issues a
// thread's 16-byte loads into registers, raw_store scales and writes them.
// Row j of an R-row tile is token row(j) (zero at or past Ct); row form
// dst[j][c], transposed dst[c][j].  Consecutive threads take consecutive
// feature groups of a row (coalesced loads, conflict-free reads of row-major
// LDS tables in the scale functor, which multiplies the V features c.. of
// token r in place: scale(j, r, c, f)).
template <typename T, int D, int R>
struct Raw {
    static constexpr int V = Tr<T>::VEC, PR = D / V, N = R * PR, IT = (N + NTHR - 1) / NTHR;
    uint4 v[IT];
};

__device__ __forceinline__ void unpack16(const uint4 &v, float *f, const float *) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4 &v, float *f, const bf16 *) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <typename T, int D, int R, typename RowF>
__device__ __forceinline__ void raw_load(Raw<T, D, R> &raw, const T *src, int Ct, RowF row) {
    using RW = Raw<T, D, R>;
#pragma unroll
    for (int u = 0; u < RW::IT; ++u) {
        const int i = u * NTHR + threadIdx.x;
        const int j = i / RW::PR, c = (i % RW::PR) * RW::V;
        const int r = row(j);
        raw.v[u] = (i < RW::N && r < Ct) ? *(const uint4 *)(src + (int64_t)r * D + c)
                                         : make_uint4(0u, 0u, 0u, 0u);
    }
}

// dst_row(j) < 0 skips tile row j; otherwise it is written as row dst_row(j).
template <typename T, int D, int R, bool TRANS, typename RowF, typename ScaleF, typename DstF>
__device__ __forceinline__ void raw_store_map(const Raw<T, D, R> &raw, T *dst, int pitch, int Ct,
                                              RowF row, ScaleF scale, DstF dst_row) {
    using RW = Raw<T, D, R>;
    constexpr int V = RW::V;
#pragma unroll
    for (int u = 0; u < RW::IT; ++u) {
        const int i = u * NTHR + threadIdx.x;
        if (i >= RW::N) continue;
        const int j = i / RW::PR, c = (i % RW::PR) * V;
        const int dj = dst_row(j);
        if (dj < 0) continue;
        const int r = row(j);
        float f[V];
        unpack16(raw.v[u], f, (const T *)nullptr);
        if (r < Ct) scale(j, r, c, f);
        if (TRANS) {
#pragma unroll
            for (int e = 0; e < V; ++e) dst[(c + e) * pitch + dj] = fromf<T>(f[e]);
        } else {
            store_vec(dst + dj * pitch + c, f);
        }
    }
}

template <typename T, int D, int R, bool TRANS, typename RowF, typename ScaleF>
__device__ __forceinline__ void raw_store(const Raw<T, D, R> &raw, T *dst, int pitch, int Ct,
                                          RowF row, ScaleF scale) {
    raw_store_map<T, D, R, TRANS>(raw, dst, pitch, Ct, row, scale, RowId());
}

// bf16: raw_store into an unpadded row-major tile in the swizzled placement
// sw_off (tile rows 0 .. R-1; rows dst_row(j) < 0 skipped), read back with
// frag_rows_sw / frag_cols_sw.
template <int D, int R, typename RowF, typename ScaleF, typename DstF = RowId>
__device__ __forceinline__ void raw_store_sw(const Raw<bf16, D, R> &raw, bf16 *dst, int Ct, RowF row,
                                             ScaleF scale, DstF dst_row = DstF()) {
    using RW = Raw<bf16, D, R>;
    constexpr int V = RW::V;
#pragma unroll
    for (int u = 0; u < RW::IT; ++u) {
        const int i = u * NTHR + threadIdx.x;
        if (i >= RW::N) continue;
        const int j = i / RW::PR, c = (i % RW::PR) * V;
        const int dj = dst_row(j);
        if (dj < 0) continue;
        const int r = row(j);
        float f[V];
        unpack16(raw.v[u], f, (const bf16 *)nullptr);
        if (r < Ct) scale(j, r, c, f);
        store_vec(dst + sw_off<D>(dj, c), f);
    }
}

// acc += X[k][m0 + i] Y[k][n0 + j] summed over k < K, X and Y swizzled bf16
// tiles whose rows are the contraction index (transpose reads for both).
template <int D, int K>
__device__ __forceinline__ void gemm_cc(f32x16 &acc, const bf16 *X, int m0, const bf16 *Y, int n0,
                                        const FragOffs<D> &fo) {
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, frag_cols_sw<D, false>(X, fo, k, m0), frag_cols_sw<D, false>(Y, fo, k, n0));
}

// acc += A[m0 + i][k] Y[k][n0 + j] summed over k < K: A bf16 rows with the
// contraction index contiguous (pitch pa), Y a swizzled bf16 tile whose rows
// are the contraction index (transpose reads).
template <int D, int K>
__device__ __forceinline__ void gemm_rc(f32x16 &acc, const bf16 *A, int pa, int m0, const bf16 *Y,
                                        int n0, const FragOffs<D> &fo, int y0 = 0) {
    // (Y's rows y0 .. y0 + K - 1; y0 a multiple of 16)
    const int l = lane_id();
    const bf16 *ap = A + (m0 + (l & 31)) * pa + (l >> 5) * 8;
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, *(const bf16x8_t *)(ap + k), frag_cols_sw<D, false>(Y, fo, y0 + k, n0));
}

// Transposed accumulation (bf16): the same products as gemm / gemm_rc with the
// MFMA operands swapped, so that acc holds the 32x32 tile transposed (lane =
// output row, its 16 values = columns crow(r)); store_tile1_t then writes it
// with 16-byte stores.
template <int K>
__device__ __forceinline__ void gemm_t(f32x16 &acc, const bf16 *As, int pa, int m0, const bf16 *Bs,
                                       int pb, int n0) {
    const int l = lane_id();
    const bf16 *ap = As + (m0 + (l & 31)) * pa + (l >> 5) * 8;
    const bf16 *bp = Bs + (n0 + (l & 31)) * pb + (l >> 5) * 8;
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, *(const bf16x8_t *)(bp + k), *(const bf16x8_t *)(ap + k));
}
template <int D, int K>
__device__ __forceinline__ void gemm_rc_t(f32x16 &acc, const bf16 *A, int pa, int m0, const bf16 *Y,
                                          int n0, const FragOffs<D> &fo) {
    const int l = lane_id();
    const bf16 *ap = A + (m0 + (l & 31)) * pa + (l >> 5) * 8;
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, frag_cols_sw<D, false>(Y, fo, k, n0), *(const bf16x8_t *)(ap + k));
}
// rows m0 + lane%32 (those below nrow), columns n0 .. n0+31 of G (row pitch
// ld) from a transposed accumulator: after one permlane32 exchange each lane
// holds 8 consecutive columns of its row twice over.  The buffer range ends
// at row nrow, so rows past it are dropped by the range check.
__device__ __forceinline__ void store_tile1_t(const f32x16 &acc, bf16 *G, int ld, int m0, int n0,
                                              int nrow) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    const int rows = nrow - m0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        G + (int64_t)m0 * ld + n0, 0, __builtin_amdgcn_readfirstlane(rows > 0 ? rows * ld * 2 : 0),
        0x00020000);
    const int l = lane_id();
    const int off = ((l & 31) * ld + (l >> 5) * 8) * 2;
    unsigned r[8];   // r[2j], r[2j+1]: columns 8j + 4*(lane/32) + [0,4), packed
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const bf16x2_t v = {(__bf16)acc[2 * q], (__bf16)acc[2 * q + 1]};
        r[q] = __builtin_bit_cast(unsigned, v);
    }
#pragma unroll
    for (int q = 0; q < 8; q += 4) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const auto x = __builtin_amdgcn_permlane32_swap(r[q + e], r[q + 2 + e], false, false);
            r[q + e] = x[0];
            r[q + 2 + e] = x[1];
        }
    }
    const u32x4_t v0 = {r[0], r[1], r[2], r[3]}, v1 = {r[4], r[5], r[6], r[7]};
    __builtin_amdgcn_raw_buffer_store_b128(v0, rs, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(v1, rs, off + 32, 0, 0);
}

// f *= 2^(b[GC-1] - b[r]) for a thread's raw_store items, which all sit at the
// same channels c .. c+V-1 (NTHR is a multiple of the pieces per row): the
// reference row's V values are read once.
template <int D, int V>
struct LastRowScale {
    const float *bS;
    float bl[V];
    __device__ LastRowScale(const float *b) : bS(b) {
        const int c = (threadIdx.x % (D / V)) * V;
#pragma unroll
        for (int e = 0; e < V; ++e) bl[e] = bS[(GC - 1) * D + c + e];
    }
    __device__ void operator()(int, int r, int c, float *f) const {
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] *= ex2(bl[e] - bS[r * D + c + e]);
    }
};

struct NoScale {
    template <typename F> __device__ void operator()(int, int, int, F) const {}
};

// Gate factors for raw_store(): f *= 2^(b[ref] - b[r]) (invert: 2^(b[r] - b[ref]));
// ref < 0: f *= 2^(b[r]).
template <int V, typename RefF>
struct GateScale {
    const float *bS;
    RefF ref;
    bool invert;
    int D;
    __device__ void operator()(int j, int r, int c, float *f) const {
        const int m = ref(j);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float br = bS[r * D + c + e];
            const float x = m < 0 ? br : (invert ? br - bS[m * D + c + e] : bS[m * D + c + e] - br);
            f[e] *= ex2(x);
        }
    }
};

template <typename T, typename RefF>
__device__ __forceinline__ GateScale<Tr<T>::VEC, RefF> gate_scale(const float *bS, int D, RefF ref,
                                                                  bool invert = false) {
    return GateScale<Tr<T>::VEC, RefF>{bS, ref, invert, D};
}

// The D x D states entering (or leaving) a chunk, combined from the segment
// state and the local one, NS of them side by side:
//   x_s[dv][dk] = g_s[dk] seg_s[dv][dk] + loc_s[dv][dk]    (loc_s null: 0)
// in the [dv][dk] layout of the state arrays.  f(dv, dk0, x) receives V
// consecutive dk of every state; loads are issued in batches of IB groups.
template <typename T, int D, int NS, int BUDGET = 8, int NDV = D, typename F>
__device__ __forceinline__ void for_states(const float *const *seg, const void *const *loc,
                                           const float *const *g, F f, int dv0 = 0) {
    // rows dv0 .. dv0 + NDV - 1 of the [dv][dk] states
    constexpr int V = Tr<T>::VEC, IT = (NDV * D + NTHR * V - 1) / (NTHR * V);
    constexpr int IB = IT < BUDGET / NS ? IT : BUDGET / NS;
    static_assert(IT % IB == 0, "batches");
    // NTHR * V is a multiple of D: a thread's dk group is the same in every batch
    const int dk0 = (threadIdx.x * V) % D;
    float gg[NS][V];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int j = 0; j < V; j += 4) load16(g[q] + dk0 + j, gg[q] + j);
    for (int b = 0; b < IT; b += IB) {
        uint4 sr[IB][NS][V / 4], lr[IB][NS];
#pragma unroll
        for (int u = 0; u < IB; ++u) {
            const int e = dv0 * D + ((b + u) * NTHR + threadIdx.x) * V;
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const bool in = e < (dv0 + NDV) * D;
#pragma unroll
                for (int j = 0; j < V / 4; ++j)
                    sr[u][q][j] = in ? *(const uint4 *)(seg[q] + e + 4 * j) : make_uint4(0u, 0u, 0u, 0u);
                lr[u][q] = (in && loc[q]) ? *(const uint4 *)((const T *)loc[q] + e)
                                          : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < IB; ++u) {
            const int e = dv0 * D + ((b + u) * NTHR + threadIdx.x) * V;
            if (e >= (dv0 + NDV) * D) continue;
            float x[NS][V];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                float sg[V], lc[V];
#pragma unroll
                for (int j = 0; j < V / 4; ++j) unpack16(sr[u][q][j], sg + 4 * j, (const float *)nullptr);
                unpack16(lr[u][q], lc, (const T *)nullptr);
#pragma unroll
                for (int j = 0; j < V; ++j) x[q][j] = gg[q][j] * sg[j] + lc[j];
            }
            f(e / D, dk0, x);
        }
    }
}

// Span test of the two 32-row tiles of a chunk (uniform over the workgroup).
template <int D>
__device__ __forceinline__ void tile_spans(const float *bS, bool &slow0, bool &slow1) {
    bool s0 = false, s1 = false;
    for (int c = threadIdx.x; c < D; c += NTHR) {
        s0 |= bS[c] - bS[31 * D + c] > SPAN2;
        s1 |= bS[32 * D + c] - bS[63 * D + c] > SPAN2;
    }
    slow0 = __syncthreads_or(s0);
    slow1 = __syncthreads_or(s1);
}

// Exact gated score of query row s and key row i (i <= s, both in the chunk):
// sum_c q_s[c] k_i[c] 2^(b_s[c] - b_i[c]), inputs read from global memory.
template <typename T, int D>
__device__ float exact_score(const T *Q, const T *K, const float *bS, int s, int i) {
    float acc = 0.f;
    for (int c = 0; c < D; ++c)
        acc += tof(Q[(int64_t)s * D + c]) * tof(K[(int64_t)i * D + c]) *
               ex2(bS[s * D + c] - bS[i * D + c]);
    return acc;
}

// ---------------------------------------------------------------------------
// Forward 1: local states, one workgroup per (segment, head), chunks in order
// from a zero state at the segment start:
//   Lc[t] = L, Gc[t] = gate product of the segment's chunks before t;
//   L = Diag(gam_t) L + (K_t 2^(b_last - b))^T V_t;   Z = L, Gs = all gates.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gfwd_local(Params p) {
    // bf16: K and V rows in swizzled row-major tiles, read transposed;
    // float32: transposed copies
    constexpr bool SW = sizeof(T) == 2;
    constexpr int PT = GC + Tr<T>::VEC;
    __shared__ float bS[GC * D];
    __shared__ __attribute__((aligned(16))) T KT_s[SW ? GC * D : D * PT];
    __shared__ __attribute__((aligned(16))) T VT_s[SW ? GC * D : D * PT];
    using TL = Tiles<D / 32, D / 32>;

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb = row_base(p, s, h);
    const T *K = (const T *)p.K + rb * D;
    const T *Vg = (const T *)p.V + rb * D;
    const float *LG = p.LG + rb * D;
    const bool store_local = p.G > 1;

    f32x16 acc[TL::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) zero(acc[k]);
    float gcum = 1.f;   // thread c < D: gate product of channel c

    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    // the next chunk's rows are loaded while the current one is multiplied
    Raw<T, D, GC> rk, rv;
    LogRows<D> rl;
    if (t0 < t1) {
        const int Ct0 = min(GC, s.len - t0 * GC);
        raw_load(rk, K + (int64_t)t0 * GC * D, Ct0, RowId());
        raw_load(rv, Vg + (int64_t)t0 * GC * D, Ct0, RowId());
        cumlog_load<D>(rl, LG + (int64_t)t0 * GC * D, Ct0);
    }
    for (int t = t0; t < t1; ++t) {
        const int tok = t * GC;
        const int Ct = min(GC, s.len - tok);
        const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
        if (store_local) {
            T *Lt = (T *)p.Lc + ch * D * D;
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) store_T(acc[k], Lt, D, mi * 32, ni * 32, Ident());
            }
        }
        if (threadIdx.x < D) p.Gc[ch * D + threadIdx.x] = gcum;
        __syncthreads();
        cumlog_scan<D>(bS, rl);
        __syncthreads();
        if constexpr (SW) {
            static_assert(NTHR % (D / 8) == 0, "a thread's items share their channels");
            raw_store_sw<D, GC>(rk, (bf16 *)KT_s, Ct, RowId(), LastRowScale<D, 8>(bS));
            raw_store_sw<D, GC>(rv, (bf16 *)VT_s, Ct, RowId(), NoScale());
        } else {
            raw_store<T, D, GC, true>(rk, KT_s, PT, Ct, RowId(),
                                      gate_scale<T>(bS, D, [](int) { return GC - 1; }));
            raw_store<T, D, GC, true>(rv, VT_s, PT, Ct, RowId(), NoScale());
        }
        if (t + 1 < t1) {
            const int Cn = min(GC, s.len - tok - GC);
            raw_load(rk, K + (int64_t)(tok + GC) * D, Cn, RowId());
            raw_load(rv, Vg + (int64_t)(tok + GC) * D, Cn, RowId());
            cumlog_load<D>(rl, LG + (int64_t)(tok + GC) * D, Cn);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) {
            int mi, ni;
            if (TL::get(k, mi, ni)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[k][r] *= ex2(bS[(GC - 1) * D + mi * 32 + crow(r)]);
                if constexpr (SW)
                    gemm_cc<D, GC>(acc[k], (const bf16 *)KT_s, mi * 32, (const bf16 *)VT_s, ni * 32,
                                   opaque(frag_offs<D>(lane_id())));
                else
                    gemm<T, GC>(acc[k], KT_s, PT, mi * 32, VT_s, PT, ni * 32);
            }
        }
        if (threadIdx.x < D) gcum *= ex2(bS[(GC - 1) * D + threadIdx.x]);
    }
    const int64_t sh = (int64_t)gs * p.H + h;
    float *Zs = p.Z + sh * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni)) store_T(acc[k], Zs, D, mi * 32, ni * 32, Ident());
    }
    if (threadIdx.x < D) p.Gs[sh * D + threadIdx.x] = gcum;
}

// ---------------------------------------------------------------------------
// Forward 2: scan over segments, one thread per state element:
//   Pseg[0] = M_in;  Pseg[s+1] = Diag(Gs[s]) Pseg[s] + Z[s];  M_out = last.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHR) void k_gfwd_segscan(Params p) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    const int ih = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * NTHR + threadIdx.x;
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;   // [dk][dv] of the API states
    float P = p.M_in ? p.M_in[mo] : 0.f;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    for (int sl = 0; sl < nS; ++sl) {
        const int64_t sh = (int64_t)(s.s0 + sl) * p.H + h;
        p.Pseg[sh * D * D + e] = P;
        P = p.Gs[sh * D + dk] * P + p.Z[sh * D * D + e];
    }
    if (p.M_out) p.M_out[mo] = P;
}

// ---------------------------------------------------------------------------
// Forward 3: output, one workgroup per (chunk, head).
//   O = (Q 2^b) P_t + sum over tile pairs J <= I of
//       [(Q_I 2^(b - b_mI)) (K_J 2^(b_mI - b))^T masked] V_J
// ---------------------------------------------------------------------------
// LDS plan of the output kernel: the running log-gates (float32) and one
// scratch area reused by three phases, small enough for two workgroups per CU:
//   1  Q 2^b rows | P_t^T rows (half of them at a time when d = 128)
//   2  Q_I 2^(b - b_mI) rows | K rows 0..63 (ref 32; then rows 0..31 with ref 0) | scores
//   3  V^T | (scores)
template <typename T, int D> struct OutLds {
    static constexpr int V = Tr<T>::VEC, PD = D + V, PS = GC + V;
    static constexpr int NHALF = D * PD * (int)sizeof(T) > 20000 ? 2 : 1, DH = D / NHALF;
    static constexpr int ROWS = GC * PD, SOFF = 2 * ROWS;
    static constexpr int P1 = ROWS + DH * PD, P2 = SOFF + GC * PS;
    static constexpr int ELEMS = P1 > P2 ? P1 : P2;
    static_assert(D * PS <= SOFF, "V^T must not reach the scores");
};

template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gfwd_out(Params p) {
    using L = OutLds<T, D>;
    constexpr int PD = L::PD, PS = L::PS, DH = L::DH;
    __shared__ float bS[GC * D];
    __shared__ __attribute__((aligned(16))) T U[L::ELEMS];
    using TO = Tiles<GC / 32, D / 32>;

    // consecutive workgroups (on one XCD) take consecutive chunks of one head:
    // the chunks of a segment then read its segment states from that XCD's L2
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid / p.n_chunks_ub, gc = lid % p.n_chunks_ub;
    if (h >= p.H) return;
    Seq s;
    int t;
    if (!chunk_seq(p, gc, s, t)) return;
    const int tok = t * GC;
    const int Ct = min(GC, s.len - tok);
    const int sl = t / p.G;
    if (s.s0 + sl >= p.n_segs_ub) return;   // only with malformed cu_seqlens
    const int64_t rb = row_base(p, s, h) + tok;
    const T *Q = (const T *)p.Q + rb * D;
    const T *K = (const T *)p.K + rb * D;
    const T *Vg = (const T *)p.V + rb * D;
    T *O = (T *)p.O + rb * D;
    const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
    const int64_t sh = (int64_t)(s.s0 + sl) * p.H + h;
    const int w = wave_id(), l = lane_id();

    // every token load of the kernel, issued up front
    auto krow = [](int j) { return j < 64 ? (j & 31) : j - 32; };   // K rows: (0|ref 0), (0|32), (1|32)
    Raw<T, D, GC> rq, rv;
    Raw<T, D, 96> rk;
    raw_load(rq, Q, Ct, RowId());
    raw_load(rk, K, Ct, krow);
    raw_load(rv, Vg, Ct, RowId());
    chunk_cumlog<D>(bS, p.LG + rb * D, Ct);

    // 1: o = (Q 2^b) P_t
    T *Qh = U, *Ph = U + L::ROWS;
    f32x16 o[TO::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TO::PER_WAVE; ++k) zero(o[k]);
    {
        const float *seg[1] = {p.Pseg + sh * D * D};
        const void *loc[1] = {p.G > 1 ? (const void *)((const T *)p.Lc + ch * D * D) : nullptr};
        const float *g[1] = {p.Gc + ch * D};
        for (int hh = 0; hh < L::NHALF; ++hh) {
            const int dv0 = hh * DH;
            if (hh) __syncthreads();
            for_states<T, D, 1, 8, DH>(seg, loc, g, [&](int dv, int dk, const float (*x)[Tr<T>::VEC]) {
                store_vec(Ph + (dv - dv0) * PD + dk, x[0]);
            }, dv0);
            if (!hh)
                raw_store<T, D, GC, false>(rq, Qh, PD, Ct, RowId(),
                                           gate_scale<T>(bS, D, [](int) { return -1; }));
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni) && ni * 32 >= dv0 && ni * 32 < dv0 + DH) {
                    // (bf16: O accumulated transposed)
                    if constexpr (sizeof(T) == 2)
                        gemm_t<D>(o[k], (const bf16 *)Qh, PD, mi * 32, (const bf16 *)Ph, PD, ni * 32 - dv0);
                    else
                        gemm<T, D>(o[k], Qh, PD, mi * 32, Ph, PD, ni * 32 - dv0);
                }
            }
        }
    }
    __syncthreads();

    // 2: masked gated scores into Sc
    T *Qt = U, *K64 = U + L::ROWS, *Sc = U + L::SOFF;
    raw_store<T, D, GC, false>(rq, Qt, PD, Ct, RowId(),
                               gate_scale<T>(bS, D, [](int j) { return j & ~31; }, true));
    raw_store_map<T, D, 96, false>(rk, K64, PD, Ct, krow,
                                   gate_scale<T>(bS, D, [](int j) { return j < 32 ? 0 : 32; }),
                                   [](int j) { return j - 32; });   // rows 0..63 with ref 32
    bool slow0, slow1;
    tile_spans<D>(bS, slow0, slow1);   // (its barrier also ends the staging)
    auto score_tile = [&](int I, int J, int krow0, bool slow) __attribute__((always_inline)) {
        f32x16 st;
        zero(st);
        if (!slow) gemm<T, D>(st, Qt, PD, 32 * I, K64, PD, krow0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qs = 32 * I + crow(r), ki = 32 * J + (l & 31);
            float x = 0.f;
            if (qs < Ct && ki < Ct && ki <= qs) x = slow ? exact_score<T, D>(Q, K, bS, qs, ki) : st[r];
            Sc[qs * PS + ki] = fromf<T>(x);
        }
    };
    if (w == 1) score_tile(1, 0, 0, false);
    if (w == 2) score_tile(1, 1, 32, slow1);
    if (w == 3) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Sc[crow(r) * PS + 32 + (l & 31)] = fromf<T>(0.f);
    }
    __syncthreads();
    raw_store_map<T, D, 96, false>(rk, K64, PD, Ct, krow,
                                   gate_scale<T>(bS, D, [](int) { return 0; }),
                                   [](int j) { return j < 32 ? j : -1; });   // rows 0..31 with ref 0
    __syncthreads();
    if (w == 0) score_tile(0, 0, 0, slow0);
    __syncthreads();

    // 3: o += Sc V (bf16: V rows in a swizzled tile, read transposed;
    // float32: a transposed copy)
    constexpr bool SW = sizeof(T) == 2;
    static_assert(GC * D <= L::SOFF, "V must not reach the scores");
    T *VT = U;
    if constexpr (SW)
        raw_store_sw<D, GC>(rv, (bf16 *)VT, Ct, RowId(), NoScale());
    else
        raw_store<T, D, GC, true>(rv, VT, PS, Ct, RowId(), NoScale());
    __syncthreads();
    const FragOffs<D> fo = frag_offs<D>(l);
#pragma unroll
    for (int k = 0; k < TO::PER_WAVE; ++k) {
        int mi, ni;
        if (TO::get(k, mi, ni)) {
            if constexpr (SW) {
                gemm_rc_t<D, GC>(o[k], (const bf16 *)Sc, PS, mi * 32, (const bf16 *)VT, ni * 32, fo);
                store_tile1_t(o[k], (bf16 *)O, D, mi * 32, ni * 32, Ct);
            } else {
                gemm<T, GC>(o[k], Sc, PS, mi * 32, VT, PS, ni * 32);
                store_rows(o[k], O, D, mi * 32, ni * 32, Ct);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward 1: local reverse states, one workgroup per (segment, head), chunks
// last to first from a zero state at the segment end:
//   Rc[t] = R, Hc[t] = gate product of the segment's chunks after t;
//   R = Diag(gam_t) R + (Q_t 2^b)^T dO_t;   W = R.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gbwd_local(Params p) {
    constexpr bool SW = sizeof(T) == 2;   // as in k_gfwd_local
    constexpr int PT = GC + Tr<T>::VEC;
    __shared__ float bS[GC * D];
    __shared__ __attribute__((aligned(16))) T QT_s[SW ? GC * D : D * PT];
    __shared__ __attribute__((aligned(16))) T OT_s[SW ? GC * D : D * PT];
    using TL = Tiles<D / 32, D / 32>;
    const FragOffs<D> fo = frag_offs<D>(lane_id());

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb = row_base(p, s, h);
    const T *Q = (const T *)p.Q + rb * D;
    const T *dO = (const T *)p.dO + rb * D;
    const float *LG = p.LG + rb * D;
    const bool store_local = p.G > 1;

    f32x16 acc[TL::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) zero(acc[k]);
    float hcum = 1.f;

    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    Raw<T, D, GC> rq, ro;   // the next (earlier) chunk's rows, loaded ahead
    LogRows<D> rl;
    if (t0 < t1) {
        const int tl = (t1 - 1) * GC, Cl = min(GC, s.len - tl);
        raw_load(rq, Q + (int64_t)tl * D, Cl, RowId());
        raw_load(ro, dO + (int64_t)tl * D, Cl, RowId());
        cumlog_load<D>(rl, LG + (int64_t)tl * D, Cl);
    }
    for (int t = t1 - 1; t >= t0; --t) {
        const int tok = t * GC;
        const int Ct = min(GC, s.len - tok);
        const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
        if (store_local) {
            T *Rt = (T *)p.Rc + ch * D * D;
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) store_T(acc[k], Rt, D, mi * 32, ni * 32, Ident());
            }
        }
        if (threadIdx.x < D) p.Hc[ch * D + threadIdx.x] = hcum;
        __syncthreads();
        cumlog_scan<D>(bS, rl);
        __syncthreads();
        if constexpr (SW) {
            raw_store_sw<D, GC>(rq, (bf16 *)QT_s, Ct, RowId(),
                                gate_scale<T>(bS, D, [](int) { return -1; }));
            raw_store_sw<D, GC>(ro, (bf16 *)OT_s, Ct, RowId(), NoScale());
        } else {
            raw_store<T, D, GC, true>(rq, QT_s, PT, Ct, RowId(),
                                      gate_scale<T>(bS, D, [](int) { return -1; }));
            raw_store<T, D, GC, true>(ro, OT_s, PT, Ct, RowId(), NoScale());
        }
        if (t - 1 >= t0) {   // chunk t - 1 is full
            raw_load(rq, Q + (int64_t)(tok - GC) * D, GC, RowId());
            raw_load(ro, dO + (int64_t)(tok - GC) * D, GC, RowId());
            cumlog_load<D>(rl, LG + (int64_t)(tok - GC) * D, GC);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) {
            int mi, ni;
            if (TL::get(k, mi, ni)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[k][r] *= ex2(bS[(GC - 1) * D + mi * 32 + crow(r)]);
                if constexpr (SW)
                    gemm_cc<D, GC>(acc[k], (const bf16 *)QT_s, mi * 32, (const bf16 *)OT_s, ni * 32, fo);
                else
                    gemm<T, GC>(acc[k], QT_s, PT, mi * 32, OT_s, PT, ni * 32);
            }
        }
        if (threadIdx.x < D) hcum *= ex2(bS[(GC - 1) * D + threadIdx.x]);
    }
    float *Ws = p.W + ((int64_t)gs * p.H + h) * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni)) store_T(acc[k], Ws, D, mi * 32, ni * 32, Ident());
    }
}

// ---------------------------------------------------------------------------
// Backward 2: reverse scan over segments, one thread per state element:
//   Rseg[S-1] = dM_out;  Rseg[s-1] = Diag(Gs[s]) Rseg[s] + W[s];  dM_in = last.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHR) void k_gbwd_segscan(Params p) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    const int ih = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * NTHR + threadIdx.x;
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;
    float R = p.dM_out ? p.dM_out[mo] : 0.f;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    for (int sl = nS - 1; sl >= 0; --sl) {
        const int64_t sh = (int64_t)(s.s0 + sl) * p.H + h;
        p.Rseg[sh * D * D + e] = R;
        R = p.Gs[sh * D + dk] * R + p.W[sh * D * D + e];
    }
    if (p.dM_in) p.dM_in[mo] = R;
}

// ---------------------------------------------------------------------------
// Backward 3: gradients, one workgroup per (chunk, head), with D_ = dO V^T:
//   dQ = 2^b . (dO P_t^T) + sum_{J<=I} 2^(b - b_mI) . ([D_ masked]_IJ (K_J 2^(b_mI - b)))
//   dV = (K 2^(b_last - b)) R_t + sum_{I>=J} [A masked]_IJ^T dO_I   (A: the gated scores)
//   dK = 2^(b_last - b) . (V R_t^T)
//        + sum_{I>=J} 2^(b_mJ' - b) . ([D_ masked]_IJ^T (Q_I 2^(b - b_mJ')))
//   dlog_g[s] = sum_{u>=s in chunk} (q_u dq_u - k_u dk_u) + rowsum(R_t . P_{t+1})
// with m_I the first row of query tile I and m'_J the last row of key tile J.
// ---------------------------------------------------------------------------
// LDS plan of the gradient kernel: the running log-gates (float32), two small
// per-channel sums and one scratch area reused by every phase, small enough
// for two workgroups per CU.  A d x d state operand is staged in NHALF parts
// (d = 128): split along the contraction index where the product allows it
// (dQ's dO P_t^T, dK's V R_t^T), along the output columns otherwise (dV's
// K R_t).  Score tiles are formed before the next product's operands are
// staged over the rows they came from.
template <typename T, int D>
struct GradLds {
    static constexpr int V = Tr<T>::VEC, PD = D + V, PS = GC + V, PK = 96 + V;
    static constexpr int NHALF = D * PD * (int)sizeof(T) > 20000 ? 2 : 1, DH = D / NHALF;
    static constexpr int PDH = DH + V;                    // pitch of a contraction-split part
    static constexpr int ROWS = GC * PD, SC = GC * PS, SOFF = 2 * ROWS;
    static constexpr int CPART = D * PDH, RPART = DH * PD;
    static constexpr int RP = NTHR * V * 4 / (int)sizeof(T);   // float partial sums of rho
    static constexpr int A1 = ROWS + CPART + RP;          // dO rows, P part, rho partials
    static constexpr int B1 = RPART + ROWS;               // R part, K rows
    static constexpr int C1 = ROWS + CPART;               // V rows, R^T part
    static constexpr int S2 = SOFF + SC;                  // two row arrays + scores
    static constexpr int M1 = A1 > B1 ? A1 : B1, M2 = C1 > S2 ? C1 : S2;
    static constexpr int ELEMS = M1 > M2 ? M1 : M2;
    static constexpr int BYTES = ELEMS * (int)sizeof(T) > GC * D * 4 ? ELEMS * (int)sizeof(T) : GC * D * 4;
    static_assert(D * PK <= SOFF && D * PS <= SOFF, "K^T / Q^T / dO^T must not reach the scores");
};

template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gbwd_grads(Params p) {
    using L = GradLds<T, D>;
    constexpr int V = Tr<T>::VEC, PD = L::PD, PS = L::PS, PK = L::PK, DH = L::DH, PDH = L::PDH;
    constexpr bool SW = sizeof(T) == 2;   // bf16: transpose reads of row tiles
    static_assert(96 * D <= L::SOFF, "K / Q rows must not reach the scores");
    static_assert(!SW || DH * D <= L::CPART, "swizzled state parts fit the transposed ones' space");
    __shared__ float bS[GC * D];
    __shared__ float rho[D], Ep[D];
    __shared__ __attribute__((aligned(16))) char U_raw[L::BYTES];
    T *U = (T *)U_raw;
    T *Sc = U + L::SOFF;   // score tiles (every phase)
    using TO = Tiles<GC / 32, D / 32>;

    // consecutive workgroups (on one XCD) take consecutive chunks of one head:
    // the chunks of a segment then read its segment states from that XCD's L2
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid / p.n_chunks_ub, gc = lid % p.n_chunks_ub;
    if (h >= p.H) return;
    Seq s;
    int t;
    if (!chunk_seq(p, gc, s, t)) return;
    const int tok = t * GC;
    const int Ct = min(GC, s.len - tok);
    const int sl = t / p.G;
    if (s.s0 + sl >= p.n_segs_ub) return;
    const int64_t rb = row_base(p, s, h) + tok;
    const T *Q = (const T *)p.Q + rb * D;
    const T *K = (const T *)p.K + rb * D;
    const T *Vg = (const T *)p.V + rb * D;
    const T *dO = (const T *)p.dO + rb * D;
    const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
    const int64_t sh = (int64_t)(s.s0 + sl) * p.H + h;
    const float *Ps = p.Pseg + sh * D * D, *Rs = p.Rseg + sh * D * D;
    const void *Lt = p.G > 1 ? (const void *)((const T *)p.Lc + ch * D * D) : nullptr;
    const void *Rt = p.G > 1 ? (const void *)((const T *)p.Rc + ch * D * D) : nullptr;
    const float *gP = p.Gc + ch * D, *gR = p.Hc + ch * D;
    const int w = wave_id(), l = lane_id();
    auto krow = [](int j) { return j < 64 ? (j & 31) : j - 32; };   // K rows of the 3 versions
    auto qrow = [](int j) { return j < 64 ? j : j - 32; };          // Q rows of the 3 versions
    // token rows in registers, loaded a phase ahead of their use (reloaded
    // from L2 rather than kept live across phases: registers bound the
    // workgroups per CU)
    chunk_cumlog<D>(bS, p.LG + rb * D, Ct);   // (its registers are free before the rows load)
    if (threadIdx.x < D) Ep[threadIdx.x] = 0.f;
    Raw<T, D, GC> rdo, rv, rkq;
    Raw<T, D, 96> rk96;
    raw_load(rdo, dO, Ct, RowId());
    raw_load(rv, Vg, Ct, RowId());
    raw_load(rk96, K, Ct, krow);
    bool slow0 = false, slow1 = false;
    // Masked 32x32 score tiles A_a . B_b^T into Sc: tiles (a, b) = (0,0), (1,0),
    // (1,1) (lower: b <= a kept) or (0,0), (0,1), (1,1) (upper: b >= a kept),
    // the tiles of mask bit w (bit i: tile i) on waves 0..2; wave 3 zeroes the
    // remaining block when zero_block.  B's rows for tile i start at brow(i).
    // Gated diagonal tiles over the span limit take exact(a, b) instead of the
    // product.  tr stores Sc[b][a].
    auto scores = [&](const T *A, const T *B, auto brow, bool upper, bool tr, bool gated,
                      auto exact, int mask, bool zero_block) __attribute__((always_inline)) {
        if (w < 3 && ((mask >> w) & 1)) {
            const int ta = upper ? (w == 2 ? 1 : 0) : (w == 0 ? 0 : 1);
            const int tb = upper ? (w == 0 ? 0 : 1) : (w == 2 ? 1 : 0);
            const bool slow = gated && ta == tb && (ta == 0 ? slow0 : slow1);
            f32x16 st;
            zero(st);
            if (!slow) gemm<T, D>(st, A, PD, 32 * ta, B, PD, brow(w));
            const int b = 32 * tb + (l & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int a = 32 * ta + crow(r);
                float x = 0.f;
                if (a < Ct && b < Ct && (upper ? b >= a : b <= a)) x = slow ? exact(a, b) : st[r];
                st[r] = x;
                if (!tr) Sc[a * PS + b] = fromf<T>(x);
            }
            // transposed: the lane's 4 consecutive rows a of each group in one store
            if (tr) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    store4(Sc + b * PS + 32 * ta + crow(4 * q), st[4 * q], st[4 * q + 1], st[4 * q + 2],
                           st[4 * q + 3]);
            }
        } else if (w == 3 && zero_block) {
            const int ta = upper ? 1 : 0, tb = upper ? 0 : 1;
            const int b = 32 * tb + (l & 31);
            if (tr) {
#pragma unroll
                for (int q = 0; q < 4; ++q) store4(Sc + b * PS + 32 * ta + crow(4 * q), 0.f, 0.f, 0.f, 0.f);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) Sc[(32 * ta + crow(r)) * PS + b] = fromf<T>(0.f);
            }
        }
    };
    auto no_exact = [](int, int) { return 0.f; };

    // ---- A: dQ -------------------------------------------------------------
    {
        f32x16 dq[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(dq[k]);
        T *dOr = U, *Pk = U + L::ROWS;   // dO rows; P_t as [dk][dv part]
        float *rpart = (float *)(U + L::ROWS + L::CPART);
        raw_store<T, D, GC, false>(rdo, dOr, PD, Ct, RowId(), NoScale());
        // rho[dk] = sum_dv R_t[dk][dv] P_t[dk][dv]; each thread keeps one group
        // of V consecutive dk (NTHR * V is a multiple of D)
        float racc[V];
#pragma unroll
        for (int j = 0; j < V; ++j) racc[j] = 0.f;
        const float *seg[2] = {Ps, Rs};
        const void *loc[2] = {Lt, Rt};
        const float *g[2] = {gP, gR};
        for (int hh = 0; hh < L::NHALF; ++hh) {
            const int dv0 = hh * DH;
            if (hh) __syncthreads();
            // (bf16: P's rows [dv][dk] in a swizzled tile, read transposed;
            // float32: a transposed copy [dk][dv])
            for_states<T, D, 2, 2, DH>(seg, loc, g, [&](int dv, int dk, const float (*x)[V]) {
                if constexpr (SW) store_vec(Pk + sw_off<D>(dv - dv0, dk), x[0]);
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    if constexpr (!SW) Pk[(dk + j) * PDH + dv - dv0] = fromf<T>(x[0][j]);
                    racc[j] += x[0][j] * x[1][j];
                }
            }, dv0);
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (!TO::get(k, mi, ni)) continue;
                if constexpr (SW)
                    gemm_rc<D, DH>(dq[k], (const bf16 *)dOr + dv0, PD, mi * 32, (const bf16 *)Pk, ni * 32,
                                   frag_offs<D>(l));
                else
                    gemm<T, DH>(dq[k], dOr + dv0, PD, mi * 32, Pk, PDH, ni * 32);
            }
        }
        // the threads sharing a dk group sum in a fixed order (no atomics:
        // the result must not depend on timing)
        constexpr int SLOTS = (NTHR * V < D * D ? NTHR * V : D * D) / D;
        if (threadIdx.x * V < D * D) {
#pragma unroll
            for (int j = 0; j < V; ++j) rpart[threadIdx.x * V + j] = racc[j];
        }
        __syncthreads();
        if (threadIdx.x < D) {
            float r = 0.f;
            for (int q = 0; q < SLOTS; ++q) r += rpart[q * D + threadIdx.x];
            rho[threadIdx.x] = r;
        }
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni)) {
                const float sc = ex2(bS[mi * 32 * D + ni * 32 + (l & 31)]);   // 2^(b_mI) of column c
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[k][r] *= sc;
            }
        }
        // D_ = dO V^T (no gates), then K^T in three versions over the rows
        __syncthreads();   // rho's partial sums are read before V's rows overwrite them
        T *Vr = U + L::ROWS;
        raw_store<T, D, GC, false>(rv, Vr, PD, Ct, RowId(), NoScale());
        tile_spans<D>(bS, slow0, slow1);   // (its barrier also ends the staging)
        scores(dOr, Vr, [](int ww) { return ww == 2 ? 32 : 0; }, false, false, false, no_exact, 7, true);
        __syncthreads();
        // (bf16: the three versions as rows of a swizzled tile, read
        // transposed; float32: transposed copies)
        T *KT3 = U;   // (J=0 | ref row 0), (J=0 | ref 32), (J=1 | ref 32)
        if constexpr (SW)
            raw_store_sw<D, 96>(rk96, (bf16 *)KT3, Ct, krow,
                                gate_scale<T>(bS, D, [](int j) { return j < 32 ? 0 : 32; }));
        else
            raw_store<T, D, 96, true>(rk96, KT3, PK, Ct, krow,
                                      gate_scale<T>(bS, D, [](int j) { return j < 32 ? 0 : 32; }));
        raw_load(rkq, K, Ct, RowId());   // K rows for B, in flight during A
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni)) continue;
            const bool slow = mi == 0 ? slow0 : slow1;
            if constexpr (SW) {
                const FragOffs<D> fo = frag_offs<D>(l);
                if (mi == 1) gemm_rc<D, 32>(dq[k], (const bf16 *)Sc, PS, 32, (const bf16 *)KT3, ni * 32, fo, 32);
                if (!slow)
                    gemm_rc<D, 32>(dq[k], (const bf16 *)Sc + 32 * mi, PS, 32 * mi, (const bf16 *)KT3, ni * 32,
                                   fo, mi ? 64 : 0);
            } else {
                if (mi == 1) gemm<T, 32>(dq[k], Sc, PS, 32, KT3 + 32, PK, ni * 32);
                if (!slow) gemm<T, 32>(dq[k], Sc + 32 * mi, PS, 32 * mi, KT3 + (mi ? 64 : 0), PK, ni * 32);
            }
            const int c = ni * 32 + (l & 31), m = mi * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qs = m + crow(r);
                dq[k][r] *= ex2(bS[qs * D + c] - bS[m * D + c]);
                if (slow && qs < Ct) {
                    float acc = 0.f;
                    for (int i = m; i <= qs; ++i)
                        acc += tof(Sc[qs * PS + i]) * tof(K[(int64_t)i * D + c]) *
                               ex2(bS[qs * D + c] - bS[i * D + c]);
                    dq[k][r] += acc;
                }
            }
            store_rows(dq[k], (T *)p.dQ + rb * D, D, mi * 32, ni * 32, Ct);
            // q . dq goes to the log-gate gradient's rows for now (each element
            // is read back by the lane that wrote it); dq's registers are then free
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qs = m + crow(r);
                if (qs < Ct) p.dLG[(rb + qs) * D + c] = tof(Q[(int64_t)qs * D + c]) * dq[k][r];
            }
        }
        __syncthreads();
    }

    // ---- B: dV -------------------------------------------------------------
    {
        f32x16 dv[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(dv[k]);
        T *Rv = U, *Kl = U + L::RPART;   // R_t rows dv part [dv][dk]; K 2^(b_last - b) rows
        raw_store<T, D, GC, false>(rkq, Kl, PD, Ct, RowId(),
                                   gate_scale<T>(bS, D, [](int) { return GC - 1; }));
        raw_load(rkq, Q, Ct, RowId());   // Q rows for B's scores
        raw_load(rdo, dO, Ct, RowId());  // dO rows for dV, and for C
        {
            const float *seg[1] = {Rs};
            const void *loc[1] = {Rt};
            const float *g[1] = {gR};
            for (int hh = 0; hh < L::NHALF; ++hh) {
                const int dv0 = hh * DH;
                if (hh) __syncthreads();
                for_states<T, D, 1, 2, DH>(seg, loc, g, [&](int dvv, int dk, const float (*x)[V]) {
                    store_vec(Rv + (dvv - dv0) * PD + dk, x[0]);
                }, dv0);
                __syncthreads();
#pragma unroll
                for (int k = 0; k < TO::PER_WAVE; ++k) {
                    int mi, ni;
                    if (TO::get(k, mi, ni) && ni * 32 >= dv0 && ni * 32 < dv0 + DH) {
                        // (bf16: dV accumulated transposed)
                        if constexpr (SW)
                            gemm_t<D>(dv[k], (const bf16 *)Kl, PD, mi * 32, (const bf16 *)Rv, PD, ni * 32 - dv0);
                        else
                            gemm<T, D>(dv[k], Kl, PD, mi * 32, Rv, PD, ni * 32 - dv0);
                    }
                }
            }
        }
        __syncthreads();
        // gated scores A (stored transposed, [key][query]): tiles (1,0), (1,1)
        // from K rows 0..63 with ref 32, then (0,0) from K rows 0..31 with ref 0
        T *Qg = U, *K64 = U + L::ROWS;
        raw_store<T, D, GC, false>(rkq, Qg, PD, Ct, RowId(),
                                   gate_scale<T>(bS, D, [](int j) { return j & ~31; }, true));
        raw_store_map<T, D, 96, false>(rk96, K64, PD, Ct, krow,
                                       gate_scale<T>(bS, D, [](int j) { return j < 32 ? 0 : 32; }),
                                       [](int j) { return j - 32; });
        __syncthreads();
        auto exact = [&](int a, int b) { return exact_score<T, D>(Q, K, bS, a, b); };
        scores(Qg, K64, [](int ww) { return ww == 2 ? 32 : 0; }, false, true, true, exact, 6, true);
        __syncthreads();
        raw_store_map<T, D, 96, false>(rk96, K64, PD, Ct, krow,
                                       gate_scale<T>(bS, D, [](int) { return 0; }),
                                       [](int j) { return j < 32 ? j : -1; });
        __syncthreads();
        scores(Qg, K64, [](int) { return 0; }, false, true, true, exact, 1, false);
        __syncthreads();
        T *OT = U;   // dO^T [dv][query] (bf16: dO rows, swizzled, read transposed)
        if constexpr (SW)
            raw_store_sw<D, GC>(rdo, (bf16 *)OT, Ct, RowId(), NoScale());
        else
            raw_store<T, D, GC, true>(rdo, OT, PS, Ct, RowId(), NoScale());
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni)) continue;
            if constexpr (SW) {
                gemm_rc_t<D, GC>(dv[k], (const bf16 *)Sc, PS, mi * 32, (const bf16 *)OT, ni * 32, frag_offs<D>(l));
                store_tile1_t(dv[k], (bf16 *)p.dV + rb * D, D, mi * 32, ni * 32, Ct);
            } else {
                gemm<T, GC>(dv[k], Sc, PS, mi * 32, OT, PS, ni * 32);
                store_rows(dv[k], (T *)p.dV + rb * D, D, mi * 32, ni * 32, Ct);
            }
        }
        __syncthreads();
    }

    // ---- C: dK -------------------------------------------------------------
    f32x16 dk[TO::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TO::PER_WAVE; ++k) zero(dk[k]);
    raw_load(rv, Vg, Ct, RowId());
    raw_load(rk96, Q, Ct, qrow);   // Q rows of the three versions (the K registers are free)
    raw_load(rkq, K, Ct, RowId());   // K rows for the X term
    {
        T *Vr = U, *RT = U + L::ROWS;   // V rows; R_t as [dk][dv part]
        raw_store<T, D, GC, false>(rv, Vr, PD, Ct, RowId(), NoScale());
        {
            const float *seg[1] = {Rs};
            const void *loc[1] = {Rt};
            const float *g[1] = {gR};
            for (int hh = 0; hh < L::NHALF; ++hh) {
                const int dv0 = hh * DH;
                if (hh) __syncthreads();
                // (stored like P in phase A)
                for_states<T, D, 1, 2, DH>(seg, loc, g, [&](int dvv, int dkk, const float (*x)[V]) {
                    if constexpr (SW) {
                        store_vec(RT + sw_off<D>(dvv - dv0, dkk), x[0]);
                    } else {
#pragma unroll
                        for (int j = 0; j < V; ++j) RT[(dkk + j) * PDH + dvv - dv0] = fromf<T>(x[0][j]);
                    }
                }, dv0);
                __syncthreads();
#pragma unroll
                for (int k = 0; k < TO::PER_WAVE; ++k) {
                    int mi, ni;
                    if (!TO::get(k, mi, ni)) continue;
                    if constexpr (SW)
                        gemm_rc<D, DH>(dk[k], (const bf16 *)Vr + dv0, PD, mi * 32, (const bf16 *)RT, ni * 32,
                                       frag_offs<D>(l));
                    else
                        gemm<T, DH>(dk[k], Vr + dv0, PD, mi * 32, RT, PDH, ni * 32);
                }
            }
        }
        // K rows where R_t was (the products above have read it)
        T *Kx = U + L::ROWS;
        static_assert(2 * L::ROWS <= L::SOFF, "K rows must not reach the scores");
        __syncthreads();
        raw_store<T, D, GC, false>(rkq, Kx, PD, Ct, RowId(), NoScale());
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni)) continue;
            // X = V R^T is in dk; rowsum(R_t . P_{t+1}) gets sum_i k_i 2^(b_last - b_i) X_i
            const int c = ni * 32 + (l & 31), mJ = mi * 32 + 31;
            const float bl = bS[(GC - 1) * D + c];
            float ep = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = mi * 32 + crow(r);
                if (i < Ct) ep += tof(Kx[i * PD + c]) * ex2(bl - bS[i * D + c]) * dk[k][r];
            }
            ep += __shfl_xor(ep, 32);
            if (l < 32) atomicAdd(&Ep[c], ep);
            const float sc = ex2(bl - bS[mJ * D + c]);
#pragma unroll
            for (int r = 0; r < 16; ++r) dk[k][r] *= sc;
        }
        __syncthreads();
        T *dOr = U + L::ROWS;   // D_^T = V dO^T (upper tiles), then Q^T in three versions
        raw_store<T, D, GC, false>(rdo, dOr, PD, Ct, RowId(), NoScale());
        __syncthreads();
        scores(Vr, dOr, [](int ww) { return ww == 0 ? 0 : 32; }, true, false, false, no_exact, 7, true);
        __syncthreads();
        T *QT3 = U;   // (I=0 | ref row 31), (I=1 | ref 31), (I=1 | ref 63), stored as KT3
        if constexpr (SW)
            raw_store_sw<D, 96>(rk96, (bf16 *)QT3, Ct, qrow,
                                gate_scale<T>(bS, D, [](int j) { return j < 64 ? 31 : 63; }, true));
        else
            raw_store<T, D, 96, true>(rk96, QT3, PK, Ct, qrow,
                                      gate_scale<T>(bS, D, [](int j) { return j < 64 ? 31 : 63; }, true));
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni)) continue;
            const bool slow = mi == 0 ? slow0 : slow1;
            if constexpr (SW) {
                const FragOffs<D> fo = frag_offs<D>(l);
                if (mi == 0) gemm_rc<D, 32>(dk[k], (const bf16 *)Sc + 32, PS, 0, (const bf16 *)QT3, ni * 32, fo, 32);
                if (!slow)
                    gemm_rc<D, 32>(dk[k], (const bf16 *)Sc + 32 * mi, PS, 32 * mi, (const bf16 *)QT3, ni * 32,
                                   fo, mi ? 64 : 0);
            } else {
                if (mi == 0) gemm<T, 32>(dk[k], Sc + 32, PS, 0, QT3 + 32, PK, ni * 32);
                if (!slow) gemm<T, 32>(dk[k], Sc + 32 * mi, PS, 32 * mi, QT3 + (mi ? 64 : 0), PK, ni * 32);
            }
            const int c = ni * 32 + (l & 31), mJ = mi * 32 + 31;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = mi * 32 + crow(r);
                dk[k][r] *= ex2(bS[mJ * D + c] - bS[i * D + c]);
                if (slow && i < Ct) {
                    float acc = 0.f;
                    const int se = min(mi * 32 + 32, Ct);
                    for (int sq = i; sq < se; ++sq)
                        acc += tof(Sc[i * PS + sq]) * tof(Q[(int64_t)sq * D + c]) *
                               ex2(bS[sq * D + c] - bS[i * D + c]);
                    dk[k][r] += acc;
                }
            }
            store_rows(dk[k], (T *)p.dK + rb * D, D, mi * 32, ni * 32, Ct);
        }
        __syncthreads();
    }

    // ---- D: log-gate gradient ------------------------------------------------
    float *dBs = (float *)U_raw;   // [GC][D]: q dq - k dk
#pragma unroll
    for (int k = 0; k < TO::PER_WAVE; ++k) {
        int mi, ni;
        if (!TO::get(k, mi, ni)) continue;
        const int c = ni * 32 + (l & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int su = mi * 32 + crow(r);
            float x = 0.f;
            if (su < Ct) x = p.dLG[(rb + su) * D + c] - tof(K[(int64_t)su * D + c]) * dk[k][r];
            dBs[su * D + c] = x;
        }
    }
    __syncthreads();
    {   // suffix sums over the chunk's rows, NTHR / D parts per channel, plus
        // rowsum(R_t . P_{t+1}) = 2^(b_last) rho + Ep
        constexpr int NP = NTHR / D, RPP = GC / NP;
        const int c = threadIdx.x % D, part = threadIdx.x / D, r0 = part * RPP;
        float x[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) x[j] = dBs[(r0 + j) * D + c];
#pragma unroll
        for (int j = RPP - 2; j >= 0; --j) x[j] += x[j + 1];
        __syncthreads();
        dBs[part * D + c] = x[0];
        __syncthreads();
        float off = ex2(bS[(GC - 1) * D + c]) * rho[c] + Ep[c];
        for (int q = part + 1; q < NP; ++q) off += dBs[q * D + c];
        // (the row offsets formed here, opaque to the compiler, rather than
        // computed at the kernel start and kept in registers throughout)
        int o0 = r0 * D + c, nrow = Ct - r0;
        asm volatile("" : "+v"(o0), "+v"(nrow));
        float *out = p.dLG + rb * D + o0;
#pragma unroll
        for (int j = 0; j < RPP; ++j)
            if (j < nrow) out[j * D] = x[j] + off;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline int round8g(int n) { return (n + 7) & ~7; }
static inline void grec(hipEvent_t *ev, int i, hipStream_t st) {
    if (ev) (void)hipEventRecord(ev[i], st);
}

template <typename T, int D>
static hipError_t gfwd(const Params &p, bool with_output, hipStream_t st, hipEvent_t *ev) {
    if (p.varlen) launch_setup(p, st);
    grec(ev, 0, st);
    hipLaunchKernelGGL((k_gfwd_local<T, D>), dim3(p.n_segs_ub * p.H), dim3(NTHR), 0, st, p);
    grec(ev, 1, st);
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    hipLaunchKernelGGL((k_gfwd_segscan<D>), dim3(p.nseq * p.H * NB), dim3(NTHR), 0, st, p);
    grec(ev, 2, st);
    if (with_output)
        hipLaunchKernelGGL((k_gfwd_out<T, D>), dim3(round8g(p.n_chunks_ub * p.H)), dim3(NTHR), 0, st, p);
    grec(ev, 3, st);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t gbwd(const Params &p, hipStream_t st, hipEvent_t *ev) {
    if (p.varlen) launch_setup(p, st);
    grec(ev, 0, st);
    hipLaunchKernelGGL((k_gbwd_local<T, D>), dim3(p.n_segs_ub * p.H), dim3(NTHR), 0, st, p);
    grec(ev, 1, st);
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    hipLaunchKernelGGL((k_gbwd_segscan<D>), dim3(p.nseq * p.H * NB), dim3(NTHR), 0, st, p);
    grec(ev, 2, st);
    hipLaunchKernelGGL((k_gbwd_grads<T, D>), dim3(round8g(p.n_chunks_ub * p.H)), dim3(NTHR), 0, st, p);
    grec(ev, 3, st);
    return hipGetLastError();
}

hipError_t launch_fwd_gated(const Params &p, bool bf, bool with_output, hipStream_t st, hipEvent_t *ev) {
    if (p.C != GC || !p.LG || !p.Gc || !p.Gs) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bf ? gfwd<bf16, 32>(p, with_output, st, ev) : gfwd<float, 32>(p, with_output, st, ev);
    case 64: return bf ? gfwd<bf16, 64>(p, with_output, st, ev) : gfwd<float, 64>(p, with_output, st, ev);
    case 128: return bf ? gfwd<bf16, 128>(p, with_output, st, ev) : gfwd<float, 128>(p, with_output, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_gated(const Params &p, bool bf, hipStream_t st, hipEvent_t *ev) {
    if (p.C != GC || !p.LG || !p.dLG || !p.Gc || !p.Gs || !p.Hc) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bf ? gbwd<bf16, 32>(p, st, ev) : gbwd<float, 32>(p, st, ev);
    case 64: return bf ? gbwd<bf16, 64>(p, st, ev) : gbwd<float, 64>(p, st, ev);
    case 128: return bf ? gbwd<bf16, 128>(p, st, ev) : gbwd<float, 128>(p, st, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace lasp
