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

// The thread's index and lane, opaque to the compiler: the offsets derived
// from them are formed where they are used instead of being hoisted out of the
// chunk loops and kept in registers across them.
__device__ __forceinline__ int otid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
__device__ __forceinline__ int olane() { return otid() & 63; }
__device__ __forceinline__ int owave() { return __builtin_amdgcn_readfirstlane(otid() >> 6); }

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
    const int c = otid() % D, r0 = (otid() / D) * RP;
    // the thread's offset, opaque to the compiler: the loads' addresses are
    // then formed here, not hoisted out of the caller's loop into registers
    // (a buffer over the chunk's Ct valid rows: loads past them return zero,
    // so the loads need no branches; every offset sits in the per-lane operand,
    // which the range check covers)
    int off = (r0 * D + c) * 4;
    asm volatile("" : "+v"(off));
    const __amdgpu_buffer_rsrc_t rs = wave_buffer(lg, Ct > 0 ? Ct * D * 4 : 0);
#pragma unroll
    for (int j = 0; j < RP; ++j)
        lr.x[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + j * D * 4, 0, 0));
}

template <int D>
__device__ __forceinline__ void cumlog_scan(float *bS, const LogRows<D> &lr) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int RP = LogRows<D>::RP;
    const int c = otid() % D, r0 = (otid() / D) * RP;
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

// (src is the chunk's first row, the same on every lane; the loads go through a
// buffer over its Ct valid rows, so rows at or past Ct read as zero without
// branches)
template <typename T, int D, int R, typename RowF>
__device__ __forceinline__ void raw_load(Raw<T, D, R> &raw, const T *src, int Ct, RowF row) {
    using RW = Raw<T, D, R>;
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = wave_buffer(src, Ct > 0 ? Ct * D * (int)sizeof(T) : 0);
#pragma unroll
    for (int u = 0; u < RW::IT; ++u) {
        const int i = u * NTHR + otid();
        const int j = i / RW::PR, c = (i % RW::PR) * RW::V;
        if (i < RW::N) {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, (row(j) * D + c) * (int)sizeof(T), 0, 0);
            raw.v[u] = make_uint4(x[0], x[1], x[2], x[3]);
        } else {
            raw.v[u] = make_uint4(0u, 0u, 0u, 0u);
        }
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
        const int i = u * NTHR + otid();
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
        const int i = u * NTHR + otid();
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

// Transposed accumulation (bf16): acc += A[m0 + i][k] B[n0 + j][k] (gemm_t: A
// and B rows with the contraction index contiguous) or A[m0 + i][k] Y[k][n0 + j]
// (gemm_rc_t: Y a swizzled tile whose rows are the contraction index, read
// transposed) with the MFMA operands swapped, so that acc holds the 32x32 tile
// transposed (lane = output row, its 16 values = columns crow(r));
// store_tile1_t then writes it with 16-byte stores.
template <int K>
__device__ __forceinline__ void gemm_t(f32x16 &acc, const bf16 *As, int pa, int m0, const bf16 *Bs,
                                       int pb, int n0) {
    const int l = olane();
    const bf16 *ap = As + (m0 + (l & 31)) * pa + (l >> 5) * 8;
    const bf16 *bp = Bs + (n0 + (l & 31)) * pb + (l >> 5) * 8;
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, *(const bf16x8_t *)(bp + k), *(const bf16x8_t *)(ap + k));
}
template <int D, int K>
__device__ __forceinline__ void gemm_rc_t(f32x16 &acc, const bf16 *A, int pa, int m0, const bf16 *Y,
                                          int n0, const FragOffs<D> &fo, int y0 = 0) {
    // (Y's rows y0 .. y0 + K - 1; y0 a multiple of 16)
    const int l = olane();
    const bf16 *ap = A + (m0 + (l & 31)) * pa + (l >> 5) * 8;
#pragma unroll
    for (int k = 0; k < K; k += 16)
        mma(acc, frag_cols_sw<D, false>(Y, fo, y0 + k, n0), *(const bf16x8_t *)(ap + k));
}

// Rows m0 + lane%32 (those below nrow), columns n0 .. n0+31 of G (row pitch
// ld, float32 or bf16) from a transposed accumulator: the lane's 4 groups of
// 4 consecutive columns, one store each.
template <typename T>
__device__ __forceinline__ void store_rows_t(const f32x16 &acc, T *G, int ld, int m0, int n0, int nrow,
                                             int l) {
    const int row = m0 + (l & 31);
    if (row >= nrow) return;
    T *g = G + (int64_t)row * ld + n0 + (l >> 5) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) store4(g + q * 8, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// The sum over the 32 lanes of x's half of the wave (lanes 0-31 or 32-63),
// in every lane of that half.
__device__ __forceinline__ float half_sum(float x) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// x[0..15] summed over the 32 lanes of each half of the wave, 16 exchanges in
// all: at each step a lane keeps half of its values and adds its partner's
// copy of them (partner lane ^ 16, 8, 4, 2), then the pair (lane ^ 1) adds.
// Returns, in lanes 2r and 2r + 1 of each half, the sum of x[r].
__device__ __forceinline__ float half_colsum16(float *x, int l) {
#pragma unroll
    for (int m = 16, n = 8; m >= 2; m >>= 1, n >>= 1) {
        const bool hi = (l & m) != 0;
#pragma unroll
        for (int j = 0; j < n; ++j) {
            const float send = hi ? x[j] : x[j + n];
            const float keep = hi ? x[j + n] : x[j];
            x[j] = keep + __shfl_xor(send, m);
        }
    }
    return x[0] + __shfl_xor(x[0], 1);
}

// 4 consecutive elements of a bf16 or float32 row as floats.
__device__ __forceinline__ void load4f(const bf16 *p, float *f) {
    const uint2 v = *(const uint2 *)p;
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void load4f(const float *p, float *f) {
    const float4 v = *(const float4 *)p;
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
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
    const __amdgpu_buffer_rsrc_t rs = wave_buffer(G + (int64_t)m0 * ld + n0, rows > 0 ? rows * ld * 2 : 0);
    const int l = olane();
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
        const int c = (otid() % (D / V)) * V;
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

// Span test of the two 32-row tiles of a chunk (uniform over the workgroup).
template <int D>
__device__ __forceinline__ void tile_spans(const float *bS, bool &slow0, bool &slow1) {
    bool s0 = false, s1 = false;
    for (int c = otid(); c < D; c += NTHR) {
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
// Forward 1: segment totals, one workgroup per (segment, head), chunks in
// order from a zero state at the segment start:
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
            if (TL::get(k, mi, ni, owave())) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[k][r] *= ex2(bS[(GC - 1) * D + mi * 32 + crow(r, olane())]);
                if constexpr (SW)
                    gemm_cc<D, GC>(acc[k], (const bf16 *)KT_s, mi * 32, (const bf16 *)VT_s, ni * 32,
                                   opaque(frag_offs<D>(olane())));
                else
                    gemm<T, GC>(acc[k], KT_s, PT, mi * 32, VT_s, PT, ni * 32, olane());
            }
        }
        if (otid() < D) gcum *= ex2(bS[(GC - 1) * D + otid()]);
    }
    const int64_t sh = (int64_t)gs * p.H + h;
    float *Zs = p.Z + sh * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni, owave())) store_T(acc[k], Zs, D, mi * 32, ni * 32, Ident());
    }
    if (otid() < D) p.Gs[sh * D + otid()] = gcum;
}

// ---------------------------------------------------------------------------
// Forward 2: scan over segments, one thread per state element:
//   Pseg[0] = M_in;  Pseg[s+1] = Diag(Gs[s]) Pseg[s] + Z[s];  M_out = last.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NTHR) void k_gfwd_segscan(Params p) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    const int ih = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * NTHR + otid();
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;   // [dk][dv] of the API states
    float P = p.M_in ? p.M_in[mo] : 0.f;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    // totals and gates loaded SCAN_BATCH segments at a time, ahead of the stores
    for (int b0 = 0; b0 < nS; b0 += SCAN_BATCH) {
        float z[SCAN_BATCH], g[SCAN_BATCH];
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            const int64_t sh = (int64_t)(s.s0 + b0 + j) * p.H + h;
            const bool in = b0 + j < nS;
            z[j] = in ? p.Z[sh * D * D + e] : 0.f;
            g[j] = in ? p.Gs[sh * D + dk] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            if (b0 + j < nS) {
                p.Pseg[((int64_t)(s.s0 + b0 + j) * p.H + h) * D * D + e] = P;
                P = g[j] * P + z[j];
            }
        }
    }
    if (p.M_out) p.M_out[mo] = P;
    if (p.Pfin) p.Pfin[(int64_t)ih * D * D + e] = P;   // [dv][dk], as Pseg
}

// LDS plan of the output walk: the running log-gates (float32) and one
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

// LDS plan of the gradient walks: the running log-gates (float32), a small
// per-channel sum and one scratch area reused by every phase, small enough
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
    static constexpr int A1 = ROWS + CPART;               // dO rows, P part
    static constexpr int B1 = RPART + ROWS;               // R part, K rows
    static constexpr int C1 = ROWS + CPART;               // V rows, R^T part
    static constexpr int S2 = SOFF + SC;                  // two row arrays + scores
    static constexpr int M1 = A1 > B1 ? A1 : B1, M2 = C1 > S2 ? C1 : S2;
    static constexpr int ELEMS = M1 > M2 ? M1 : M2;
    static constexpr int BYTES = ELEMS * (int)sizeof(T) > GC * D * 4 ? ELEMS * (int)sizeof(T) : GC * D * 4;
    static_assert(D * PK <= SOFF && D * PS <= SOFF, "K^T / Q^T / dO^T must not reach the scores");
};

// ---------------------------------------------------------------------------
// A D x D state carried in registers by the walks below: tile k of the wave
// (Tiles<D/32, D/32>) holds S[dk block mi][dv block ni] as a float32 MFMA
// accumulator (element r: dk = 32 mi + crow(r), dv = 32 ni + lane % 32).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void state_load(f32x16 *S, const float *src) {   // src [dv][dk]
    using TL = Tiles<D / 32, D / 32>;
    const int l = olane();
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (!TL::get(k, mi, ni, owave())) continue;
        // (the lane's dk are 4 runs of 4 consecutive channels: 16-byte loads)
        const float *row = src + (ni * 32 + (l & 31)) * D + mi * 32 + (l >> 5) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *(const float4 *)(row + 8 * q);
            S[k][4 * q] = v.x;
            S[k][4 * q + 1] = v.y;
            S[k][4 * q + 2] = v.z;
            S[k][4 * q + 3] = v.w;
        }
    }
}

// The state into dst [dv][dk] (float32), 16-byte stores.
template <int D>
__device__ __forceinline__ void state_store(const f32x16 *S, float *dst) {
    using TL = Tiles<D / 32, D / 32>;
    const int l = olane();
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (!TL::get(k, mi, ni, owave())) continue;
        float *row = dst + (ni * 32 + (l & 31)) * D + mi * 32 + (l >> 5) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) store4(row + 8 * q, S[k][4 * q], S[k][4 * q + 1], S[k][4 * q + 2], S[k][4 * q + 3]);
    }
}

// part[ni][dk] = sum over the dv of block ni of S[dk][dv] X[dk][dv], X given
// as src [dv][dk] (float32): the row sums of S . X once the D/32 parts of each
// dk are added (by the caller, after a barrier).
template <int D>
__device__ __forceinline__ void state_rowdot(const f32x16 *S, const float *src, float (*part)[D]) {
    using TL = Tiles<D / 32, D / 32>;
    const int l = olane();
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (!TL::get(k, mi, ni, owave())) continue;
        const float *row = src + (ni * 32 + (l & 31)) * D + mi * 32 + (l >> 5) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *(const float4 *)(row + 8 * q);
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float y = half_sum(S[k][4 * q + e] * x[e]);
                if ((l & 31) == 0) part[ni][mi * 32 + 8 * q + (l >> 5) * 4 + e] = y;
            }
        }
    }
}

// Rows dv0 .. dv0 + DH - 1 of the state's [dv][dk] form: f(dv - dv0, dk, x)
// receives 4 consecutive dk of one row.
template <int D, int DH, typename F>
__device__ __forceinline__ void state_rows(const f32x16 *S, int dv0, F f) {
    using TL = Tiles<D / 32, D / 32>;
    const int l = olane();
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (!TL::get(k, mi, ni, owave()) || ni * 32 < dv0 || ni * 32 >= dv0 + DH) continue;
        const int dv = ni * 32 + (l & 31) - dv0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float x[4] = {S[k][4 * q], S[k][4 * q + 1], S[k][4 * q + 2], S[k][4 * q + 3]};
            f(dv, mi * 32 + q * 8 + (l >> 5) * 4, x);
        }
    }
}

// S <- Diag(2^(b_last)) S: row dk scaled by the chunk's gate product.
template <int D>
__device__ __forceinline__ void state_decay(f32x16 *S, const float *bS) {
    using TL = Tiles<D / 32, D / 32>;
    const int l = olane();
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (!TL::get(k, mi, ni, owave())) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[k][r] *= ex2(bS[(GC - 1) * D + mi * 32 + crow(r, l)]);
    }
}

// The running sums of the chunk's log-gates into bS (the caller synchronizes
// before anyone reads them): loaded here, at the chunk's start (a prefetch
// held in registers across the chunk would not fit beside the state).
template <int D>
__device__ __forceinline__ void chunk_gates(float *bS, const float *lg, int Ct) {
    LogRows<D> rl;
    cumlog_load<D>(rl, lg, Ct);
    __syncthreads();   // the previous chunk's readers of bS are done
    cumlog_scan<D>(bS, rl);
}

// ---------------------------------------------------------------------------
// Forward 3: output, one workgroup per (segment, head), walking the segment's
// chunks in order with the state P in registers (float32 MFMA accumulators,
// tile (mi, ni) = P[dk block mi][dv block ni]), from the segment's entering
// state Pseg:
//   O_t = (Q 2^b) P + sum over tile pairs J <= I of
//         [(Q_I 2^(b - b_mI)) (K_J 2^(b_mI - b))^T masked] V_J
//   P  <- Diag(2^(b_last)) P + (K 2^(b_last - b))^T V
// The next chunk's rows are loaded while the current one is worked on, each
// set once its registers have been staged for the last time.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gfwd_walk(Params p) {
    using L = OutLds<T, D>;
    constexpr int PD = L::PD, PS = L::PS, DH = L::DH;
    constexpr bool SW = sizeof(T) == 2;
    constexpr int KOFF = SW ? GC * D : D * PS;   // K 2^(b_last - b) for the update, past V
    static_assert(KOFF + (SW ? GC * D : D * PS) <= L::ELEMS, "update operands fit");
    __shared__ float bS[GC * D];
    __shared__ __attribute__((aligned(16))) T U[L::ELEMS];
    using TO = Tiles<GC / 32, D / 32>;
    using TL = Tiles<D / 32, D / 32>;

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb0 = row_base(p, s, h);
    const int64_t sh = (int64_t)gs * p.H + h;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    const int w = owave();

    f32x16 P[TL::PER_WAVE];
    state_load<D>(P, p.Pseg + sh * D * D);

    Raw<T, D, GC> rq, rk, rv;
    if (t0 < t1) {
        const int64_t rb = rb0 + (int64_t)t0 * GC;
        const int Ct0 = min(GC, s.len - t0 * GC);
        raw_load(rq, (const T *)p.Q + rb * D, Ct0, RowId());
        raw_load(rk, (const T *)p.K + rb * D, Ct0, RowId());
        raw_load(rv, (const T *)p.V + rb * D, Ct0, RowId());
    }
    for (int t = t0; t < t1; ++t) {
        const int tok = t * GC;
        const int Ct = min(GC, s.len - tok);
        const bool more = t + 1 < t1;
        const int Cn = more ? min(GC, s.len - tok - GC) : 0;
        const int64_t rb = rb0 + tok;
        const T *Q = (const T *)p.Q + rb * D;
        const T *K = (const T *)p.K + rb * D;
        T *O = (T *)p.O + rb * D;
        const int l = olane();   // (once per chunk: see otid)
        chunk_gates<D>(bS, p.LG + rb * D, Ct);   // (its first barrier also frees U)
        __syncthreads();

        // 1: o = (Q 2^b) P, P^T rows [dv][dk] written from the registers
        T *Qh = U, *Ph = U + L::ROWS;
        f32x16 o[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(o[k]);
        for (int hh = 0; hh < L::NHALF; ++hh) {
            const int dv0 = hh * DH;
            if (hh) __syncthreads();
            state_rows<D, DH>(P, dv0, [&](int dv, int dk, const float *x) {
                store4(Ph + dv * PD + dk, x[0], x[1], x[2], x[3]);
            });
            if (!hh)
                raw_store<T, D, GC, false>(rq, Qh, PD, Ct, RowId(),
                                           gate_scale<T>(bS, D, [](int) { return -1; }));
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni, owave()) && ni * 32 >= dv0 && ni * 32 < dv0 + DH) {
                    // (bf16: O accumulated transposed)
                    if constexpr (SW)
                        gemm_t<D>(o[k], (const bf16 *)Qh, PD, mi * 32, (const bf16 *)Ph, PD, ni * 32 - dv0);
                    else
                        gemm<T, D>(o[k], Qh, PD, mi * 32, Ph, PD, ni * 32 - dv0, olane());
                }
            }
        }
        __syncthreads();

        // 2: masked gated scores into Sc
        T *Qt = U, *K64 = U + L::ROWS, *Sc = U + L::SOFF;
        raw_store<T, D, GC, false>(rq, Qt, PD, Ct, RowId(),
                                   gate_scale<T>(bS, D, [](int j) { return j & ~31; }, true));
        raw_store<T, D, GC, false>(rk, K64, PD, Ct, RowId(),
                                   gate_scale<T>(bS, D, [](int) { return 32; }));   // rows 0..63 with ref 32
        bool slow0, slow1;
        tile_spans<D>(bS, slow0, slow1);   // (its barrier also ends the staging)
        auto score_tile = [&](int I, int J, int krow0, bool slow) __attribute__((always_inline)) {
            f32x16 st;
            zero(st);
            if (!slow) gemm<T, D>(st, Qt, PD, 32 * I, K64, PD, krow0, olane());
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qs = 32 * I + crow(r, olane()), ki = 32 * J + (l & 31);
                float x = 0.f;
                if (qs < Ct && ki < Ct && ki <= qs) x = slow ? exact_score<T, D>(Q, K, bS, qs, ki) : st[r];
                Sc[qs * PS + ki] = fromf<T>(x);
            }
        };
        if (w == 1) score_tile(1, 0, 0, false);
        if (w == 2) score_tile(1, 1, 32, slow1);
        if (w == 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Sc[crow(r, olane()) * PS + 32 + (l & 31)] = fromf<T>(0.f);
        }
        __syncthreads();
        raw_store_map<T, D, GC, false>(rk, K64, PD, Ct, RowId(),
                                       gate_scale<T>(bS, D, [](int) { return 0; }),
                                       [](int j) { return j < 32 ? j : -1; });   // rows 0..31 with ref 0
        __syncthreads();
        if (w == 0) score_tile(0, 0, 0, slow0);
        __syncthreads();

        // 3: o += Sc V (bf16: V rows in a swizzled tile, read transposed;
        // float32: a transposed copy); V stays for the state update
        static_assert(GC * D <= L::SOFF && D * PS <= L::SOFF, "V must not reach the scores");
        T *VT = U;
        if constexpr (SW)
            raw_store_sw<D, GC>(rv, (bf16 *)VT, Ct, RowId(), NoScale());
        else
            raw_store<T, D, GC, true>(rv, VT, PS, Ct, RowId(), NoScale());
        if (more) {
            raw_load(rq, Q + GC * D, Cn, RowId());
            raw_load(rv, (const T *)p.V + (rb + GC) * D, Cn, RowId());
        }
        __syncthreads();
        const FragOffs<D> fo = frag_offs<D>(l);
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni, owave())) {
                if constexpr (SW) {
                    gemm_rc_t<D, GC>(o[k], (const bf16 *)Sc, PS, mi * 32, (const bf16 *)VT, ni * 32, fo);
                    store_tile1_t(o[k], (bf16 *)O, D, mi * 32, ni * 32, Ct);
                } else {
                    gemm<T, GC>(o[k], Sc, PS, mi * 32, VT, PS, ni * 32, olane());
                    store_rows(o[k], O, D, mi * 32, ni * 32, Ct, olane());
                }
            }
        }
        if (!more) break;   // (the state after the segment comes from the scan)

        // 4: P <- Diag(2^(b_last)) P + (K 2^(b_last - b))^T V
        __syncthreads();   // the products above have read Sc
        T *KT = U + KOFF;
        if constexpr (SW)
            raw_store_sw<D, GC>(rk, (bf16 *)KT, Ct, RowId(), LastRowScale<D, 8>(bS));
        else
            raw_store<T, D, GC, true>(rk, KT, PS, Ct, RowId(),
                                      gate_scale<T>(bS, D, [](int) { return GC - 1; }));
        __syncthreads();
        state_decay<D>(P, bS);
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) {
            int mi, ni;
            if (!TL::get(k, mi, ni, owave())) continue;
            if constexpr (SW)
                gemm_cc<D, GC>(P[k], (const bf16 *)KT, mi * 32, (const bf16 *)VT, ni * 32, opaque(fo));
            else
                gemm<T, GC>(P[k], KT, PS, mi * 32, VT, PS, ni * 32, olane());
        }
        raw_load(rk, K + GC * D, Cn, RowId());
    }
}

// ---------------------------------------------------------------------------
// Backward 1: reverse segment totals, one workgroup per (segment, head),
// chunks last to first from a zero state at the segment end:
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
    const FragOffs<D> fo = frag_offs<D>(olane());

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb = row_base(p, s, h);
    const T *Q = (const T *)p.Q + rb * D;
    const T *dO = (const T *)p.dO + rb * D;
    const float *LG = p.LG + rb * D;

    f32x16 acc[TL::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) zero(acc[k]);

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
            if (TL::get(k, mi, ni, owave())) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[k][r] *= ex2(bS[(GC - 1) * D + mi * 32 + crow(r, olane())]);
                if constexpr (SW)
                    gemm_cc<D, GC>(acc[k], (const bf16 *)QT_s, mi * 32, (const bf16 *)OT_s, ni * 32, fo);
                else
                    gemm<T, GC>(acc[k], QT_s, PT, mi * 32, OT_s, PT, ni * 32, olane());
            }
        }
    }
    float *Ws = p.W + ((int64_t)gs * p.H + h) * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni, owave())) store_T(acc[k], Ws, D, mi * 32, ni * 32, Ident());
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
    const int e = (blockIdx.x % NB) * NTHR + otid();
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;
    float R = p.dM_out ? p.dM_out[mo] : 0.f;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    // (last segment first; loads batched as in the forward scan)
    for (int b0 = nS - 1; b0 >= 0; b0 -= SCAN_BATCH) {
        float wv[SCAN_BATCH], g[SCAN_BATCH];
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            const int64_t sh = (int64_t)(s.s0 + b0 - j) * p.H + h;
            const bool in = b0 - j >= 0;
            wv[j] = in ? p.W[sh * D * D + e] : 0.f;
            g[j] = in ? p.Gs[sh * D + dk] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            if (b0 - j >= 0) {
                p.Rseg[((int64_t)(s.s0 + b0 - j) * p.H + h) * D * D + e] = R;
                R = g[j] * R + wv[j];
            }
        }
    }
    if (p.dM_in) p.dM_in[mo] = R;
}

// ---------------------------------------------------------------------------
// Masked 32x32 score tiles A_a . B_b^T into Sc (pitch PS; A and B rows of
// pitch PD): tiles (a, b) = (0,0), (1,0), (1,1) (lower: b <= a kept) or
// (0,0), (0,1), (1,1) (upper: b >= a kept), the tiles of mask bit w (bit i:
// tile i) on waves 0..2; wave 3 zeroes the remaining block when zero_block.
// B's rows for tile i start at brow(i).  Gated diagonal tiles over the span
// limit (slow0 / slow1) take exact(a, b) instead of the product.  tr stores
// Sc[b][a].
// ---------------------------------------------------------------------------
template <typename T, int D, int PD, int PS, typename BRow, typename Exact>
__device__ __forceinline__ void score_tiles(T *Sc, const T *A, const T *B, BRow brow, bool upper, bool tr,
                                            bool gated, Exact exact, int mask, bool zero_block, int Ct,
                                            bool slow0, bool slow1) {
    const int w = owave(), l = olane();
    if (w < 3 && ((mask >> w) & 1)) {
        const int ta = upper ? (w == 2 ? 1 : 0) : (w == 0 ? 0 : 1);
        const int tb = upper ? (w == 0 ? 0 : 1) : (w == 2 ? 1 : 0);
        const bool slow = gated && ta == tb && (ta == 0 ? slow0 : slow1);
        f32x16 st;
        zero(st);
        if (!slow) gemm<T, D>(st, A, PD, 32 * ta, B, PD, brow(w), l);
        const int b = 32 * tb + (l & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int a = 32 * ta + crow(r, l);
            float x = 0.f;
            if (a < Ct && b < Ct && (upper ? b >= a : b <= a)) x = slow ? exact(a, b) : st[r];
            st[r] = x;
            if (!tr) Sc[a * PS + b] = fromf<T>(x);
        }
        // transposed: the lane's 4 consecutive rows a of each group in one store
        if (tr) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                store4(Sc + b * PS + 32 * ta + crow(4 * q, l), st[4 * q], st[4 * q + 1], st[4 * q + 2],
                       st[4 * q + 3]);
        }
    } else if (w == 3 && zero_block) {
        const int ta = upper ? 1 : 0, tb = upper ? 0 : 1;
        const int b = 32 * tb + (l & 31);
        if (tr) {
#pragma unroll
            for (int q = 0; q < 4; ++q) store4(Sc + b * PS + 32 * ta + crow(4 * q, l), 0.f, 0.f, 0.f, 0.f);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) Sc[(32 * ta + crow(r, l)) * PS + b] = fromf<T>(0.f);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward 3: dQ, one workgroup per (segment, head), walking the segment's
// chunks in order with the forward state P in registers (as the output walk),
// from Pseg; with D_ = dO V^T and m_I the first row of query tile I:
//   dQ = 2^b . (dO P^T) + sum_{J<=I} 2^(b - b_mI) . ([D_ masked]_IJ (K_J 2^(b_mI - b)))
//   P <- Diag(2^(b_last)) P + (K 2^(b_last - b))^T V
// q . dq goes to the log-gate gradient's rows, where the reverse walk reads it.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gbwd_walk_q(Params p) {
    using L = GradLds<T, D>;
    constexpr int PD = L::PD, PS = L::PS, PK = L::PK, DH = L::DH, PDH = L::PDH;
    constexpr bool SW = sizeof(T) == 2;   // bf16: transpose reads of row tiles
    constexpr int UPD = SW ? GC * D : D * PS;   // one operand of the state update
    static_assert(96 * D <= L::SOFF && D * PK <= L::SOFF, "K versions must not reach the scores");
    static_assert(2 * UPD * (int)sizeof(T) <= L::BYTES, "update operands fit");
    __shared__ float bS[GC * D];
    __shared__ float Ap[GC / 32][D];   // row block mi's part of the chunk's q . dq-inter sums
    __shared__ __attribute__((aligned(16))) char U_raw[L::BYTES];
    T *U = (T *)U_raw;
    T *Sc = U + L::SOFF;
    using TO = Tiles<GC / 32, D / 32>;
    using TL = Tiles<D / 32, D / 32>;

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb0 = row_base(p, s, h);
    const int64_t sh = (int64_t)gs * p.H + h;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);

    f32x16 P[TL::PER_WAVE];
    state_load<D>(P, p.Pseg + sh * D * D);

    Raw<T, D, GC> rdo, rv, rk;   // the chunk's dO, V, K rows (the next chunk's, loaded ahead)
    if (t0 < t1) {
        const int64_t rb = rb0 + (int64_t)t0 * GC;
        const int Ct0 = min(GC, s.len - t0 * GC);
        raw_load(rdo, (const T *)p.dO + rb * D, Ct0, RowId());
        raw_load(rv, (const T *)p.V + rb * D, Ct0, RowId());
        raw_load(rk, (const T *)p.K + rb * D, Ct0, RowId());
    }
    for (int t = t0; t < t1; ++t) {
        const int tok = t * GC;
        const int Ct = min(GC, s.len - tok);
        const bool more = t + 1 < t1;
        const int Cn = more ? min(GC, s.len - tok - GC) : 0;
        const int64_t rb = rb0 + tok;
        const T *Q = (const T *)p.Q + rb * D;
        const T *K = (const T *)p.K + rb * D;
        const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
        const int l = olane();   // (once per chunk: see otid)
        chunk_gates<D>(bS, p.LG + rb * D, Ct);
        auto no_exact = [](int, int) { return 0.f; };

        // dO P^T over the state's dv halves
        f32x16 dq[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(dq[k]);
        T *dOr = U, *Pk = U + L::ROWS;   // dO rows; P as [dk][dv part]
        raw_store<T, D, GC, false>(rdo, dOr, PD, Ct, RowId(), NoScale());
        for (int hh = 0; hh < L::NHALF; ++hh) {
            const int dv0 = hh * DH;
            __syncthreads();   // (first half: bS is written; later: the last products are done)
            // (bf16: P's rows [dv][dk] in a swizzled tile, read transposed;
            // float32: a transposed copy [dk][dv])
            state_rows<D, DH>(P, dv0, [&](int dv, int dk, const float *x) {
                if constexpr (SW) {
                    store4(Pk + sw_off<D>(dv, dk), x[0], x[1], x[2], x[3]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) Pk[(dk + j) * PDH + dv] = x[j];
                }
            });
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (!TO::get(k, mi, ni, owave())) continue;
                // (dQ accumulated transposed: lane = token row, 4 groups of 4
                // consecutive channels)
                if constexpr (SW)
                    gemm_rc_t<D, DH>(dq[k], (const bf16 *)dOr + dv0, PD, mi * 32, (const bf16 *)Pk, ni * 32,
                                     frag_offs<D>(l));
                else
                    gemm<T, DH>(dq[k], Pk, PDH, ni * 32, dOr + dv0, PD, mi * 32, l);
            }
        }
        // the chunk's sum over its tokens of q . 2^b (dO P^T), per channel: with
        // the reverse walk's sum of k . 2^(b_last - b) (V R^T) it is the chunk's
        // total of q dq - k dk exactly (the terms between the chunk's own tokens
        // cancel over the whole chunk, a shift of all its running log-gates
        // leaving them unchanged), free of those terms' rounding
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni, owave())) continue;
            const int qs = mi * 32 + (l & 31), c0 = ni * 32 + (l >> 5) * 4;
            float x[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float qv[4] = {0.f, 0.f, 0.f, 0.f};
                if (qs < Ct) load4f(Q + (int64_t)qs * D + c0 + 8 * q, qv);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * q + e] = qv[e] * ex2(bS[qs * D + c0 + 8 * q + e]) * dq[k][4 * q + e];
            }
            const float a = half_colsum16(x, l);
            if (!(l & 1)) Ap[mi][ni * 32 + crow((l >> 1) & 15, l)] = a;
            // 2^(b_mI) of each column
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[k][r] *= ex2(bS[mi * 32 * D + ni * 32 + crow(r, l)]);
        }
        // D_ = dO V^T (no gates), then K^T in three versions
        __syncthreads();
        T *Vr = U + L::ROWS;
        raw_store<T, D, GC, false>(rv, Vr, PD, Ct, RowId(), NoScale());
        bool slow0, slow1;
        tile_spans<D>(bS, slow0, slow1);   // (its barrier also ends the staging)
        if (otid() < D) p.Tq[ch * D + otid()] = Ap[0][otid()] + Ap[1][otid()];
        score_tiles<T, D, PD, PS>(Sc, dOr, Vr, [](int ww) { return ww == 2 ? 32 : 0; }, false, false, false,
                                  no_exact, 7, true, Ct, slow0, slow1);
        __syncthreads();
        // (bf16: the versions as rows of a swizzled tile, read transposed;
        // float32: transposed copies) rows 0..31 with ref row 0 as tile rows
        // 0..31, rows 0..63 with ref 32 as tile rows 32..95
        T *KT3 = U;
        if constexpr (SW) {
            raw_store_sw<D, GC>(rk, (bf16 *)KT3, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 0; }),
                                [](int j) { return j < 32 ? j : -1; });
            raw_store_sw<D, GC>(rk, (bf16 *)KT3, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 32; }),
                                [](int j) { return j + 32; });
        } else {
            raw_store_map<T, D, GC, true>(rk, KT3, PK, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 0; }),
                                          [](int j) { return j < 32 ? j : -1; });
            raw_store_map<T, D, GC, true>(rk, KT3, PK, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 32; }),
                                          [](int j) { return j + 32; });
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni, owave())) continue;
            const bool slow = mi == 0 ? slow0 : slow1;
            if constexpr (SW) {
                const FragOffs<D> fo = frag_offs<D>(l);
                if (mi == 1) gemm_rc_t<D, 32>(dq[k], (const bf16 *)Sc, PS, 32, (const bf16 *)KT3, ni * 32, fo, 32);
                if (!slow)
                    gemm_rc_t<D, 32>(dq[k], (const bf16 *)Sc + 32 * mi, PS, 32 * mi, (const bf16 *)KT3, ni * 32,
                                     fo, mi ? 64 : 0);
            } else {
                if (mi == 1) gemm<T, 32>(dq[k], KT3 + 32, PK, ni * 32, Sc, PS, 32, l);
                if (!slow) gemm<T, 32>(dq[k], KT3 + (mi ? 64 : 0), PK, ni * 32, Sc + 32 * mi, PS, 32 * mi, l);
            }
            const int qs = mi * 32 + (l & 31), m = mi * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = ni * 32 + crow(r, l);
                dq[k][r] *= ex2(bS[qs * D + c] - bS[m * D + c]);
                if (slow && qs < Ct) {
                    float acc = 0.f;
                    for (int i = m; i <= qs; ++i)
                        acc += tof(Sc[qs * PS + i]) * tof(K[(int64_t)i * D + c]) *
                               ex2(bS[qs * D + c] - bS[i * D + c]);
                    dq[k][r] += acc;
                }
            }
            if constexpr (SW)
                store_tile1_t(dq[k], (bf16 *)p.dQ + rb * D, D, mi * 32, ni * 32, Ct);
            else
                store_rows_t(dq[k], (T *)p.dQ + rb * D, D, mi * 32, ni * 32, Ct, l);
            if (qs < Ct) {
                const int c0 = ni * 32 + (l >> 5) * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float qv[4];
                    load4f(Q + (int64_t)qs * D + c0 + 8 * q, qv);
                    store4(p.dLG + (rb + qs) * D + c0 + 8 * q, qv[0] * dq[k][4 * q], qv[1] * dq[k][4 * q + 1],
                           qv[2] * dq[k][4 * q + 2], qv[3] * dq[k][4 * q + 3]);
                }
            }
        }
        if (!more) break;   // (the state after the segment is not needed)

        // P <- Diag(2^(b_last)) P + (K 2^(b_last - b))^T V
        __syncthreads();   // the products above have read KT3 and Sc
        T *KU = U, *VU = U + UPD;
        if constexpr (SW) {
            raw_store_sw<D, GC>(rk, (bf16 *)KU, Ct, RowId(), LastRowScale<D, 8>(bS));
            raw_store_sw<D, GC>(rv, (bf16 *)VU, Ct, RowId(), NoScale());
        } else {
            raw_store<T, D, GC, true>(rk, KU, PS, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return GC - 1; }));
            raw_store<T, D, GC, true>(rv, VU, PS, Ct, RowId(), NoScale());
        }
        raw_load(rdo, (const T *)p.dO + (rb + GC) * D, Cn, RowId());
        raw_load(rv, (const T *)p.V + (rb + GC) * D, Cn, RowId());
        raw_load(rk, K + GC * D, Cn, RowId());
        __syncthreads();
        state_decay<D>(P, bS);
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) {
            int mi, ni;
            if (!TL::get(k, mi, ni, owave())) continue;
            if constexpr (SW)
                gemm_cc<D, GC>(P[k], (const bf16 *)KU, mi * 32, (const bf16 *)VU, ni * 32, opaque(frag_offs<D>(l)));
            else
                gemm<T, GC>(P[k], KU, PS, mi * 32, VU, PS, ni * 32, l);
        }
        // every GATED_CK chunks inside the segment: P for the reverse walk's
        // exact reset of its log-gate gradient sum
        const int done = t - t0 + 1;
        if (p.Pck && done % GATED_CK == 0)
            state_store<D>(P, p.Pck + (sh * ((p.G - 1) / GATED_CK) + done / GATED_CK - 1) * D * D);
    }
}

// ---------------------------------------------------------------------------
// Backward 4: dV, dK and dlog_g, one workgroup per (segment, head), walking
// the segment's chunks last to first with the reverse state R in registers,
// from the segment's state Rseg; m'_J the last row of key tile J:
//   dV = (K 2^(b_last - b)) R + sum_{I>=J} [A masked]_IJ^T dO_I   (A: the gated scores)
//   dK = 2^(b_last - b) . (V R^T)
//        + sum_{I>=J} 2^(b_mJ' - b) . ([D_ masked]_IJ^T (Q_I 2^(b - b_mJ')))
//   dlog_g[s] = sum over the sequence's u >= s of (q_u dq_u - k_u dk_u)
//   R <- Diag(2^(b_last)) R + (Q 2^b)^T dO
// The suffix sum of dlog_g runs inside the chunk over the tokens' q dq - k dk
// and is carried from chunk to chunk in registers as the chunks' totals,
// formed from the inter-chunk terms only.  Its part beyond the segment is the
// log-gate gradient of everything after it, rowsum(R . P) over the states at
// the segment's end (the reverse state entering it from the right and the
// forward state leaving it: the next segment's Pseg, or the sequence's final
// state).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NTHR, (WgPerCu<T, D>::N)) void k_gbwd_walk_kv(Params p) {
    using L = GradLds<T, D>;
    constexpr int PD = L::PD, PS = L::PS, PK = L::PK, DH = L::DH, PDH = L::PDH;
    constexpr bool SW = sizeof(T) == 2;
    constexpr int UPD = SW ? GC * D : D * PS;
    static_assert(96 * D <= L::SOFF && D * PK <= L::SOFF, "Q versions must not reach the scores");
    static_assert(GC * D * 4 <= L::BYTES, "the log-gate rows fit");
    static_assert(2 * UPD * (int)sizeof(T) <= L::BYTES, "update operands fit");
    __shared__ float bS[GC * D];
    __shared__ float Ep[GC / 32][D];   // row block mi's part of the chunk's k . dk-inter sums
    __shared__ float Cp[D / 32][D];    // dv block ni's part of rowsum(R . P) at a checkpoint
    __shared__ __attribute__((aligned(16))) char U_raw[L::BYTES];
    T *U = (T *)U_raw;
    T *Sc = U + L::SOFF;
    using TO = Tiles<GC / 32, D / 32>;
    using TL = Tiles<D / 32, D / 32>;
    constexpr int NP = NTHR / D, RPP = GC / NP;   // log-gate gradient: parts of the rows per channel

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int64_t rb0 = row_base(p, s, h);
    const int64_t sh = (int64_t)gs * p.H + h;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    const int nS = min(s.S, p.n_segs_ub - s.s0);

    f32x16 R[TL::PER_WAVE];
    state_load<D>(R, p.Rseg + sh * D * D);
    // thread (channel c, part): the log-gate gradient beyond the current chunk
    float carry;
    {
        const float *Rs = p.Rseg + sh * D * D;
        const float *Pa = sl + 1 < nS ? p.Pseg + (sh + p.H) * D * D
                                      : p.Pfin + ((int64_t)s.i * p.H + h) * D * D;
        const int c = otid() % D, part = otid() / D;
        float x = 0.f;
        for (int dv = part; dv < D; dv += NP) x += Rs[dv * D + c] * Pa[dv * D + c];
        bS[part * D + c] = x;
        __syncthreads();
        carry = 0.f;
        for (int q = 0; q < NP; ++q) carry += bS[q * D + c];
    }

    // the chunk's Q, K, dO rows (the next chunk's, loaded ahead) and V rows
    // (loaded once K's have been staged for the last time)
    Raw<T, D, GC> rq, rk, rdo, rv;
    if (t0 < t1) {
        const int64_t rb = rb0 + (int64_t)(t1 - 1) * GC;
        const int Cl = min(GC, s.len - (t1 - 1) * GC);
        raw_load(rq, (const T *)p.Q + rb * D, Cl, RowId());
        raw_load(rk, (const T *)p.K + rb * D, Cl, RowId());
        raw_load(rdo, (const T *)p.dO + rb * D, Cl, RowId());
    }
    for (int t = t1 - 1; t >= t0; --t) {
        const int tok = t * GC;
        const int Ct = min(GC, s.len - tok);
        const bool more = t - 1 >= t0;   // (chunk t - 1 is full)
        const int64_t rb = rb0 + tok;
        const T *Q = (const T *)p.Q + rb * D;
        const T *K = (const T *)p.K + rb * D;
        const int64_t ch = (int64_t)(s.c0 + t) * p.H + h;
        const int l = olane();   // (once per chunk: see otid)
        // a checkpoint after this chunk: the carry is reset there to its exact
        // value, rowsum(R_t . P_{t+1}), the running sum's rounding dropped
        const int done = t - t0 + 1;
        const bool ck = p.Pck && done % GATED_CK == 0 && t + 1 < t1;
        if (ck) state_rowdot<D>(R, p.Pck + (sh * ((p.G - 1) / GATED_CK) + done / GATED_CK - 1) * D * D, Cp);
        chunk_gates<D>(bS, p.LG + rb * D, Ct);   // (its barriers also publish Cp)
        if (ck) {
            const int c = otid() % D;
            carry = 0.f;
#pragma unroll
            for (int q = 0; q < D / 32; ++q) carry += Cp[q][c];
        }
        auto exact = [&](int a, int b) { return exact_score<T, D>(Q, K, bS, a, b); };
        auto no_exact = [](int, int) { return 0.f; };

        // ---- dV ------------------------------------------------------------
        f32x16 dv[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(dv[k]);
        {
            T *Rv = U, *Kl = U + L::RPART;   // R rows [dv part][dk]; K 2^(b_last - b) rows
            for (int hh = 0; hh < L::NHALF; ++hh) {
                const int dv0 = hh * DH;
                __syncthreads();   // (first half: bS is written; later: the last products are done)
                if (!hh)
                    raw_store<T, D, GC, false>(rk, Kl, PD, Ct, RowId(),
                                               gate_scale<T>(bS, D, [](int) { return GC - 1; }));
                state_rows<D, DH>(R, dv0, [&](int dvv, int dk, const float *x) {
                    store4(Rv + dvv * PD + dk, x[0], x[1], x[2], x[3]);
                });
                __syncthreads();
#pragma unroll
                for (int k = 0; k < TO::PER_WAVE; ++k) {
                    int mi, ni;
                    if (TO::get(k, mi, ni, owave()) && ni * 32 >= dv0 && ni * 32 < dv0 + DH) {
                        // (bf16: dV accumulated transposed)
                        if constexpr (SW)
                            gemm_t<D>(dv[k], (const bf16 *)Kl, PD, mi * 32, (const bf16 *)Rv, PD, ni * 32 - dv0);
                        else
                            gemm<T, D>(dv[k], Kl, PD, mi * 32, Rv, PD, ni * 32 - dv0, l);
                    }
                }
            }
        }
        __syncthreads();
        // gated scores A (stored transposed, [key][query]): tiles (1,0), (1,1)
        // from K rows 0..63 with ref 32, then (0,0) from K rows 0..31 with ref 0
        T *Qg = U, *K64 = U + L::ROWS;
        raw_store<T, D, GC, false>(rq, Qg, PD, Ct, RowId(),
                                   gate_scale<T>(bS, D, [](int j) { return j & ~31; }, true));
        raw_store<T, D, GC, false>(rk, K64, PD, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 32; }));
        bool slow0, slow1;
        tile_spans<D>(bS, slow0, slow1);   // (its barrier also ends the staging)
        score_tiles<T, D, PD, PS>(Sc, Qg, K64, [](int ww) { return ww == 2 ? 32 : 0; }, false, true, true,
                                  exact, 6, true, Ct, slow0, slow1);
        __syncthreads();
        raw_store_map<T, D, GC, false>(rk, K64, PD, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 0; }),
                                       [](int j) { return j < 32 ? j : -1; });
        raw_load(rv, (const T *)p.V + rb * D, Ct, RowId());
        __syncthreads();
        score_tiles<T, D, PD, PS>(Sc, Qg, K64, [](int) { return 0; }, false, true, true, exact, 1, false, Ct,
                                  slow0, slow1);
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
            if (!TO::get(k, mi, ni, owave())) continue;
            if constexpr (SW) {
                gemm_rc_t<D, GC>(dv[k], (const bf16 *)Sc, PS, mi * 32, (const bf16 *)OT, ni * 32, frag_offs<D>(l));
                store_tile1_t(dv[k], (bf16 *)p.dV + rb * D, D, mi * 32, ni * 32, Ct);
            } else {
                gemm<T, GC>(dv[k], Sc, PS, mi * 32, OT, PS, ni * 32, l);
                store_rows(dv[k], (T *)p.dV + rb * D, D, mi * 32, ni * 32, Ct, olane());
            }
        }
        __syncthreads();

        // ---- dK ------------------------------------------------------------
        f32x16 dk[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) zero(dk[k]);
        T *Vr = U, *RT = U + L::ROWS;   // V rows; R as [dk][dv part]
        raw_store<T, D, GC, false>(rv, Vr, PD, Ct, RowId(), NoScale());
        for (int hh = 0; hh < L::NHALF; ++hh) {
            const int dv0 = hh * DH;
            if (hh) __syncthreads();
            // (stored like P in the dQ walk)
            state_rows<D, DH>(R, dv0, [&](int dvv, int dkk, const float *x) {
                if constexpr (SW) {
                    store4(RT + sw_off<D>(dvv, dkk), x[0], x[1], x[2], x[3]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) RT[(dkk + j) * PDH + dvv] = x[j];
                }
            });
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (!TO::get(k, mi, ni, owave())) continue;
                // (dK accumulated transposed, as dQ in the dQ walk)
                if constexpr (SW)
                    gemm_rc_t<D, DH>(dk[k], (const bf16 *)Vr + dv0, PD, mi * 32, (const bf16 *)RT, ni * 32,
                                     frag_offs<D>(l));
                else
                    gemm<T, DH>(dk[k], RT, PDH, ni * 32, Vr + dv0, PD, mi * 32, l);
            }
        }
        // the chunk's sum over its tokens of k . 2^(b_last - b) (V R^T), per
        // channel (see the dQ walk), then dk's scale for the in-chunk terms
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni, owave())) continue;
            const int i = mi * 32 + (l & 31), mJ = mi * 32 + 31, c0 = ni * 32 + (l >> 5) * 4;
            float x[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float kv[4] = {0.f, 0.f, 0.f, 0.f};
                if (i < Ct) load4f(K + (int64_t)i * D + c0 + 8 * q, kv);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = c0 + 8 * q + e;
                    const float bl = bS[(GC - 1) * D + c];
                    x[4 * q + e] = kv[e] * ex2(bl - bS[i * D + c]) * dk[k][4 * q + e];
                    dk[k][4 * q + e] *= ex2(bl - bS[mJ * D + c]);
                }
            }
            const float ep = half_colsum16(x, l);
            if (!(l & 1)) Ep[mi][ni * 32 + crow((l >> 1) & 15, l)] = ep;
        }
        __syncthreads();   // R's parts have been read
        T *dOr = U + L::ROWS;   // D_^T = V dO^T (upper tiles), then Q^T in three versions
        raw_store<T, D, GC, false>(rdo, dOr, PD, Ct, RowId(), NoScale());
        __syncthreads();
        score_tiles<T, D, PD, PS>(Sc, Vr, dOr, [](int ww) { return ww == 0 ? 0 : 32; }, true, false, false,
                                  no_exact, 7, true, Ct, slow0, slow1);
        __syncthreads();
        // rows 0..63 with ref row 31 as tile rows 0..63, rows 32..63 with ref
        // 63 as tile rows 64..95 (stored as the K versions of the dQ walk)
        T *QT3 = U;
        if constexpr (SW) {
            raw_store_sw<D, GC>(rq, (bf16 *)QT3, Ct, RowId(),
                                gate_scale<T>(bS, D, [](int) { return 31; }, true));
            raw_store_sw<D, GC>(rq, (bf16 *)QT3, Ct, RowId(),
                                gate_scale<T>(bS, D, [](int) { return 63; }, true),
                                [](int j) { return j >= 32 ? j + 32 : -1; });
        } else {
            raw_store<T, D, GC, true>(rq, QT3, PK, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return 31; }, true));
            raw_store_map<T, D, GC, true>(rq, QT3, PK, Ct, RowId(),
                                          gate_scale<T>(bS, D, [](int) { return 63; }, true),
                                          [](int j) { return j >= 32 ? j + 32 : -1; });
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni, owave())) continue;
            const bool slow = mi == 0 ? slow0 : slow1;
            if constexpr (SW) {
                const FragOffs<D> fo = frag_offs<D>(l);
                if (mi == 0)
                    gemm_rc_t<D, 32>(dk[k], (const bf16 *)Sc + 32, PS, 0, (const bf16 *)QT3, ni * 32, fo, 32);
                if (!slow)
                    gemm_rc_t<D, 32>(dk[k], (const bf16 *)Sc + 32 * mi, PS, 32 * mi, (const bf16 *)QT3, ni * 32,
                                     fo, mi ? 64 : 0);
            } else {
                if (mi == 0) gemm<T, 32>(dk[k], QT3 + 32, PK, ni * 32, Sc + 32, PS, 0, l);
                if (!slow) gemm<T, 32>(dk[k], QT3 + (mi ? 64 : 0), PK, ni * 32, Sc + 32 * mi, PS, 32 * mi, l);
            }
            const int i = mi * 32 + (l & 31), mJ = mi * 32 + 31;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = ni * 32 + crow(r, l);
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
            if constexpr (SW)
                store_tile1_t(dk[k], (bf16 *)p.dK + rb * D, D, mi * 32, ni * 32, Ct);
            else
                store_rows_t(dk[k], (T *)p.dK + rb * D, D, mi * 32, ni * 32, Ct, l);
        }
        __syncthreads();

        // ---- log-gate gradient ---------------------------------------------
        float *dBs = (float *)U_raw;   // [GC][D]: q dq - k dk
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni, owave())) continue;
            const int su = mi * 32 + (l & 31), c0 = ni * 32 + (l >> 5) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float x[4] = {0.f, 0.f, 0.f, 0.f};
                if (su < Ct) {
                    float kv[4];
                    load4f(K + (int64_t)su * D + c0 + 8 * q, kv);
                    load4f(p.dLG + (rb + su) * D + c0 + 8 * q, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] -= kv[e] * dk[k][4 * q + e];
                }
                store4(dBs + su * D + c0 + 8 * q, x[0], x[1], x[2], x[3]);
            }
        }
        __syncthreads();
        {   // suffix sums over the chunk's rows, NP parts per channel, plus the carry
            const int c = otid() % D, part = otid() / D, r0 = part * RPP;
            float x[RPP];
#pragma unroll
            for (int j = 0; j < RPP; ++j) x[j] = dBs[(r0 + j) * D + c];
#pragma unroll
            for (int j = RPP - 2; j >= 0; --j) x[j] += x[j + 1];
            __syncthreads();
            dBs[part * D + c] = x[0];
            __syncthreads();
            float off = carry;
            for (int q = part + 1; q < NP; ++q) off += dBs[q * D + c];
            // the chunk's total of q dq - k dk from the inter terms (see above)
            carry += p.Tq[ch * D + c] - (Ep[0][c] + Ep[1][c]);
            int o0 = r0 * D + c, nrow = Ct - r0;
            asm volatile("" : "+v"(o0), "+v"(nrow));
            float *out = p.dLG + rb * D + o0;
#pragma unroll
            for (int j = 0; j < RPP; ++j)
                if (j < nrow) out[j * D] = x[j] + off;
        }
        if (!more) break;

        // R <- Diag(2^(b_last)) R + (Q 2^b)^T dO
        __syncthreads();   // the part sums have been read
        T *QU = U, *OU = U + UPD;
        if constexpr (SW) {
            raw_store_sw<D, GC>(rq, (bf16 *)QU, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return -1; }));
            raw_store_sw<D, GC>(rdo, (bf16 *)OU, Ct, RowId(), NoScale());
        } else {
            raw_store<T, D, GC, true>(rq, QU, PS, Ct, RowId(), gate_scale<T>(bS, D, [](int) { return -1; }));
            raw_store<T, D, GC, true>(rdo, OU, PS, Ct, RowId(), NoScale());
        }
        raw_load(rq, Q - GC * D, GC, RowId());
        raw_load(rk, K - GC * D, GC, RowId());
        raw_load(rdo, (const T *)p.dO + (rb - GC) * D, GC, RowId());
        __syncthreads();
        state_decay<D>(R, bS);
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) {
            int mi, ni;
            if (!TL::get(k, mi, ni, owave())) continue;
            if constexpr (SW)
                gemm_cc<D, GC>(R[k], (const bf16 *)QU, mi * 32, (const bf16 *)OU, ni * 32, opaque(frag_offs<D>(l)));
            else
                gemm<T, GC>(R[k], QU, PS, mi * 32, OU, PS, ni * 32, l);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t gfwd(const Params &p, bool with_output, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY(launch_k(k_gfwd_local<T, D>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_gfwd_segscan<D>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    if (with_output) LASP_TRY(launch_k(k_gfwd_walk<T, D>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    return rec_event(ev, 3, st);
}

template <typename T, int D>
static hipError_t gbwd(const Params &p, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY(launch_k(k_gbwd_local<T, D>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_gbwd_segscan<D>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    LASP_TRY(launch_k(k_gbwd_walk_q<T, D>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(launch_k(k_gbwd_walk_kv<T, D>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    return rec_event(ev, 3, st);
}

hipError_t launch_fwd_gated(const Params &p, bool bf, bool with_output, hipStream_t st, hipEvent_t *ev) {
    if (p.C != GC || !p.LG || !p.Gs || !p.Pfin) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bf ? gfwd<bf16, 32>(p, with_output, st, ev) : gfwd<float, 32>(p, with_output, st, ev);
    case 64: return bf ? gfwd<bf16, 64>(p, with_output, st, ev) : gfwd<float, 64>(p, with_output, st, ev);
    case 128: return bf ? gfwd<bf16, 128>(p, with_output, st, ev) : gfwd<float, 128>(p, with_output, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_gated(const Params &p, bool bf, hipStream_t st, hipEvent_t *ev) {
    if (p.C != GC || !p.LG || !p.dLG || !p.Gs || !p.Pfin || !p.Tq) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bf ? gbwd<bf16, 32>(p, st, ev) : gbwd<float, 32>(p, st, ev);
    case 64: return bf ? gbwd<bf16, 64>(p, st, ev) : gbwd<float, 64>(p, st, ev);
    case 128: return bf ? gbwd<bf16, 128>(p, st, ev) : gbwd<float, 128>(p, st, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace lasp
