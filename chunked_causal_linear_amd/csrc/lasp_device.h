// Device-side helpers shared by the HIP kernel files of the library: element
// types, the MFMA micro-kernel, sequence bookkeeping of plain and packed
// batches, LDS staging and 32x32 tile GEMM / store helpers.  Not installed.
#pragma once
#include "lasp_internal.h"

namespace lasp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16 {
    uint16_t u;
};

template <typename T> struct Tr;
template <> struct Tr<float> {
    using frag = f32x4;
    static constexpr int VEC = 4;   // elements per 16 bytes
};
template <> struct Tr<bf16> {
    using frag = bf16x8_t;
    static constexpr int VEC = 8;
};

constexpr int NTHR = 256;   // 4 waves of 64
constexpr int NWAVE = 4;

// ---------------------------------------------------------------------------
// MFMA micro-kernel.  32x32 output tile, fp32 accumulate.  Lane l holds, for
// both element types, output rows (r/4)*8 + (l/32)*4 + r%4 (r = 0..15) of
// column l%32.  An operand fragment is 16 bytes per lane: row (l%32) of A (or
// column of B), contraction elements [(l/32)*VEC, (l/32)*VEC + VEC) of a
// 2*VEC-wide k-step.  bf16: one 32x32x16 MFMA; f32: four 32x32x2 MFMAs where
// step s pairs element s of both lane halves (A and B agree on the pairing).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma(f32x16 &c, const bf16x8_t &a, const bf16x8_t &b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16 &c, const f32x4 &a, const f32x4 &b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Host side: launch a kernel that takes Params by value and return that
// launch's own status (no hipGetLastError: an error the caller left pending is
// neither reported nor cleared here).
// ---------------------------------------------------------------------------
template <typename Kern>
inline hipError_t launch_k(Kern kernel, dim3 grid, dim3 block, hipStream_t st, const Params &p) {
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, st);
}
// Record event i of ev (if any) on st.
inline hipError_t rec_event(hipEvent_t *ev, int i, hipStream_t st) {
    return ev ? hipEventRecord(ev[i], st) : hipSuccess;
}
#define LASP_TRY(x)                                  \
    do {                                             \
        const hipError_t lasp_e_ = (x);              \
        if (lasp_e_ != hipSuccess) return lasp_e_;   \
    } while (0)

constexpr int SCAN_BATCH = 8;   // segment totals loaded per round trip in the segment scans

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// A buffer descriptor for `bytes` bytes from p, made from lane 0's address and
// size: every caller passes an address and size that are the same on all
// lanes of the wave, and saying so spares the compiler a loop over lanes
// around each buffer access.  Stores past `bytes` are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_buffer(const void *p, int bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)u, 0, __builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}
// Row (within the 32x32 tile) of accumulator element r for this lane.
__device__ __forceinline__ int crow(int r, int l = threadIdx.x & 63) {
    return (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
}

__device__ __forceinline__ float tof(float x) { return x; }
__device__ __forceinline__ float tof(bf16 x) { return __uint_as_float(((uint32_t)x.u) << 16); }
template <typename T> __device__ __forceinline__ T fromf(float x);
template <> __device__ __forceinline__ float fromf<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 fromf<bf16>(float x) {
    __bf16 h = (__bf16)x;   // round to nearest even (v_cvt_pk_bf16_f32)
    bf16 r;
    r.u = __builtin_bit_cast(uint16_t, h);
    return r;
}

// 16-byte load of VEC elements, widened to float.
__device__ __forceinline__ void load16(const float *p, float *f) {
    float4 v = *(const float4 *)p;
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}
__device__ __forceinline__ void load16(const bf16 *p, float *f) {
    uint4 v = *(const uint4 *)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Store 4 consecutive values (converted) at p.
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *(float4 *)p = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    const bf16x4_t v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};   // RNE, two packed cvts
    *(bf16x4_t *)p = v;
}

// lambda^e with lambda = 2^l2; lambda^0 = 1 exactly (also for lambda = 0).
__device__ __forceinline__ float dpow(float l2, float e) {
    return e == 0.f ? 1.f : __builtin_amdgcn_exp2f(e * l2);
}
__device__ __forceinline__ float head_log2_decay(const Params &p, int h) {
    return p.decay ? log2f(p.decay[h]) : 0.f;
}

// ---------------------------------------------------------------------------
// Sequence bookkeeping
// ---------------------------------------------------------------------------
struct Seq {
    int i;          // sequence index
    int64_t tok0;   // first token (packed batch: offset inside N)
    int len;        // tokens
    int T, S;       // chunks, segments
    int c0, s0;     // first global chunk / segment
};

__device__ __forceinline__ int last_le(const int32_t *pre, int n, int x) {
    // largest i in [0, n) with pre[i] <= x (pre non-decreasing, pre[0] = 0)
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Token range of packed sequence i, clamped into [0, N] so that malformed
// cu_seqlens can never address outside the tensors.
__device__ __forceinline__ void packed_bounds(const Params &p, int i, int &tok0, int &len) {
    const int a = min(max(p.cu[i], 0), p.N);
    const int b = min(max(p.cu[i + 1], a), p.N);
    tok0 = a;
    len = b - a;
}

__device__ __forceinline__ void seq_fill(const Params &p, int i, Seq &s) {
    s.i = i;
    if (!p.varlen) {
        s.tok0 = 0;
        s.len = p.N;
        s.T = p.T_fixed;
        s.S = p.S_fixed;
        s.c0 = i * p.T_fixed;
        s.s0 = i * p.S_fixed;
    } else {
        int tok0, len;
        packed_bounds(p, i, tok0, len);
        s.tok0 = tok0;
        s.len = len;
        s.c0 = p.chunk_prefix[i];
        s.T = p.chunk_prefix[i + 1] - s.c0;
        s.s0 = p.seg_prefix[i];
        s.S = p.seg_prefix[i + 1] - s.s0;
    }
}

// Global chunk gc -> (sequence, local chunk t).  False if gc is past the end.
__device__ __forceinline__ bool chunk_seq(const Params &p, int gc, Seq &s, int &t) {
    int i;
    if (!p.varlen) {
        if (gc >= p.nseq * p.T_fixed) return false;
        i = gc / p.T_fixed;
    } else {
        if (gc >= p.chunk_prefix[p.nseq]) return false;
        i = last_le(p.chunk_prefix, p.nseq, gc);
    }
    seq_fill(p, i, s);
    t = gc - s.c0;
    return gc < p.n_chunks_ub;
}

__device__ __forceinline__ bool seg_seq(const Params &p, int gs, Seq &s, int &sl) {
    int i;
    if (!p.varlen) {
        if (gs >= p.nseq * p.S_fixed) return false;
        i = gs / p.S_fixed;
    } else {
        if (gs >= p.seg_prefix[p.nseq]) return false;
        i = last_le(p.seg_prefix, p.nseq, gs);
    }
    seq_fill(p, i, s);
    sl = gs - s.s0;
    return gs < p.n_segs_ub;
}

// With p.end_by_sweep the sweep whose walk ends at a sequence's end writes the
// state there, and that segment's total is skipped: forwards, the sequence's
// last segment (when it reaches the sequence's last chunk); backwards, its
// first.  nS: the sequence's segments, min(s.S, p.n_segs_ub - s.s0).
__device__ __forceinline__ bool fwd_end_by_sweep(const Params &p, const Seq &s, int nS) {
    if (!p.end_by_sweep || nS <= 0) return false;
    const int t0 = (nS - 1) * p.G;
    const int t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    return t1 == s.T && t1 > t0;
}
__device__ __forceinline__ bool bwd_end_by_sweep(const Params &p, const Seq &s, int nS) {
    return p.end_by_sweep && nS > 0 && min(min(p.G, s.T), p.n_chunks_ub - s.c0) > 0;
}

// First row (token) of sequence s, head h, in the [B, H, N, d] layout.
__device__ __forceinline__ int64_t row_base(const Params &p, const Seq &s, int h) {
    return p.varlen ? ((int64_t)h * p.N + s.tok0) : (((int64_t)s.i * p.H + h) * p.N);
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Map ids so
// that each XCD gets a contiguous range of logical work items: neighbouring
// chunks of one head then share that XCD's L2.  n is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

// ---------------------------------------------------------------------------
// LDS staging and tile GEMM helpers (all 256 threads take part in staging)
// ---------------------------------------------------------------------------
// dst[r][c] = src[r][c] for a R x W tile; rows >= nvalid become zero.
template <typename T, int R, int W>
__device__ __forceinline__ void stage_rows(T *dst, int pitch, const T *src, int nvalid) {
    constexpr int V = Tr<T>::VEC;
    constexpr int PR = W / V;
    for (int i = threadIdx.x; i < R * PR; i += NTHR) {
        const int r = i / PR, c = (i % PR) * V;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < nvalid) v = *(const uint4 *)(src + (int64_t)r * W + c);
        *(uint4 *)(dst + r * pitch + c) = v;
    }
}

// dst[c][r] = scale(r) * src[r][c] (transposed, token index contiguous);
// rows >= nvalid become zero.
template <typename T, int R, int W, typename F>
__device__ __forceinline__ void stage_rows_T(T *dst, int pitch, const T *src, int nvalid,
                                             F scale) {
    constexpr int V = Tr<T>::VEC;
    for (int i = threadIdx.x; i < R * (W / V); i += NTHR) {
        const int r = i % R, c = (i / R) * V;
        float f[V];
        if (r < nvalid) {
            load16(src + (int64_t)r * W + c, f);
            const float s = scale(r);
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] *= s;
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) dst[(c + e) * pitch + r] = fromf<T>(f[e]);
    }
}

struct One {
    __device__ float operator()(int) const { return 1.f; }
};

// acc += A[m0..m0+32)[0..K) * B[n0..n0+32)[0..K)^T, A and B in LDS with the
// contraction index contiguous (pitches pa, pb in elements).
template <typename T, int K>
__device__ __forceinline__ void gemm(f32x16 &acc, const T *As, int pa, int m0, const T *Bs,
                                     int pb, int n0, int l = lane_id()) {
    constexpr int V = Tr<T>::VEC;
    using Fr = typename Tr<T>::frag;
    const T *ap = As + (m0 + (l & 31)) * pa + (l >> 5) * V;
    const T *bp = Bs + (n0 + (l & 31)) * pb + (l >> 5) * V;
#pragma unroll
    for (int k = 0; k < K; k += 2 * V) {
        const Fr a = *(const Fr *)(ap + k);
        const Fr b = *(const Fr *)(bp + k);
        mma(acc, a, b);
    }
}

// Y[n0 + col][m0 + row] = f(acc, m0 + row, n0 + col): transposed store of a
// 32x32 tile (4 consecutive rows per lane per store).  Y in LDS or global.
template <typename T, typename F>
__device__ __forceinline__ void store_T(const f32x16 &acc, T *Y, int64_t py, int m0, int n0,
                                        F f) {
    const int l = lane_id(), col = l & 31, g = l >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int m = m0 + q * 8 + g * 4;
        store4(Y + (int64_t)(n0 + col) * py + m, f(acc[q * 4 + 0], m + 0, n0 + col),
               f(acc[q * 4 + 1], m + 1, n0 + col), f(acc[q * 4 + 2], m + 2, n0 + col),
               f(acc[q * 4 + 3], m + 3, n0 + col));
    }
}

struct Ident {
    __device__ float operator()(float x, int, int) const { return x; }
};

// G[(m0+row)][n0+col] = acc for rows < nvalid (row-major global store).
template <typename T>
__device__ __forceinline__ void store_rows(const f32x16 &acc, T *G, int64_t ld, int m0, int n0,
                                           int nvalid, int l = lane_id()) {
    const int col = l & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = m0 + crow(r, l);
        if (row < nvalid) G[(int64_t)row * ld + n0 + col] = fromf<T>(acc[r]);
    }
}

// Tiles of a (MT*32) x (NT*32) output are dealt to the 4 waves round-robin.
template <int MT, int NT>
struct Tiles {
    static constexpr int N = MT * NT;
    static constexpr int PER_WAVE = (N + NWAVE - 1) / NWAVE;
    __device__ static bool get(int k, int &mi, int &ni, int w = wave_id()) {
        const int tile = w + k * NWAVE;
        mi = tile / NT;
        ni = tile % NT;
        return tile < N;
    }
};

__device__ __forceinline__ void zero(f32x16 &a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// ---------------------------------------------------------------------------
// bf16 operand fragments for the 32x32x16 MFMA, read from LDS tiles.  Operands
// whose contraction index is the token index come from row-major tiles via the
// LDS transpose read (ds_read_b64_tr_b16), so no transposed copies are made.
// ---------------------------------------------------------------------------
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Operand fragment from an LDS tile stored X[k][n] (n contiguous), operand row
// n0 + lane%32.  With g = lane/32 the 8 contraction elements are
// k0 + 8g + [0, 8) (PERM = false) or k0 + 4g + {0..3, 8..11} (PERM = true).
// ds_read_b64_tr_b16 works on groups of 16 lanes: when lane i of a group reads
// the 4 elements at row rb + i/4, columns cb + 4*(i%4), lane j of the group
// receives rows rb + 0..3 of column cb + j.
template <bool PERM>
__device__ __forceinline__ bf16x8_t frag_cols(const bf16 *X, int pitch, int k0, int n0,
                                              int l = lane_id()) {
    const int i = l & 15, h = l >> 4, g = h >> 1;
    const int col = n0 + (h & 1) * 16 + 4 * (i & 3);
    const int ra = k0 + (PERM ? 4 * g : 8 * g) + (i >> 2);
    const int rb = ra + (PERM ? 8 : 4);
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(X + ra * pitch + col));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(X + rb * pitch + col));
    const v8s c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, c);
}

__device__ __forceinline__ bf16x8_t pack8(float a0, float a1, float a2, float a3, float a4,
                                          float a5, float a6, float a7) {
    bf16x8_t r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// ---------------------------------------------------------------------------
// Unpadded LDS tiles.  global_load_lds_dwordx4 writes lane l's 16 bytes to
// lds_base + 16*l, so token tiles are stored without padding and their 16-byte
// pieces are permuted within each row: piece p of row r sits in slot
// r*PR + (p ^ key(r)), PR = pieces per row.  key(r) depends on r mod 16 and is
// linear over GF(2) in its four bits; it is chosen (by exhaustive search over
// such keys) so that the operand reads below touch every LDS bank once per
// access group, both for 128-byte and for 256-byte bank rows:
//   frag_rows_sw  ds_read_b128, 32 consecutive rows, one piece each;
//   frag_cols_sw  ds_read_b64_tr_b16, 4 consecutive rows x 2 or 4 pieces.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <int D> struct SwKey {
    // images of row bits 0..3; key(r) = XOR of the images of the set bits
    static constexpr int m0 = D == 128 ? 4 : (D == 64 ? 2 : 0);
    static constexpr int m1 = D == 128 ? 10 : (D == 64 ? 4 : 2);
    static constexpr int m2 = 1, m3 = 2;
    static constexpr unsigned long long table() {
        unsigned long long t = 0;
        for (int r = 0; r < 16; ++r) {
            const int k = ((r & 1) ? m0 : 0) ^ ((r & 2) ? m1 : 0) ^ ((r & 4) ? m2 : 0) ^
                          ((r & 8) ? m3 : 0);
            t |= (unsigned long long)k << (4 * r);
        }
        return t;
    }
    static constexpr unsigned long long T = table();
};

template <int D>
__device__ __forceinline__ int sw_key(int r) {
    return (int)((SwKey<D>::T >> (4 * (r & 15))) & 15);
}

template <int D>
__device__ __forceinline__ int sw_off(int r, int c) {
    constexpr int PR = D / 8;
    return (r * PR + ((c >> 3) ^ sw_key<D>(r))) * 8 + (c & 7);
}

// Operand fragments from swizzled tiles (the layout of frag_cols above, with
// sw_off placement).  The lane-dependent part of every fragment address is a
// per-lane byte offset computed once (FragOffs); a fragment address is then
// that offset XOR a wave-uniform term, plus a wave-uniform base: one VALU
// operation.  This holds for tiles whose first row is a multiple of 16: the
// XOR only touches the piece bits of the offset.
//   frag_rows: rows r0 + lane%32, k = k0 + (lane/32)*8 + [0, 8)   (k0 % 16 == 0)
//   frag_cols: operand row n0 + lane%32 of a tile stored [k][n]      (n0 % 32 == 0)
template <int D> struct FragOffs {
    uint32_t rows;          // frag_rows: XOR 2*k0, add 2*r0*D
    uint32_t cols[2][2];    // frag_cols [PERM][first/second read]: XOR 2*n0, add 2*k0*D
};

template <int D>
__device__ __forceinline__ FragOffs<D> frag_offs(int l) {
    FragOffs<D> o;
    o.rows = 2u * sw_off<D>(l & 31, (l >> 5) * 8);
    const int i = l & 15, h = l >> 4, g = h >> 1;
    const int col = (h & 1) * 16 + 4 * (i & 3);
#pragma unroll
    for (int perm = 0; perm < 2; ++perm) {
        const int ra = (perm ? 4 * g : 8 * g) + (i >> 2);
        o.cols[perm][0] = 2u * sw_off<D>(ra, col);
        o.cols[perm][1] = 2u * sw_off<D>(ra + (perm ? 8 : 4), col);
    }
    return o;
}

// A copy of o that the compiler cannot see through: address terms derived from
// it are then computed where they are used rather than hoisted out of loops
// into registers of their own.
template <int D>
__device__ __forceinline__ FragOffs<D> opaque(FragOffs<D> o) {
    asm volatile("" : "+v"(o.rows), "+v"(o.cols[0][0]), "+v"(o.cols[0][1]), "+v"(o.cols[1][0]),
                 "+v"(o.cols[1][1]));
    return o;
}

template <int D>
__device__ __forceinline__ bf16x8_t frag_rows_sw(const bf16 *X, const FragOffs<D> &o, int r0, int k0) {
    const char *b = (const char *)X + 2 * r0 * D;
    return *(const bf16x8_t *)(b + (o.rows ^ (uint32_t)(2 * k0)));
}

template <int D, bool PERM>
__device__ __forceinline__ bf16x8_t frag_cols_sw(const bf16 *X, const FragOffs<D> &o, int k0, int n0) {
    const char *b = (const char *)X + 2 * k0 * D;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s *)(b + (o.cols[PERM][0] ^ (uint32_t)(2 * n0))));
    const v4s c = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s *)(b + (o.cols[PERM][1] ^ (uint32_t)(2 * n0))));
    const v8s r = __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, r);
}

}  // namespace lasp
