// HIP kernels (gfx950 / MI355X) for chunked causal linear attention.
//
// Sources: "Linear Attention Sequence Parallelism" (arXiv 2404.02882), Sec. 3.2:
// chunk decomposition into intra-chunk (Eq. 7) and inter-chunk (Eq. 9) terms,
// the chunk state update (Eq. 10), backward terms (Eqs. 14-23); and the LASP-2
// review page (arXiv 2502.07563): chunk memory states M_t and their prefix /
// suffix sums replace the serial exchange.
//
// Notation (one head of one sequence, chunk t of length C_t, 0-based row i):
//   D_t[i][j]  = lambda^(i-j) for i >= j else 0      (the decayed causal mask)
//   Lam_t      = diag(lambda^(i+1))                   (Lambda of Alg. 2)
//   Gam_t      = diag(lambda^(C_t-1-j))               (lambda^C Lambda^-1 of Eq. 10)
//   P_t        = state entering chunk t (the cached KV_{t-1})
//   R_t        = reverse state entering chunk t from the right (dKV_{t+1})
//   fwd:  O_t  = [(Q_t K_t^T) . D_t] V_t + Lam_t Q_t P_t
//         P_{t+1} = lambda^C_t P_t + (Gam_t K_t)^T V_t
//   bwd:  R_{t-1} = lambda^C_t R_t + (Lam_t Q_t)^T dO_t
//         dQ_t = [(dO_t V_t^T) . D_t] K_t + Lam_t dO_t P_t^T
//         dK_t = [(dO_t V_t^T) . D_t]^T Q_t + Gam_t V_t R_t^T
//         dV_t = [(Q_t K_t^T) . D_t]^T dO_t + Gam_t K_t R_t
//
// The serial recurrence over chunks is split two-level for parallelism: G
// chunks form a segment; one workgroup per (segment, head) sweeps its chunks
// carrying a local state in MFMA accumulators (k_*_local), a small scan carries
// states across segments (k_*_segscan), and the output / gradient kernels run
// one workgroup per (chunk, head), combining the segment state with the local
// one.  All products run on MFMA (32x32x16 bf16 or 32x32x2 f32) with operands
// staged in LDS so that the contraction index is contiguous for every operand.
#include "lasp_device.h"

#include <mutex>

namespace lasp {

// ---------------------------------------------------------------------------
// Packed-batch tables: chunk_prefix[i] = sum_{i'<i} ceil(L_i'/C),
// seg_prefix[i] = sum_{i'<i} ceil(T_i'/G).  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR) void k_setup(Params p) {
    __shared__ int sc[NTHR], ss[NTHR];
    __shared__ int carry_c, carry_s;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry_c = 0;
        carry_s = 0;
    }
    __syncthreads();
    for (int base = 0; base < p.nseq; base += NTHR) {
        const int i = base + tid;
        int tc = 0, ts = 0;
        if (i < p.nseq) {
            int t0, L;
            packed_bounds(p, i, t0, L);
            tc = L > 0 ? (L + p.C - 1) / p.C : 0;
            ts = (tc + p.G - 1) / p.G;
        }
        sc[tid] = tc;
        ss[tid] = ts;
        __syncthreads();
        for (int off = 1; off < NTHR; off <<= 1) {   // inclusive scan
            const int a = tid >= off ? sc[tid - off] : 0;
            const int b = tid >= off ? ss[tid - off] : 0;
            __syncthreads();
            sc[tid] += a;
            ss[tid] += b;
            __syncthreads();
        }
        if (i < p.nseq) {
            p.chunk_prefix[i] = carry_c + sc[tid] - tc;
            p.seg_prefix[i] = carry_s + ss[tid] - ts;
        }
        __syncthreads();
        if (tid == NTHR - 1) {
            carry_c += sc[tid];
            carry_s += ss[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        p.chunk_prefix[p.nseq] = carry_c;
        p.seg_prefix[p.nseq] = carry_s;
    }
}

// ---------------------------------------------------------------------------
// Forward 1: local states.  One workgroup per (segment, head).  Sweeps the
// segment's chunks in order, with L = 0 at the segment start:
//   Lc[t] = L (stored, bf16/f32, [dv][dk]);  L = lambda^C_t L + (Gam_t K_t)^T V_t
// and finally Z[segment] = L (f32).  (LASP Eq. 10 / Alg. 2 state update;
// LASP-2's M_t = K_t^T V_t accumulated.)
// ---------------------------------------------------------------------------
template <typename T, int D, int BT>
__global__ __launch_bounds__(NTHR) void k_fwd_local(Params p) {
    constexpr int PT = BT + Tr<T>::VEC;
    __shared__ __attribute__((aligned(16))) T KT_s[D * PT];
    __shared__ __attribute__((aligned(16))) T VT_s[D * PT];
    using TL = Tiles<D / 32, D / 32>;

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const float l2 = head_log2_decay(p, h);
    const int64_t rb = row_base(p, s, h);
    const T *K = (const T *)p.K + rb * D;
    const T *V = (const T *)p.V + rb * D;
    const bool store_local = p.G > 1;

    f32x16 acc[TL::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) zero(acc[k]);

    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    for (int t = t0; t < t1; ++t) {
        const int tok = t * p.C;
        const int Ct = min(p.C, s.len - tok);
        if (store_local) {
            T *Lt = (T *)p.Lc + ((int64_t)(s.c0 + t) * p.H + h) * D * D;
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) store_T(acc[k], Lt, D, mi * 32, ni * 32, Ident());
            }
        }
        const float dc = dpow(l2, (float)Ct);
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) acc[k] *= dc;
        for (int b0 = 0; b0 < Ct; b0 += BT) {
            const int nv = min(BT, Ct - b0);
            __syncthreads();
            stage_rows_T<T, BT, D>(KT_s, PT, K + (int64_t)(tok + b0) * D, nv,
                                   [&](int r) { return dpow(l2, (float)(Ct - 1 - (b0 + r))); });
            stage_rows_T<T, BT, D>(VT_s, PT, V + (int64_t)(tok + b0) * D, nv, One());
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) gemm<T, BT>(acc[k], KT_s, PT, mi * 32, VT_s, PT, ni * 32);
            }
        }
    }
    float *Zs = p.Z + ((int64_t)gs * p.H + h) * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni)) store_T(acc[k], Zs, D, mi * 32, ni * 32, Ident());
    }
}

// ---------------------------------------------------------------------------
// Forward 2: scan over segments, one thread per state element.
//   Pseg[0] = M_in;  Pseg[s+1] = lambda^len_s Pseg[s] + Z[s];  M_out = Pfin = last.
// (LASP-2 prefix sum of gathered states; LASP Alg. 2 receive/send as a scan.)
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(NTHR) void k_fwd_segscan(Params p) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    const int ih = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * NTHR + threadIdx.x;
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const float l2 = head_log2_decay(p, h);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;   // [dk][dv] of the API states
    float P = p.M_in ? p.M_in[mo] : 0.f;
    const int seg_tokens = p.G * p.C;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    // with end_by_sweep the last segment's total is not computed: the state
    // after it comes from the output sweep
    const bool by_sweep = fwd_end_by_sweep(p, s, nS);
    const int nZ = by_sweep ? nS - 1 : nS;
    // the totals are loaded SCAN_BATCH segments at a time, ahead of the
    // stores: one memory latency per batch instead of one per segment
    for (int b0 = 0; b0 < nS; b0 += SCAN_BATCH) {
        float z[SCAN_BATCH];
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j)
            z[j] = b0 + j < nZ ? p.Z[((int64_t)(s.s0 + b0 + j) * p.H + h) * D * D + e] : 0.f;
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            const int sl = b0 + j;
            if (sl < nS) {
                const int64_t idx = ((int64_t)(s.s0 + sl) * p.H + h) * D * D + e;
                ((T *)p.Pseg)[idx] = fromf<T>(P);
                const int len_s = min(seg_tokens, s.len - sl * seg_tokens);
                P = dpow(l2, (float)len_s) * P + z[j];
            }
        }
    }
    if (by_sweep) return;
    if (p.M_out) p.M_out[mo] = P;
    if (p.Pfin) p.Pfin[(int64_t)ih * D * D + e] = P;
}

// ---------------------------------------------------------------------------
// Forward 3: output, one workgroup per (chunk, head).
//   O_t = [(Q_t K_t^T) . D_t] V_t + Lam_t Q_t P_t      (LASP Eqs. 7, 9, 11)
// with P_t = lambda^off Pseg + Lc[t] (off = tokens from the segment start).
// Query blocks of 64 rows; key blocks 0..qb; the score tile is computed
// transposed (keys x queries) so that its transposed store gives the A operand.
// ---------------------------------------------------------------------------
template <typename T, int D, int BT>
__global__ __launch_bounds__(NTHR) void k_fwd_out(Params p) {
    constexpr int V = Tr<T>::VEC;
    constexpr int PD = D + V;    // pitch: feature-contiguous rows
    constexpr int PT = BT + V;   // pitch: token-contiguous rows
    __shared__ __attribute__((aligned(16))) T PT_s[D * PD];   // P^T [dv][dk]
    __shared__ __attribute__((aligned(16))) T Q_s[BT * PD];
    __shared__ __attribute__((aligned(16))) T K_s[BT * PD];
    __shared__ __attribute__((aligned(16))) T VT_s[D * PT];   // V^T [dv][key]
    __shared__ __attribute__((aligned(16))) T S_s[BT * PT];   // masked scores [query][key]
    using TO = Tiles<BT / 32, D / 32>;
    using TS = Tiles<BT / 32, BT / 32>;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid % p.H, gc = lid / p.H;
    Seq s;
    int t;
    if (!chunk_seq(p, gc, s, t)) return;
    const float l2 = head_log2_decay(p, h);
    const int tok = t * p.C;
    const int Ct = min(p.C, s.len - tok);
    const int sl = t / p.G;
    if (s.s0 + sl >= p.n_segs_ub) return;   // only with malformed cu_seqlens
    const int off = (t - sl * p.G) * p.C;
    const int64_t rb = row_base(p, s, h) + tok;
    const T *Q = (const T *)p.Q + rb * D;
    const T *K = (const T *)p.K + rb * D;
    const T *Vg = (const T *)p.V + rb * D;
    T *O = (T *)p.O + rb * D;

    {   // P_t^T into LDS
        const float *Ps = p.Pseg + ((int64_t)(s.s0 + sl) * p.H + h) * D * D;
        const T *Lt = (const T *)p.Lc + ((int64_t)(s.c0 + t) * p.H + h) * D * D;
        const float doff = dpow(l2, (float)off);
        const bool has_local = p.G > 1;
        for (int e = threadIdx.x * V; e < D * D; e += NTHR * V) {
            float pf[V], lf[V];
#pragma unroll
            for (int j = 0; j < V; j += 4) load16(Ps + e + j, pf + j);
            if (has_local) load16(Lt + e, lf);
            else {
#pragma unroll
                for (int j = 0; j < V; ++j) lf[j] = 0.f;
            }
            const int dv = e / D, dk = e % D;
#pragma unroll
            for (int j = 0; j < V; ++j) PT_s[dv * PD + dk + j] = fromf<T>(doff * pf[j] + lf[j]);
        }
    }

    const int nb = (Ct + BT - 1) / BT;
    for (int qb = 0; qb < nb; ++qb) {
        const int nvq = min(BT, Ct - qb * BT);
        __syncthreads();
        stage_rows<T, BT, D>(Q_s, PD, Q + (int64_t)qb * BT * D, nvq);
        __syncthreads();
        f32x16 o[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            zero(o[k]);
            int mi, ni;
            if (TO::get(k, mi, ni)) {
                gemm<T, D>(o[k], Q_s, PD, mi * 32, PT_s, PD, ni * 32);   // Q_t P_t
#pragma unroll
                for (int r = 0; r < 16; ++r)                              // Lam_t rows
                    o[k][r] *= dpow(l2, (float)(qb * BT + mi * 32 + crow(r) + 1));
            }
        }
        for (int kb = 0; kb <= qb; ++kb) {
            const int nvk = min(BT, Ct - kb * BT);
            __syncthreads();
            stage_rows<T, BT, D>(K_s, PD, K + (int64_t)kb * BT * D, nvk);
            stage_rows_T<T, BT, D>(VT_s, PT, Vg + (int64_t)kb * BT * D, nvk, One());
            __syncthreads();
            {   // S^T tiles (keys x queries)
                for (int k = 0; k < TS::PER_WAVE; ++k) {
                    int mi, ni;
                    if (!TS::get(k, mi, ni)) continue;
                    f32x16 st;
                    zero(st);
                    gemm<T, D>(st, K_s, PD, mi * 32, Q_s, PD, ni * 32);
                    store_T(st, S_s, PT, mi * 32, ni * 32, [&](float x, int j, int i) {
                        const int gi = qb * BT + i, gj = kb * BT + j;
                        return (gi >= gj && gi < Ct) ? x * dpow(l2, (float)(gi - gj)) : 0.f;
                    });
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni)) gemm<T, BT>(o[k], S_s, PT, mi * 32, VT_s, PT, ni * 32);
            }
        }
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni))
                store_rows(o[k], O + (int64_t)qb * BT * D, D, mi * 32, ni * 32, nvq);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward 1: local reverse states, one workgroup per (segment, head), chunks
// swept last to first with Rl = 0 at the segment end:
//   Rc[t] = Rl;  Rl = lambda^C_t Rl + (Lam_t Q_t)^T dO_t;   W[segment] = Rl.
// (LASP Eq. 20 / Alg. 3 dKV update; LASP-2 suffix sums of dM_t.)
// ---------------------------------------------------------------------------
template <typename T, int D, int BT>
__global__ __launch_bounds__(NTHR) void k_bwd_local(Params p) {
    constexpr int PT = BT + Tr<T>::VEC;
    __shared__ __attribute__((aligned(16))) T QT_s[D * PT];
    __shared__ __attribute__((aligned(16))) T OT_s[D * PT];
    using TL = Tiles<D / 32, D / 32>;

    const int h = blockIdx.x % p.H, gs = blockIdx.x / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const float l2 = head_log2_decay(p, h);
    const int64_t rb = row_base(p, s, h);
    const T *Q = (const T *)p.Q + rb * D;
    const T *dO = (const T *)p.dO + rb * D;
    const bool store_local = p.G > 1;

    f32x16 acc[TL::PER_WAVE];
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) zero(acc[k]);

    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    for (int t = t1 - 1; t >= t0; --t) {
        const int tok = t * p.C;
        const int Ct = min(p.C, s.len - tok);
        if (store_local) {
            T *Rt = (T *)p.Rc + ((int64_t)(s.c0 + t) * p.H + h) * D * D;
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) store_T(acc[k], Rt, D, mi * 32, ni * 32, Ident());
            }
        }
        const float dc = dpow(l2, (float)Ct);
#pragma unroll
        for (int k = 0; k < TL::PER_WAVE; ++k) acc[k] *= dc;
        for (int b0 = 0; b0 < Ct; b0 += BT) {
            const int nv = min(BT, Ct - b0);
            __syncthreads();
            stage_rows_T<T, BT, D>(QT_s, PT, Q + (int64_t)(tok + b0) * D, nv,
                                   [&](int r) { return dpow(l2, (float)(b0 + r + 1)); });
            stage_rows_T<T, BT, D>(OT_s, PT, dO + (int64_t)(tok + b0) * D, nv, One());
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TL::PER_WAVE; ++k) {
                int mi, ni;
                if (TL::get(k, mi, ni)) gemm<T, BT>(acc[k], QT_s, PT, mi * 32, OT_s, PT, ni * 32);
            }
        }
    }
    float *Ws = p.W + ((int64_t)gs * p.H + h) * D * D;
#pragma unroll
    for (int k = 0; k < TL::PER_WAVE; ++k) {
        int mi, ni;
        if (TL::get(k, mi, ni)) store_T(acc[k], Ws, D, mi * 32, ni * 32, Ident());
    }
}

// ---------------------------------------------------------------------------
// Backward 2: reverse scan over segments, one thread per state element.
//   Rseg[S-1] = dM_out;  Rseg[s-1] = lambda^len_s Rseg[s] + W[s];  dM_in = Rfin = last.
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(NTHR) void k_bwd_segscan(Params p) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    const int ih = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * NTHR + threadIdx.x;
    if (e >= D * D) return;
    const int i = ih / p.H, h = ih % p.H;
    Seq s;
    seq_fill(p, i, s);
    const float l2 = head_log2_decay(p, h);
    const int dv = e / D, dk = e % D;
    const int64_t mo = ((int64_t)ih * D + dk) * D + dv;
    float R = p.dM_out ? p.dM_out[mo] : 0.f;
    const int seg_tokens = p.G * p.C;
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    // with end_by_sweep the first segment's total is not computed: the state
    // before it comes from the dV sweep
    const bool by_sweep = bwd_end_by_sweep(p, s, nS);
    const int w0 = by_sweep ? 1 : 0;
    for (int b0 = nS - 1; b0 >= 0; b0 -= SCAN_BATCH) {   // batches as in the forward scan
        float wv[SCAN_BATCH];
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j)
            wv[j] = b0 - j >= w0 ? p.W[((int64_t)(s.s0 + b0 - j) * p.H + h) * D * D + e] : 0.f;
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
            const int sl = b0 - j;
            if (sl >= 0) {
                const int64_t idx = ((int64_t)(s.s0 + sl) * p.H + h) * D * D + e;
                ((T *)p.Rseg)[idx] = fromf<T>(R);
                const int len_s = min(seg_tokens, s.len - sl * seg_tokens);
                R = dpow(l2, (float)len_s) * R + wv[j];
            }
        }
    }
    if (by_sweep) return;
    if (p.dM_in) p.dM_in[mo] = R;
    if (p.Rfin) p.Rfin[(int64_t)ih * D * D + e] = R;
}

// Combine a segment state and a local state into LDS:
//   X = scale * seg[dv][dk] + loc[dv][dk];  stored as Y[dv][dk] (transpose =
//   false) or Y[dk][dv] (transpose = true).
template <typename T, int D>
__device__ __forceinline__ void combine_state(T *Y, int py, const float *seg, const T *loc,
                                              float scale, bool transpose) {
    constexpr int V = Tr<T>::VEC;
    for (int e = threadIdx.x * V; e < D * D; e += NTHR * V) {
        float pf[V], lf[V];
#pragma unroll
        for (int j = 0; j < V; j += 4) load16(seg + e + j, pf + j);
        if (loc) load16(loc + e, lf);
        else {
#pragma unroll
            for (int j = 0; j < V; ++j) lf[j] = 0.f;
        }
        const int dv = e / D, dk = e % D;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const T x = fromf<T>(scale * pf[j] + lf[j]);
            if (transpose) Y[(dk + j) * py + dv] = x;
            else Y[dv * py + dk + j] = x;
        }
    }
}

// ---------------------------------------------------------------------------
// Backward 3: gradients, one workgroup per (chunk, head), three phases that
// share one LDS footprint:
//   A  dQ_t = [(dO_t V_t^T) . D_t] K_t + Lam_t dO_t P_t^T      (LASP Eqs. 14, 16)
//   B  dV_t = [(Q_t K_t^T) . D_t]^T dO_t + Gam_t K_t R_t        (LASP Eqs. 21, 22)
//   C  dK_t = [(dO_t V_t^T) . D_t]^T Q_t + Gam_t V_t R_t^T      (LASP Eqs. 17, 19)
// ---------------------------------------------------------------------------
template <typename T, int D, int BT>
__global__ __launch_bounds__(NTHR) void k_bwd_grads(Params p) {
    constexpr int V = Tr<T>::VEC;
    constexpr int PD = D + V;
    constexpr int PT = BT + V;
    __shared__ __attribute__((aligned(16))) T St_s[D * PD];   // state operand
    __shared__ __attribute__((aligned(16))) T A_s[BT * PD];   // query-block rows
    __shared__ __attribute__((aligned(16))) T B_s[BT * PD];   // key-block rows
    __shared__ __attribute__((aligned(16))) T X_s[D * PT];    // transposed block
    __shared__ __attribute__((aligned(16))) T S_s[BT * PT];   // masked score tile
    using TO = Tiles<BT / 32, D / 32>;
    using TS = Tiles<BT / 32, BT / 32>;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid % p.H, gc = lid / p.H;
    Seq s;
    int t;
    if (!chunk_seq(p, gc, s, t)) return;
    const float l2 = head_log2_decay(p, h);
    const int tok = t * p.C;
    const int Ct = min(p.C, s.len - tok);
    const int sl = t / p.G;
    if (s.s0 + sl >= p.n_segs_ub) return;   // only with malformed cu_seqlens
    const int off = (t - sl * p.G) * p.C;                                // tokens before, in segment
    const int seg_end = min((sl + 1) * p.G * p.C, s.len);
    const int roff = seg_end - (tok + Ct);                               // tokens after, in segment
    const int64_t rb = row_base(p, s, h) + tok;
    const T *Q = (const T *)p.Q + rb * D;
    const T *K = (const T *)p.K + rb * D;
    const T *Vg = (const T *)p.V + rb * D;
    const T *dO = (const T *)p.dO + rb * D;
    const int64_t sidx = ((int64_t)(s.s0 + sl) * p.H + h) * D * D;
    const int64_t cidx = ((int64_t)(s.c0 + t) * p.H + h) * D * D;
    const bool has_local = p.G > 1;
    const int nb = (Ct + BT - 1) / BT;

    // ---- phase A: dQ ----
    combine_state<T, D>(St_s, PD, p.Pseg + sidx, has_local ? (const T *)p.Lc + cidx : nullptr,
                        dpow(l2, (float)off), true);                    // P [dk][dv]
    for (int qb = 0; qb < nb; ++qb) {
        const int nvq = min(BT, Ct - qb * BT);
        __syncthreads();
        stage_rows<T, BT, D>(A_s, PD, dO + (int64_t)qb * BT * D, nvq);
        __syncthreads();
        f32x16 acc[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            zero(acc[k]);
            int mi, ni;
            if (TO::get(k, mi, ni)) {
                gemm<T, D>(acc[k], A_s, PD, mi * 32, St_s, PD, ni * 32);   // dO_t P_t^T
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[k][r] *= dpow(l2, (float)(qb * BT + mi * 32 + crow(r) + 1));
            }
        }
        for (int kb = 0; kb <= qb; ++kb) {
            const int nvk = min(BT, Ct - kb * BT);
            __syncthreads();
            stage_rows<T, BT, D>(B_s, PD, Vg + (int64_t)kb * BT * D, nvk);
            stage_rows_T<T, BT, D>(X_s, PT, K + (int64_t)kb * BT * D, nvk, One());
            __syncthreads();
            {   // E^T tiles (keys x queries) = V dO^T
                for (int k = 0; k < TS::PER_WAVE; ++k) {
                    int mi, ni;
                    if (!TS::get(k, mi, ni)) continue;
                    f32x16 et;
                    zero(et);
                    gemm<T, D>(et, B_s, PD, mi * 32, A_s, PD, ni * 32);
                    store_T(et, S_s, PT, mi * 32, ni * 32, [&](float x, int j, int i) {
                        const int gi = qb * BT + i, gj = kb * BT + j;
                        return (gi >= gj && gi < Ct) ? x * dpow(l2, (float)(gi - gj)) : 0.f;
                    });
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni)) gemm<T, BT>(acc[k], S_s, PT, mi * 32, X_s, PT, ni * 32);
            }
        }
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni))
                store_rows(acc[k], (T *)p.dQ + (rb + (int64_t)qb * BT) * D, D, mi * 32, ni * 32,
                           nvq);
        }
    }

    // ---- phase B: dV ----
    const float droff = dpow(l2, (float)roff);
    const T *Rloc = has_local ? (const T *)p.Rc + cidx : nullptr;
    __syncthreads();
    combine_state<T, D>(St_s, PD, p.Rseg + sidx, Rloc, droff, false);   // R^T [dv][dk]
    for (int kb = 0; kb < nb; ++kb) {
        const int nvk = min(BT, Ct - kb * BT);
        __syncthreads();
        stage_rows<T, BT, D>(B_s, PD, K + (int64_t)kb * BT * D, nvk);
        __syncthreads();
        f32x16 acc[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            zero(acc[k]);
            int mi, ni;
            if (TO::get(k, mi, ni)) {
                gemm<T, D>(acc[k], B_s, PD, mi * 32, St_s, PD, ni * 32);   // K_t R_t
#pragma unroll
                for (int r = 0; r < 16; ++r)                                // Gam_t rows
                    acc[k][r] *= dpow(l2, (float)(Ct - 1 - (kb * BT + mi * 32 + crow(r))));
            }
        }
        for (int qb = kb; qb < nb; ++qb) {
            const int nvq = min(BT, Ct - qb * BT);
            __syncthreads();
            stage_rows<T, BT, D>(A_s, PD, Q + (int64_t)qb * BT * D, nvq);
            stage_rows_T<T, BT, D>(X_s, PT, dO + (int64_t)qb * BT * D, nvq, One());
            __syncthreads();
            {   // S tiles (queries x keys) = Q K^T, stored transposed: [key][query]
                for (int k = 0; k < TS::PER_WAVE; ++k) {
                    int mi, ni;
                    if (!TS::get(k, mi, ni)) continue;
                    f32x16 st;
                    zero(st);
                    gemm<T, D>(st, A_s, PD, mi * 32, B_s, PD, ni * 32);
                    store_T(st, S_s, PT, mi * 32, ni * 32, [&](float x, int i, int j) {
                        const int gi = qb * BT + i, gj = kb * BT + j;
                        return (gi >= gj && gi < Ct) ? x * dpow(l2, (float)(gi - gj)) : 0.f;
                    });
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni)) gemm<T, BT>(acc[k], S_s, PT, mi * 32, X_s, PT, ni * 32);
            }
        }
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni))
                store_rows(acc[k], (T *)p.dV + (rb + (int64_t)kb * BT) * D, D, mi * 32, ni * 32,
                           nvk);
        }
    }

    // ---- phase C: dK ----
    __syncthreads();
    combine_state<T, D>(St_s, PD, p.Rseg + sidx, Rloc, droff, true);    // R [dk][dv]
    for (int kb = 0; kb < nb; ++kb) {
        const int nvk = min(BT, Ct - kb * BT);
        __syncthreads();
        stage_rows<T, BT, D>(B_s, PD, Vg + (int64_t)kb * BT * D, nvk);
        __syncthreads();
        f32x16 acc[TO::PER_WAVE];
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            zero(acc[k]);
            int mi, ni;
            if (TO::get(k, mi, ni)) {
                gemm<T, D>(acc[k], B_s, PD, mi * 32, St_s, PD, ni * 32);   // V_t R_t^T
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[k][r] *= dpow(l2, (float)(Ct - 1 - (kb * BT + mi * 32 + crow(r))));
            }
        }
        for (int qb = kb; qb < nb; ++qb) {
            const int nvq = min(BT, Ct - qb * BT);
            __syncthreads();
            stage_rows<T, BT, D>(A_s, PD, dO + (int64_t)qb * BT * D, nvq);
            stage_rows_T<T, BT, D>(X_s, PT, Q + (int64_t)qb * BT * D, nvq, One());
            __syncthreads();
            {   // E tiles (queries x keys) = dO V^T, stored transposed: [key][query]
                for (int k = 0; k < TS::PER_WAVE; ++k) {
                    int mi, ni;
                    if (!TS::get(k, mi, ni)) continue;
                    f32x16 et;
                    zero(et);
                    gemm<T, D>(et, A_s, PD, mi * 32, B_s, PD, ni * 32);
                    store_T(et, S_s, PT, mi * 32, ni * 32, [&](float x, int i, int j) {
                        const int gi = qb * BT + i, gj = kb * BT + j;
                        return (gi >= gj && gi < Ct) ? x * dpow(l2, (float)(gi - gj)) : 0.f;
                    });
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TO::PER_WAVE; ++k) {
                int mi, ni;
                if (TO::get(k, mi, ni)) gemm<T, BT>(acc[k], S_s, PT, mi * 32, X_s, PT, ni * 32);
            }
        }
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (TO::get(k, mi, ni))
                store_rows(acc[k], (T *)p.dK + (rb + (int64_t)kb * BT) * D, D, mi * 32, ni * 32,
                           nvk);
        }
    }
}

// ===========================================================================
// bf16 path for gfx950.  Operand tiles are staged row-major (16-byte copies);
// operands whose contraction index is the token index are read with the LDS
// transpose read (ds_read_b64_tr_b16), so no transposed copies are made.
// Score tiles stay in registers: the 32x32 accumulator of S^T (tokens c x
// rows r) is, lane for lane, the A operand of S.Cv once its k order is
// permuted, and the Cv operand is read in the same permuted order.
// ===========================================================================
// global -> LDS copy of 16 bytes per lane (lane l's bytes land at dst + 16*l).
// Issued from inline assembly on purpose: the compiler then does not track the
// copy as a pending LDS write, and so does not wait for it before LDS reads it
// cannot prove disjoint (it cannot for the transpose reads).  The caller waits
// (vmcnt) and synchronizes before reading the destination, like for any
// asynchronous copy.  M0 holds the LDS address; the kernels that use this
// leave M0 to these copies alone.  lds: the destination's LDS byte address
// (the same on every lane), formed from lds_addr of a shared array plus an
// offset, so that it stays a 32-bit scalar: a generic pointer into LDS would
// be held in two VGPRs and converted back (with its null check) per copy.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is clobbered on purpose
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

// LDS byte address of a shared array (a constant once the kernel is laid out).
__device__ __forceinline__ uint32_t lds_addr(const bf16 *a) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)a;
}

// s_waitcnt: vmcnt(vm), no wait on the other counters.
#define LASP_WAIT_VM(vm) __builtin_amdgcn_s_waitcnt(((vm) & 15) | (((vm) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier for LDS traffic only.  A release fence would also wait for
// every outstanding global->LDS copy (they count in vmcnt), draining the
// prefetch ring; instead each wave drains its own LDS operations (lgkmcnt) and,
// before calling this, waits (vmcnt) for exactly the copies whose data the
// workgroup reads next.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N> struct IC { static constexpr int value = N; };

// Rows out of a 32-row output tile accumulated transposed: acc[nt] holds
// [feature nt*32 + crow(e)][row lane%32], i.e. each lane holds 4-feature
// pieces of one row.  Lanes l and l+32 exchange halves (permlane32 swap) so
// that each lane holds two 8-feature pieces of its row: lanes < 32 features
// 0-7 and 16-23 of a 32-feature block, lanes >= 32 features 8-15 and 24-31.
// A second exchange between neighbouring 16-lane rows (permlane16 swap: the
// odd rows of the first operand with the even rows of the second) gathers,
// in the first register group, the four 16-byte pieces of the block for rows
// 0-15 and, in the second, those of rows 16-31: lane l then writes row l%16
// (+16) at byte 16 * (2 (l/16 % 2) + l/32) of the block, so that each 16-byte
// store covers 16 rows x 64 contiguous bytes rather than 32 rows x 32.  The
// stores go through a buffer descriptor that covers exactly the tile's `rows`
// valid rows (none when rows <= 0): the hardware drops stores past its end,
// so every wave issues the same NDT*2 stores and the count of memory
// operations in flight after them is known.  neg = 0x80008000 flips the sign
// of every packed bf16 pair.
template <int D>
__device__ __forceinline__ void store_tile_t(const f32x16 *acc, bf16 *tile, int rows, int lz, unsigned neg) {
    constexpr int NDT = D / 32;
    const __amdgpu_buffer_rsrc_t rs = wave_buffer(tile, rows > 0 ? rows * D * 2 : 0);
    const int g = lz >> 4;
    const int off = (lz & 15) * D * 2 + 16 * ((g & 1) * 2 + (g >> 1));
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
        unsigned r[8];   // r[2j], r[2j+1]: features 8j + 4*(lane/32) + [0,4), packed
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bf16x2_t v = {(__bf16)acc[nt][2 * q], (__bf16)acc[nt][2 * q + 1]};
            r[q] = __builtin_bit_cast(unsigned, v) ^ neg;
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
        // r[0..3]: features 0-7 (lanes < 32) or 8-15; r[4..7]: 16-23 or 24-31
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto x = __builtin_amdgcn_permlane16_swap(r[e], r[4 + e], false, false);
            r[e] = x[0];
            r[4 + e] = x[1];
        }
        const u32x4_t v0 = {r[0], r[1], r[2], r[3]}, v1 = {r[4], r[5], r[6], r[7]};
        __builtin_amdgcn_raw_buffer_store_b128(v0, rs, off + nt * 64, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v1, rs, off + 16 * D * 2 + nt * 64, 0, 0);
    }
}

// Norm of LASP Eq. 2 on the rows of a 32-row output tile accumulated
// transposed (acc[nt] = [feature nt*32 + crow(e)][row lane%32]): lanes l and
// l^32 hold the two halves of row l%32's features, so the row's sum of squares
// is the lane's own sum plus its partner's.  Every acc element is scaled by
// r = 1/sqrt(mean(o^2) + eps); lanes < 32 write r for their row (rows below
// `rows` only).
template <int D>
__device__ __forceinline__ void norm_rows(f32x16 *acc, float *rstd, int rows, int lz) {
    constexpr int NDT = D / 32;
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss += acc[nt][e] * acc[nt][e];
    ss += __shfl_xor(ss, 32);
    const float r = rsqrtf(ss * (1.f / D) + kNormEps);
#pragma unroll
    for (int nt = 0; nt < NDT; ++nt) acc[nt] *= r;
    if (lz < 32 && lz < rows) rstd[lz] = r;
}

// ---------------------------------------------------------------------------
// Segment sweep (bf16).  One workgroup per (segment, head, role) walks the
// segment's chunks in sweep order (forward for O and dQ, backward for dV and
// dK), carrying the d x d state in float32 accumulators spread over the waves
// and a bf16 copy in LDS for the inter-chunk product:
//   forward roles:  P <- lambda^Ct P + (Gam_t K_t)^T V_t   (LASP Eq. 10)
//   backward roles: R <- lambda^Ct R + (Lam_t Q_t)^T dO_t  (LASP Eq. 20)
// The state update reads the same token tiles as the intra-chunk product, so
// no per-chunk state is ever written to memory.
//
// Roles.  O, dQ, dV and dK are one computation.  For the rows r of one chunk
// (length Ct) and the state X carried into it ([dv][dk] in memory):
//   Out[r] = sum_{c in causal range of r} lambda^|r-c| (A_r . B_c) Cv_c
//            + lambda^e(r) A_r X
//   0  O  : A=Q,  B=K,  Cv=V,  X=P,   c <= r, e = r+1        (LASP Eqs. 7, 9, 11)
//   1  dQ : A=dO, B=V,  Cv=K,  X=P^T, c <= r, e = r+1        (LASP Eqs. 14-16)
//   2  dV : A=K,  B=Q,  Cv=dO, X=R,   c >= r, e = Ct-1-r     (LASP Eqs. 21-22)
//   3  dK : A=V,  B=dO, Cv=Q,  X=R^T, c >= r, e = Ct-1-r     (LASP Eqs. 17-19)
// Roles 0 and 1 carry P forward, roles 2 and 3 carry R backward; the state
// update takes its token rows from B (roles 0, 2) or from Cv (roles 1, 3).
//
// dQ of a head without decay walks backwards too, so that the three gradient
// roles of a segment read the same chunks at the same time (one HBM read of
// Q, K, V, dO, shared in L2).  With lambda = 1 the state before chunk t is the
// state after it minus the chunk's own term, P_t = P_(t+1) - K_t^T V_t, hence
//   dQ[r] = dO_r P_(t+1)^T - sum_{c > r} (dO_r . V_c) K_c,
// the role-1 computation with the strict reverse causal range, a state that
// starts at minus the state after the segment (the next segment's entering
// state, or the sequence's final state) and accumulates as usual, and the
// output negated.  (With decay the subtraction would divide by lambda^Ct,
// which is not stable; those heads keep the forward walk.)  The subtraction
// costs precision where P_t is small next to the segment's final state: the
// rounding error of a row is of order 2^-9 |dO_r| |P_(t+1)|.  Callers whose dO
// rows differ widely in size (the normalised form's dO is scaled by 1/rms of
// each output row) set dq_forward: dQ then runs in its own launch and walks
// forwards, as with decay.
//
// Work split.  Wave w owns one 32-row tile of every chunk (its A rows live in
// registers, loaded one chunk ahead) and a fixed share of the 32x32 state
// tiles.  The chunk's B and Cv rows are all resident in LDS, so the waves run
// through the chunk's 32-token tiles without a barrier per tile.  The tiles
// are taken in two groups, the outer ones ({0,1,6,7} of 8) and the inner ones,
// which give every SIMD (two waves with row tiles s and 7-s) the same amount
// of causal work in each group.  One barrier separates the groups: after it
// the first group's LDS slots are refilled with the next chunk, and after the
// chunk-start barrier the second group's.  The output is accumulated
// transposed (features x rows), so each lane holds whole 4-feature pieces of
// one row and stores them directly.
// ---------------------------------------------------------------------------
template <int C> struct SweepCfg {
    static constexpr int NCT = C / 32;                 // token tiles per chunk
    static constexpr int NW = NCT < 4 ? 4 : NCT;       // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int NG = NCT / 2;                 // tiles per group
    // waves w and w+4 share a SIMD; pair row tiles s and 7-s on SIMD s
    __device__ static int tile(int w) {
        return NCT == 8 ? (w < 4 ? w : 11 - w) : (w < NCT ? w : -1);
    }
    // k-th tile of group g: 8 tiles {0,1,6,7},{2,3,4,5}; 4 tiles {0,3},{1,2}; 2 tiles {0},{1}
    __device__ static int group_tile(int g, int k) {
        if (NCT == 2) return g;
        constexpr int q = NCT / 4;
        return g == 0 ? (k < q ? k : NCT - 2 * q + k) : q + k;
    }
};

// f[e] *= b lambda^e (up) or b lambda^(7-e): the decay weights of 8
// consecutive tokens from the weight b of the first (up) or last of them, by
// successive products (the factors are at most 1, so no overflow).
__device__ __forceinline__ void geo8(float *f, float b, float lam, bool up) {
    if (up) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { f[e] *= b; b *= lam; }
    } else {
#pragma unroll
        for (int e = 7; e >= 0; --e) { f[e] *= b; b *= lam; }
    }
}

// The same over the 16 elements of a lane's 32x32 MFMA result tile, which sit
// at offsets 8 (e >> 2) + (e & 3) along the tile's rows: s[e] *= b lambda^k(e),
// k(e) = that offset (up), or 27 minus it.
__device__ __forceinline__ void geo16(f32x16 &s, float b, float lam, bool up) {
    const float lam4 = (lam * lam) * (lam * lam);
    if (up) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { s[4 * g + i] *= b; b *= lam; }
            b *= lam4;
        }
    } else {
#pragma unroll
        for (int g = 3; g >= 0; --g) {
#pragma unroll
            for (int i = 3; i >= 0; --i) { s[4 * g + i] *= b; b *= lam; }
            b *= lam4;
        }
    }
}

// What one launch computes:
enum SweepKind {
    SWEEP_OUT = 0,     // role 0 (O)
    SWEEP_GRADS = 1,   // roles 1-3 (dQ, dV, dK), neighbours in launch order so
                       // that the roles of one segment run at the same time and
                       // share their reads of Q, K, V, dO in L2
    // With decay the dQ role walks forwards while dV and dK walk backwards,
    // at other speeds: in one launch the three drift apart and share nothing.
    // Such calls launch dV and dK together (each workgroup's body compiled
    // with its role fixed, so registers are sized per role), then dQ alone.
    // At C = 64 the two-role kernel spills SGPRs, so there dV and dK run as
    // single-role launches and read Q and dO each.
    SWEEP_DQ = 2,       // role 1
    SWEEP_DV = 3,       // role 2
    SWEEP_OUT_NORM = 4, // role 0, rows normalised (Norm of LASP Eq. 2) in the store
    SWEEP_DK = 5,       // role 3
    SWEEP_DVDK = 6      // roles 2 and 3 (dV, dK), neighbours in launch order: both
                        // walk backwards at one speed and share their reads of
                        // Q and dO in L2
};
// The role of a sweep workgroup: fixed at compile time, or the launch's
// first role plus the workgroup's index within the launch's roles.
template <int R> struct FixedRole {
    __device__ constexpr int operator()(int) const { return R; }
};
struct RoleOf {
    int first;
    __device__ int operator()(int sel) const { return first + sel; }
};
// DEC = false: the call has no decay array (every lambda is 1); the decay
// arithmetic is compiled out.
template <int D, int C, int KIND, bool DEC>
__global__ __launch_bounds__(SweepCfg<C>::NT) void k_sweep_bf16(Params p) {
    constexpr int role0 = KIND == SWEEP_GRADS || KIND == SWEEP_DQ ? 1
                          : KIND == SWEEP_DV || KIND == SWEEP_DVDK ? 2 : KIND == SWEEP_DK ? 3 : 0;   // OUT, OUT_NORM: 0
    constexpr int nroles = KIND == SWEEP_GRADS ? 3 : KIND == SWEEP_DVDK ? 2 : 1;
    using Cfg = SweepCfg<C>;
    constexpr int NCT = Cfg::NCT, NW = Cfg::NW, NG = Cfg::NG;
    constexpr int PR = D / 8, KS = D / 16, NDT = D / 32;
    constexpr int TILE = 32 * D;                       // elements of one 32-token operand tile
    constexpr int CPT = TILE / 512;                    // wave copies per operand tile
    constexpr int NIG = NG * 2 * CPT;                  // wave copies per group (B and Cv)
    constexpr int CPW = (NIG + NW - 1) / NW;           // copies per wave per group (at most)
    constexpr int NSTT = NDT * NDT;                    // 32x32 state tiles
    constexpr int STW = (NSTT + NW - 1) / NW;
    __shared__ __attribute__((aligned(16))) bf16 XS[D * D];
    // B and Cv tiles of the two groups.  Two distinct arrays: the compiler
    // then sees that copies in flight into one group's slots do not alias
    // reads of the other's, and does not wait for them.
    __shared__ __attribute__((aligned(16))) bf16 BG0[NG * 2 * TILE];
    __shared__ __attribute__((aligned(16))) bf16 BG1[NG * 2 * TILE];

    const uint32_t bg0_l = lds_addr(BG0), bg1_l = lds_addr(BG1);
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rsel = lid % nroles;
    const int rest = lid / nroles;
    // The body, with the role a compile-time constant (FixedRole) for the
    // gradient kinds (once per role in the three-role launch, which then gets
    // registers sized for each role's own code).
    auto body = [&](auto RS) __attribute__((always_inline)) {
    const int role = RS(rsel);
    const int h = rest % p.H, gs = rest / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    const int nch = t1 - t0;
    if (nch <= 0) return;
    const float l2 = DEC ? head_log2_decay(p, h) : 0.f;
    const bool decay = DEC && l2 != 0.f;
    // The walk ends at the sequence's end (the output walk of its last
    // segment, the dV walk of its first): with end_by_sweep it carries the
    // state through its last chunk as well and writes the end state, whose
    // segment total is then skipped.
    // fin_ih: that sequence's (sequence, head) index, else -1 (one scalar kept
    // across the walk).
    const int nS = min(s.S, p.n_segs_ub - s.s0);
    const int fin_ih = (role == 0 && sl == nS - 1 && fwd_end_by_sweep(p, s, nS)) ||
                               (role == 2 && sl == 0 && bwd_end_by_sweep(p, s, nS))
                           ? s.i * p.H + h : -1;
    // dQ by subtraction, walked backwards, for heads without decay; the
    // separate dQ launch serves calls with a decay array (its heads with
    // lambda = 1 still subtract, so that an all-ones array gives the bits of
    // no array) and calls with dq_forward (never subtracts)
    const bool sub = role == 1 && !decay && (KIND == SWEEP_GRADS || !p.dq_forward);
    const bool rev = role >= 2 || sub;         // chunks swept backwards
    const int dmin = sub ? 1 : 0;              // causal range: dist(r, c) >= dmin
    const bool xt = role & 1;                  // the role uses X^T: state tiles accumulated transposed
    const bool u_is_b = !(role & 1);           // state rows from B (else from Cv)
    const int64_t rbase = row_base(p, s, h);
    const bf16 *Qg = (const bf16 *)p.Q + rbase * D, *Kg = (const bf16 *)p.K + rbase * D;
    const bf16 *Vg = (const bf16 *)p.V + rbase * D;
    const bf16 *Og = role ? (const bf16 *)p.dO + rbase * D : nullptr;
    const bf16 *A, *Bm, *Cv;
    bf16 *Out;
    switch (role) {
    case 0: A = Qg; Bm = Kg; Cv = Vg; Out = (bf16 *)p.O + rbase * D; break;
    case 1: A = Og; Bm = Vg; Cv = Kg; Out = (bf16 *)p.dQ + rbase * D; break;
    case 2: A = Kg; Bm = Qg; Cv = Og; Out = (bf16 *)p.dV + rbase * D; break;
    default: A = Vg; Bm = Og; Cv = Qg; Out = (bf16 *)p.dK + rbase * D; break;
    }
    const int64_t seg_off = ((int64_t)(s.s0 + sl) * p.H + h) * D * D;
    const float *seg = role >= 2 ? p.Rseg + seg_off : p.Pseg + seg_off;
    if (sub)   // the state after this segment
        seg = sl + 1 < nS ? seg + (int64_t)p.H * D * D
                                                    : p.Pfin + ((int64_t)s.i * p.H + h) * D * D;
    const float sgn = sub ? -1.f : 1.f;
    const float lam = dpow(l2, 1.f);

    const int w = wave_id(), l = lane_id();
    const int rt = Cfg::tile(w);
    // The lane index is made opaque at each use site so that lane-derived
    // addresses are recomputed where they are used instead of being hoisted
    // out of the loops, where they would pin many registers.
    auto opaque_lane = [&]() __attribute__((always_inline)) {
        int lz = l;
        asm volatile("" : "+v"(lz));
        return lz;
    };
    const FragOffs<D> fo0 = frag_offs<D>(l);
    auto chunk_t = [&](int i) __attribute__((always_inline)) { return rev ? t1 - 1 - i : t0 + i; };
    auto chunk_len = [&](int t) __attribute__((always_inline)) { return min(p.C, s.len - t * p.C); };

    // group g of chunk i: 32-token tiles of B and Cv (swizzled rows) into their slots
    auto dma_group = [&](int i, auto G) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value;
        const uint32_t bg = g == 0 ? bg0_l : bg1_l;
        const int lz = opaque_lane();
        const int t = chunk_t(i);
        const int tok = t * p.C, Ct = chunk_len(t);
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            const int jj = w + k * NW;
            if (NIG % NW == 0 || jj < NIG) {
                const int ti = jj / (2 * CPT), half = (jj / CPT) & 1, pc0 = jj % CPT;
                const int ct = Cfg::group_tile(g, ti);
                const int slot = pc0 * 64 + lz;
                const int r = slot / PR, pc = (slot % PR) ^ sw_key<D>(r);
                const int row = tok + min(ct * 32 + r, Ct - 1);   // rows past Ct: a valid row
                const bf16 *src = (half ? Cv : Bm) + (int64_t)row * D + pc * 8;
                dma16(src, bg + 2u * (uint32_t)(ti * 2 * TILE + half * TILE + pc0 * 512));
            }
        }
    };
    // chunk i's A rows of this wave's row tile, as MFMA operand fragments
    auto load_a = [&](int i, bf16x8_t *dst) __attribute__((always_inline)) {
        if (rt >= 0) {
            const int lz = opaque_lane();
            const int t = chunk_t(i);
            const int row = t * p.C + min(rt * 32 + (lz & 31), chunk_len(t) - 1);
            const bf16 *src = A + (int64_t)row * D + (lz >> 5) * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) dst[ks] = *(const bf16x8_t *)(src + ks * 16);
        }
    };

    // ---- prologue: first chunk's A rows and first group, incoming state ----
    bf16x8_t af[KS];
    dma_group(0, IC<0>());
    load_a(0, af);

    f32x16 sacc[STW];
#pragma unroll
    for (int k = 0; k < STW; ++k) {
        const int tl = w + k * NW;
        zero(sacc[k]);
        if (tl < NSTT) {
            const int mi = tl / NDT, ni = tl % NDT, lc = l & 31, lg = l >> 5;
            if (xt) {   // transposed tile: rows W features, lanes U features
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sacc[k][e] = sgn * seg[(int64_t)(ni * 32 + crow(e, l)) * D + mi * 32 + lc];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *(const float4 *)(seg + (int64_t)(ni * 32 + lc) * D + mi * 32 + q * 8 + lg * 4);
                    sacc[k][q * 4 + 0] = sgn * v.x; sacc[k][q * 4 + 1] = sgn * v.y;
                    sacc[k][q * 4 + 2] = sgn * v.z; sacc[k][q * 4 + 3] = sgn * v.w;
                }
            }
        }
    }
    // XS = bf16(state) as the inter-chunk product's row operand: [W feature][U
    // feature] (the state's memory layout), or its transpose for the roles that
    // use X^T (their state tiles are accumulated transposed, so the same lane
    // pattern writes the transpose)
    auto write_state = [&]() __attribute__((always_inline)) {
        const int lz = opaque_lane();
        const int lc = lz & 31, lg = lz >> 5;
#pragma unroll
        for (int k = 0; k < STW; ++k) {
            const int tl = w + k * NW;
            if (tl < NSTT) {
                const int rb = xt ? tl / NDT : tl % NDT, cb = xt ? tl % NDT : tl / NDT;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    store4(XS + sw_off<D>(rb * 32 + lc, cb * 32 + q * 8 + lg * 4), sacc[k][q * 4 + 0],
                           sacc[k][q * 4 + 1], sacc[k][q * 4 + 2], sacc[k][q * 4 + 3]);
            }
        }
    };
    write_state();

    // acc[nt]: output tile transposed, [feature nt*32 + crow(e)][row rt*32 + lane%32]
    f32x16 acc[NDT];

    // pair products of row tile rt with NP column tiles ct[] (in range,
    // causal) whose B and Cv rows are at Bt[]; the NP score tiles are
    // independent MFMA chains until they meet in acc
    auto pair = [&](auto NPC, const bf16 *const *Bt, const int *ct, int Ct, auto after_scores)
                    __attribute__((always_inline)) {
        constexpr int NP = decltype(NPC)::value;
        const FragOffs<D> fo = opaque(fo0);
        const int lz = opaque_lane();
        const int lc = lz & 31;
        f32x16 st[NP];                 // S^T: [column token ct*32 + crow(e)][row rt*32 + lane%32]
#pragma unroll
        for (int u = 0; u < NP; ++u) zero(st[u]);
        // The B fragments of k-step ks+BPD are read while the MFMAs of step ks
        // run (scheduling barriers keep the compiler from serializing each
        // read with its MFMA to save registers).
        constexpr int BPD = 1;
        bf16x8_t bf[BPD + 1][NP];
#pragma unroll
        for (int ks = 0; ks < BPD; ++ks)
#pragma unroll
            for (int u = 0; u < NP; ++u) bf[ks][u] = frag_rows_sw<D>(Bt[u], fo, 0, ks * 16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks + BPD < KS) {
#pragma unroll
                for (int u = 0; u < NP; ++u)
                    bf[(ks + BPD) % (BPD + 1)][u] = frag_rows_sw<D>(Bt[u], fo, 0, (ks + BPD) * 16);
            }
#pragma unroll
            for (int u = 0; u < NP; ++u) mma(st[u], bf[ks % (BPD + 1)][u], af[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
        after_scores();   // af has been read
        // S^T Cv: NJ MFMAs, each with its own Cv fragment (two transpose
        // reads); the fragments are read CPD MFMAs ahead of their use, the
        // first ones while the score tiles are masked and converted.
        constexpr int NJ = NDT * NP * 2, CPD = 4;
        // (MFMA j: feature tile j % NDT, score tile and half q = j / NDT, so
        // that consecutive MFMAs accumulate into different tiles)
        auto cv_frag = [&](int j) __attribute__((always_inline)) {
            const int nt = j / (NP * 2), u = (j >> 1) % NP, kh = j & 1;
            return frag_cols_sw<D, true>(Bt[u] + TILE, fo, kh * 16, nt * 32);
        };
        bf16x8_t cf[CPD];
#pragma unroll
        for (int j = 0; j < CPD; ++j) cf[j] = cv_frag(j);
        bf16x8_t s0[NP], s1[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            if (ct[u] == rt || (ct[u] + 1) * 32 > Ct) {
                const int r = rt * 32 + lc;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int c = ct[u] * 32 + crow(e, lz);
                    const int dist = rev ? (c - r) : (r - c);
                    const float f = decay ? dpow(l2, (float)max(dist, 0)) : 1.f;
                    st[u][e] = (dist >= dmin && c < Ct) ? st[u][e] * f : 0.f;
                }
            } else if (decay) {
                // off-diagonal tile inside the chunk: every distance is
                // positive; one power for the lane's nearest column
                const int r = rt * 32 + lc, c0 = ct[u] * 32 + crow(0, lz);
                geo16(st[u], dpow(l2, (float)(rev ? c0 - r : r - c0 - 27)), lam, rev);
            }
            // as an operand, S^T's k order is permuted; the Cv fragment follows it
            s0[u] = pack8(st[u][0], st[u][1], st[u][2], st[u][3], st[u][4], st[u][5], st[u][6], st[u][7]);
            s1[u] = pack8(st[u][8], st[u][9], st[u][10], st[u][11], st[u][12], st[u][13], st[u][14],
                          st[u][15]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const int nt = j / (NP * 2), u = (j >> 1) % NP;
            mma(acc[nt], cf[j % CPD], (j & 1) ? s1[u] : s0[u]);
            if (j + CPD < NJ) cf[j % CPD] = cv_frag(j + CPD);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // state += U^T (scaled W) over the tokens of the group's column tiles.
    // Steps (column tile, 16-token half): the W fragment is shared by the
    // wave's state tiles (they have the same column block ni), each tile reads
    // its own U fragment; the fragments of step j+1 are read while the MFMAs
    // of step j run.  The token weights (lambda^(Ct-1-tk), or lambda^(tk+1)
    // when walking backwards) go on the shared W fragment, the token index
    // being the contraction index: one power per fragment times the per-lane
    // successive factors lambda (geo8).  Tokens past the chunk end are masked to zero there
    // (their LDS slots hold clamped, valid rows).
    static_assert(NW % NDT == 0, "state tiles of one wave must share their column block");
    auto state_updates = [&](const bf16 *BG, auto G, int Ct, auto XTC) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value;
        constexpr bool XT = decltype(XTC)::value;   // accumulate the tiles transposed
        constexpr int NSU = NG * 2;
        const FragOffs<D> fo = opaque(fo0);
        const int lz = opaque_lane();
        const int lg = lz >> 5;
        const int ni = w % NDT;
        bf16x8_t wf[2], uf[2][STW];
        auto fetch = [&](int j, bf16x8_t &wd, bf16x8_t *ud) __attribute__((always_inline)) {
            const bf16 *Bt = BG + (j >> 1) * 2 * TILE;
            const bf16 *Ut = Bt + (u_is_b ? 0 : TILE), *Wt = Bt + (u_is_b ? TILE : 0);
            const int kk = j & 1;
            wd = frag_cols_sw<D, false>(Wt, fo, kk * 16, ni * 32);
#pragma unroll
            for (int k = 0; k < STW; ++k)
                if (w + k * NW < NSTT) ud[k] = frag_cols_sw<D, false>(Ut, fo, kk * 16, ((w + k * NW) / NDT) * 32);
        };
        fetch(0, wf[0], uf[0]);
#pragma unroll
        for (int j = 0; j < NSU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < NSU) fetch(j + 1, wf[(j + 1) & 1], uf[(j + 1) & 1]);
            const int ct = Cfg::group_tile(g, j >> 1), kk = j & 1;
            const bool scale = decay || (ct + 1) * 32 > Ct;
            bf16x8_t wa = wf[j & 1];
            if (scale) {
                float f[8];
                load16((const bf16 *)&wa, f);
                const int tk0 = ct * 32 + kk * 16 + lg * 8;
                if (tk0 + 7 < Ct) {   // the 8 tokens are in the chunk
                    if (decay) geo8(f, dpow(l2, (float)(rev ? tk0 + 1 : Ct - 1 - (tk0 + 7))), lam, rev);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tk = tk0 + e;
                        const float sc = decay ? dpow(l2, (float)max(rev ? tk + 1 : Ct - 1 - tk, 0)) : 1.f;
                        f[e] = tk < Ct ? f[e] * sc : 0.f;
                    }
                }
                wa = pack8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
            }
#pragma unroll
            for (int k = 0; k < STW; ++k) {
                if (w + k * NW < NSTT) {
                    if (XT)
                        mma(sacc[k], wa, uf[j & 1][k]);
                    else
                        mma(sacc[k], uf[j & 1][k], wa);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // one group of column tiles: pair products, then the state updates.
    // after_a() runs once the pair products have read af: right after the
    // score products of the group's last pair (its S^T Cv products and the
    // state updates then hide the latency), or at once without pairs
    auto run_group = [&](auto G, int Ct, bool upd, auto after_a) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value;
        const bf16 *BG = g == 0 ? BG0 : BG1;
        bool a_done = false;
        if (rt >= 0 && rt * 32 < Ct) {
            // the group's causal tiles, two at a time
            int need = 0;
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                const int ct = Cfg::group_tile(g, k);
                if (ct * 32 < Ct && (ct == rt || (rev ? ct > rt : ct < rt))) need |= 1 << k;
            }
#pragma unroll 1
            while (need) {
                const int ka = __builtin_ctz(need);
                need &= need - 1;
                if (need) {
                    const int kb = __builtin_ctz(need);
                    need &= need - 1;
                    const bf16 *bt[2] = {BG + ka * 2 * TILE, BG + kb * 2 * TILE};
                    const int cts[2] = {Cfg::group_tile(g, ka), Cfg::group_tile(g, kb)};
                    const bool last = need == 0;
                    pair(IC<2>(), bt, cts, Ct, [&]() __attribute__((always_inline)) {
                        if (last) { after_a(); a_done = true; }
                    });
                } else {
                    const bf16 *bt[1] = {BG + ka * 2 * TILE};
                    const int cts[1] = {Cfg::group_tile(g, ka)};
                    pair(IC<1>(), bt, cts, Ct, [&]() __attribute__((always_inline)) {
                        after_a();
                        a_done = true;
                    });
                }
            }
        }
        if (!a_done) after_a();
        if (upd) {
            if (xt)
                state_updates(BG, G, Ct, IC<1>());
            else
                state_updates(BG, G, Ct, IC<0>());
        }
    };

#pragma unroll 1
    for (int i = 0; i < nch; ++i) {
        const int t = chunk_t(i), Ct = chunk_len(t);
        // (the state after the segment's last chunk is needed only at the
        // sequence's end; the other segment totals come from their own kernel)
        const bool upd = i + 1 < nch || fin_ih >= 0;
        // chunk start: this chunk's first group and A rows have landed (only the
        // previous chunk's NDT*2 output stores, issued after them, may still be
        // in flight), every wave has published the state into XS
        if (i > 0)
            LASP_WAIT_VM(NDT * 2);
        else
            LASP_WAIT_VM(0);
        lds_barrier();
        dma_group(i, IC<1>());         // slots of the second group are free now
        // inter-chunk term: acc = (A X)^T, rows scaled by lambda^e(r)
        {
#pragma unroll
            for (int nt = 0; nt < NDT; ++nt) zero(acc[nt]);
            // MFMA j = (k-step j / NDT, feature tile j % NDT): consecutive MFMAs
            // accumulate into different tiles; fragments are read XPD ahead
            // (XS holds the operand in row form for every role: X, or X^T for
            // the roles whose state tiles are accumulated transposed)
            auto inter = [&]() __attribute__((always_inline)) {
                const FragOffs<D> fo = opaque(fo0);
                constexpr int NJ = NDT * KS, XPD = 4;
                auto x_frag = [&](int j) __attribute__((always_inline)) {
                    return frag_rows_sw<D>(XS, fo, (j % NDT) * 32, (j / NDT) * 16);
                };
                bf16x8_t xf[XPD];
#pragma unroll
                for (int j = 0; j < XPD; ++j) xf[j] = x_frag(j);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    __builtin_amdgcn_sched_barrier(0);
                    mma(acc[j % NDT], xf[j % XPD], af[j / NDT]);
                    if (j + XPD < NJ) xf[j % XPD] = x_frag(j + XPD);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            if (rt >= 0 && rt * 32 < Ct) inter();
            const int lz = opaque_lane();
            if (decay && rt >= 0) {
                const int r = rt * 32 + (lz & 31);
                const float sc = dpow(l2, (float)(rev ? (Ct - 1 - r) : (r + 1)));
#pragma unroll
                for (int nt = 0; nt < NDT; ++nt) acc[nt] *= sc;
            }
        }
        if (upd && decay) {
            const float dc = dpow(l2, (float)Ct);
#pragma unroll
            for (int k = 0; k < STW; ++k) sacc[k] *= dc;
        }
        run_group(IC<0>(), Ct, upd, [] {});
        // mid-chunk: the second group has landed; the first group's slots and
        // XS are no longer read by any wave
        LASP_WAIT_VM(0);
        lds_barrier();
        if (i + 1 < nch) dma_group(i + 1, IC<0>());
        // the next chunk's A rows go into af once this chunk's pair products
        // have read it; the state updates and stores hide their latency
        run_group(IC<1>(), Ct, upd, [&]() __attribute__((always_inline)) {
            if (i + 1 < nch) load_a(i + 1, af);
        });
        // rows out (the tile's rows past the chunk end are dropped); the
        // output role normalises its rows first when asked to
        if (KIND == SWEEP_OUT_NORM)
            norm_rows<D>(acc, p.rstd + rbase + (int64_t)t * p.C + rt * 32,
                         rt >= 0 ? Ct - rt * 32 : 0, opaque_lane());
        store_tile_t<D>(acc, Out + ((int64_t)t * p.C + rt * 32) * D, rt >= 0 ? Ct - rt * 32 : 0,
                        opaque_lane(), sub ? 0x80008000u : 0u);
        if (i + 1 < nch) write_state();
    }
    if (fin_ih >= 0) {
        // the end state: P after the sequence's last token (role 0) or R
        // before its first (role 2), as Pfin / Rfin ([dv][dk], the tile
        // layout of the entering state read above) and M_out / dM_in ([dk][dv])
        const int64_t so = (int64_t)fin_ih * D * D;
        float *fs = role == 0 ? p.Pfin : p.Rfin;
        float *api = role == 0 ? p.M_out : p.dM_in;
        const int lz = opaque_lane();
        const int lc = lz & 31, lg = lz >> 5;
#pragma unroll
        for (int k = 0; k < STW; ++k) {
            const int tl = w + k * NW;
            if (tl < NSTT) {
                const int mi = tl / NDT, ni = tl % NDT;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int dk = mi * 32 + q * 8 + lg * 4, dv = ni * 32 + lc;
                    if (fs)
                        *(float4 *)(fs + so + (int64_t)dv * D + dk) =
                            make_float4(sacc[k][q * 4 + 0], sacc[k][q * 4 + 1], sacc[k][q * 4 + 2],
                                        sacc[k][q * 4 + 3]);
                    if (api) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) api[so + (int64_t)(dk + j) * D + dv] = sacc[k][q * 4 + j];
                    }
                }
            }
        }
    }
    };
    if constexpr (KIND == SWEEP_GRADS) {
        if (rsel == 0) body(FixedRole<1>());
        else if (rsel == 1) body(FixedRole<2>());
        else body(FixedRole<3>());
    } else if constexpr (KIND == SWEEP_DVDK) {
        if (rsel == 0) body(FixedRole<2>());
        else body(FixedRole<3>());
    } else if constexpr (KIND == SWEEP_DV || KIND == SWEEP_DK) {
        body(FixedRole<role0>());
    } else {
        body(RoleOf{role0});   // (the output kinds spill less this way)
    }
}


// ---------------------------------------------------------------------------
// Segment totals (bf16): per (segment, head), the state recursion of the
// segment started from zero, which collapses to one weighted contraction over
// the segment's tokens tau = 0 .. L-1:
//   forward  Z = sum_tau lambda^(L-1-tau) k_tau^T v_tau      (LASP-2's M_t, Eq. 10)
//   backward W = sum_tau lambda^(tau+1)   q_tau^T dO_tau     (LASP Eq. 20)
// stored [dv][dk] like the scanned states.  The chunking does not enter, so
// the kernel streams steps of TPS 32-token tiles of U (K or Q) and W (V or dO)
// through a ring of LDS slots, NSLOT-1 steps in flight: the work per tile is
// small and the kernel lives on memory parallelism.  Each wave owns the same
// 32x32 state tiles as in the sweep and accumulates (scaled U)^T W with the
// same fragment reads.
// ---------------------------------------------------------------------------
template <int D> struct SegTotCfg {
    static constexpr int NW = 8, NT = 64 * NW;
    static constexpr int TILE = 32 * D;                            // elements of one 32-token tile
    static constexpr int TPS = 2;                                  // tiles per step (one barrier each)
    static constexpr int SLOT = 2 * TILE * TPS;                    // U tiles, W tiles of one step
    // slots in 160 KiB of LDS at d = 128; in 80 KiB at smaller d, whose
    // segments are short (packed batches): two workgroups then share a CU and
    // one's ring fill overlaps the other's stream (totals -12 % at d = 64)
    static constexpr int NSLOT = ((D == 128 ? 160 : 80) * 1024) / (SLOT * 2);
    static constexpr int CPT = TILE / 512;                         // 1 KiB wave copies per tile
    static constexpr int CPS = 2 * CPT * TPS;                      // copies per slot
    static constexpr int CPW = (CPS + NW - 1) / NW;                // copies per wave per slot (at most)
};

enum TotKind { TOT_F = 0, TOT_B = 1 };   // forward Z, backward W

template <int D, int KIND, bool DEC>
__global__ __launch_bounds__(SegTotCfg<D>::NT) void k_segtot_bf16(Params p) {
    using Cfg = SegTotCfg<D>;
    constexpr int NW = Cfg::NW, TILE = Cfg::TILE, TPS = Cfg::TPS, SLOT = Cfg::SLOT;
    constexpr int NSLOT = Cfg::NSLOT, CPT = Cfg::CPT, CPS = Cfg::CPS, CPW = Cfg::CPW;
    constexpr int PR = D / 8, NDT = D / 32, NSTT = NDT * NDT, STW = (NSTT + NW - 1) / NW;
    constexpr bool BWD = KIND == TOT_B;
    static_assert(NW % NDT == 0, "state tiles of one wave must share their column block");
    // the wait below keeps (NSLOT - 2) slots of copies of this wave in flight
    static_assert((NSLOT - 2) * CPW <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(16))) bf16 ring[NSLOT * SLOT];
    const uint32_t ring_l = lds_addr(ring);

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid % p.H, gs = lid / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    if (t1 <= t0) return;
    {   // a total that the sweeps make unnecessary (they write the end state)
        const int nS = min(s.S, p.n_segs_ub - s.s0);
        if (BWD ? (sl == 0 && bwd_end_by_sweep(p, s, nS))
                : (sl == nS - 1 && fwd_end_by_sweep(p, s, nS)))
            return;
    }
    const int tok0 = t0 * p.C;                                     // first token of the segment
    const int L = min(t1 * p.C, s.len) - tok0;                     // tokens in the segment
    const int nsteps = (L + 32 * TPS - 1) / (32 * TPS);
    const float l2 = DEC ? head_log2_decay(p, h) : 0.f;
    const bool decay = DEC && l2 != 0.f;
    const int64_t rbase = row_base(p, s, h) + tok0;
    const bf16 *U = (const bf16 *)(BWD ? p.Q : p.K) + rbase * D;
    const bf16 *Wm = (const bf16 *)(BWD ? p.dO : p.V) + rbase * D;

    const int w = wave_id(), l = lane_id();
    const FragOffs<D> fo0 = frag_offs<D>(l);
    f32x16 sacc[STW];
#pragma unroll
    for (int k = 0; k < STW; ++k) zero(sacc[k]);
    const float lam = dpow(l2, 1.f);

    // step j: tiles TPS j .. TPS j + TPS - 1 (swizzled rows, rows past L
    // clamped to a valid row) into ring slot j % NSLOT, as [tile][U, W]
    auto issue = [&](int j) __attribute__((always_inline)) {
        int lz = l;
        asm volatile("" : "+v"(lz));
        const uint32_t dst = ring_l + 2u * (uint32_t)((j % NSLOT) * SLOT);
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            const int jj = w + k * NW;
            if (CPS % NW == 0 || jj < CPS) {
                const int q = jj / (2 * CPT), half = (jj / CPT) & 1, pc0 = jj % CPT;
                const int slot = pc0 * 64 + lz;
                const int r = slot / PR, pc = (slot % PR) ^ sw_key<D>(r);
                const int row = min((j * TPS + q) * 32 + r, L - 1);
                dma16((half ? Wm : U) + (int64_t)row * D + pc * 8,
                      dst + 2u * (uint32_t)(q * 2 * TILE + half * TILE + pc0 * 512));
            }
        }
    };
    // state += (scaled U)^T W over 32-token tile tq of the segment, at Ut, Wt
    auto update = [&](const bf16 *Ut, const bf16 *Wt, int tq) __attribute__((always_inline)) {
        const FragOffs<D> fo = opaque(fo0);
        int lz = l;
        asm volatile("" : "+v"(lz));
        const int lg = lz >> 5, ni = w % NDT;
        const bool scale = decay || (tq + 1) * 32 > L;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // the token weights go on the shared W fragment (see the sweep's
            // state updates)
            bf16x8_t wf = frag_cols_sw<D, false>(Wt, fo, kk * 16, ni * 32);
            if (scale) {
                float f[8];
                load16((const bf16 *)&wf, f);
                const int tau0 = tq * 32 + kk * 16 + lg * 8;
                if (tau0 + 7 < L) {
                    if (decay) geo8(f, dpow(l2, (float)(BWD ? tau0 + 1 : L - 1 - (tau0 + 7))), lam, BWD);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tau = tau0 + e;
                        const float sc = decay ? dpow(l2, (float)(BWD ? tau + 1 : L - 1 - tau)) : 1.f;
                        f[e] = tau < L ? f[e] * sc : 0.f;
                    }
                }
                wf = pack8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
            }
#pragma unroll
            for (int k = 0; k < STW; ++k) {
                if (w + k * NW < NSTT)
                    mma(sacc[k], frag_cols_sw<D, false>(Ut, fo, kk * 16, ((w + k * NW) / NDT) * 32), wf);
            }
        }
    };

#pragma unroll 1
    for (int j = 0; j < NSLOT - 1 && j < nsteps; ++j) issue(j);

#pragma unroll 1
    for (int j = 0; j < nsteps; ++j) {
        // step j has landed: this wave's copies of later steps may still be in flight
        if (j + NSLOT - 2 < nsteps)
            LASP_WAIT_VM((NSLOT - 2) * CPW);
        else
            LASP_WAIT_VM(0);
        lds_barrier();
        // every wave is done with step j-1: its slot takes step j + NSLOT - 1
        if (j + NSLOT - 1 < nsteps) issue(j + NSLOT - 1);
        const bf16 *Sl = ring + (j % NSLOT) * SLOT;
#pragma unroll
        for (int q = 0; q < TPS; ++q) update(Sl + q * 2 * TILE, Sl + q * 2 * TILE + TILE, j * TPS + q);
    }

    float *tot = (BWD ? p.W : p.Z) + ((int64_t)(s.s0 + sl) * p.H + h) * D * D;
#pragma unroll
    for (int k = 0; k < STW; ++k) {
        const int tl = w + k * NW;
        if (tl < NSTT) {
            const int mi = tl / NDT, ni = tl % NDT, lc = l & 31, lg = l >> 5;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(float4 *)(tot + (int64_t)(ni * 32 + lc) * D + mi * 32 + q * 8 + lg * 4) =
                    make_float4(sacc[k][q * 4 + 0], sacc[k][q * 4 + 1], sacc[k][q * 4 + 2],
                                sacc[k][q * 4 + 3]);
        }
    }
}


// ---------------------------------------------------------------------------
// Row-block products of the unmasked (bidirectional) form ([LASP] Eq. 3, the
// right-product version; LASP-2's O_t = Q_t M_(1:T)): Out = A X over every row
// of a segment, with one d x d matrix X per (sequence, head):
//   forward  O  = Q  M       (X = M,     the summed state Pfin)
//   backward dQ = dO M^T,  dV = K dM,  dK = V dM^T   (dM: Rfin)
// Pfin and Rfin are [dv][dk]: M[dk][dv] = Pfin[dv][dk].  One workgroup per
// (segment, head, product); it converts X once into a bf16 LDS operand
// XS[n][k] (n output feature, k contracted feature), then its waves take
// 32-row tiles in turn: A rows into registers (the next tile's loaded while
// the current one's MFMAs run), (XS A^T) accumulated transposed as in the
// sweep, rows out through store_tile_t.  A segment's rows are split into
// p.parts contiguous ranges of whole tiles, one workgroup each, so that the
// launch has several workgroups per CU.
// ---------------------------------------------------------------------------
enum RowMatKind { RM_FWD = 0, RM_BWD = 1 };
constexpr int RM_NW = 8;   // waves per workgroup

template <int D, int KIND>
__global__ __launch_bounds__(64 * RM_NW) void k_rowmat_bf16(Params p) {
    constexpr int NW = RM_NW, NDT = D / 32, KS = D / 16;
    constexpr int nprod = KIND == RM_BWD ? 3 : 1;
    __shared__ __attribute__((aligned(16))) bf16 XS[D * D];

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int prod = lid % nprod, rest0 = lid / nprod;
    const int part = rest0 % p.parts, rest = rest0 / p.parts;
    const int h = rest % p.H, gs = rest / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    if (t1 <= t0) return;
    const int seg_rows = min(t1 * p.C, s.len) - t0 * p.C;
    const int tpp = ((seg_rows + 31) / 32 + p.parts - 1) / p.parts;   // tiles per part
    const int row0 = t0 * p.C + part * tpp * 32;               // first row of this part
    const int nrows = min(seg_rows - part * tpp * 32, tpp * 32);
    if (nrows <= 0) return;
    const int64_t rbase = (row_base(p, s, h) + row0) * D;
    const float *X = (KIND == RM_FWD || prod == 0 ? p.Pfin : p.Rfin) + ((int64_t)s.i * p.H + h) * D * D;
    const bool trans = KIND == RM_BWD && prod != 1;            // dQ, dK use the transpose
    const bf16 *A;
    bf16 *Out;
    if (KIND == RM_FWD) {
        A = (const bf16 *)p.Q + rbase; Out = (bf16 *)p.O + rbase;
    } else if (prod == 0) {
        A = (const bf16 *)p.dO + rbase; Out = (bf16 *)p.dQ + rbase;
    } else if (prod == 1) {
        A = (const bf16 *)p.K + rbase; Out = (bf16 *)p.dV + rbase;
    } else {
        A = (const bf16 *)p.V + rbase; Out = (bf16 *)p.dK + rbase;
    }

    // XS[n][k] = bf16(X[n][k]), or bf16(X[k][n]) for the transpose
    for (int c = threadIdx.x; c < D * D / 4; c += NW * 64) {
        int n, k0;
        float f[4];
        if (trans) {   // lanes take consecutive n: coalesced reads of X rows
            n = c % D;
            k0 = (c / D) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) f[j] = X[(int64_t)(k0 + j) * D + n];
        } else {
            n = c / (D / 4);
            k0 = (c % (D / 4)) * 4;
            const float4 v = *(const float4 *)(X + (int64_t)n * D + k0);
            f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
        }
        store4(XS + sw_off<D>(n, k0), f[0], f[1], f[2], f[3]);
    }
    __syncthreads();

    const int w = wave_id(), l = lane_id();
    const FragOffs<D> fo0 = frag_offs<D>(l);
    const int ntiles = (nrows + 31) / 32;
    // A rows of tile `tile` (rows past the segment end: a valid row)
    auto load_rows = [&](int tile, bf16x8_t *dst) __attribute__((always_inline)) {
        int lz = l;
        asm volatile("" : "+v"(lz));
        const int row = min(tile * 32 + (lz & 31), nrows - 1);
        const bf16 *src = A + (int64_t)row * D + (lz >> 5) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dst[ks] = *(const bf16x8_t *)(src + ks * 16);
    };
    // one tile: acc = (XS A^T), the XS fragments read XPD MFMAs ahead, rows out
    auto process = [&](int tile, const bf16x8_t *a) __attribute__((always_inline)) {
        f32x16 acc[NDT];
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) zero(acc[nt]);
        const FragOffs<D> fo = opaque(fo0);
        constexpr int NJ = NDT * KS, XPD = 4;
        bf16x8_t xf[XPD];
#pragma unroll
        for (int j = 0; j < XPD; ++j) xf[j] = frag_rows_sw<D>(XS, fo, (j % NDT) * 32, (j / NDT) * 16);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            mma(acc[j % NDT], xf[j % XPD], a[j / NDT]);
            if (j + XPD < NJ)
                xf[j % XPD] = frag_rows_sw<D>(XS, fo, ((j + XPD) % NDT) * 32, ((j + XPD) / NDT) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
        int lz = l;
        asm volatile("" : "+v"(lz));
        store_tile_t<D>(acc, Out + (int64_t)tile * 32 * D, nrows - tile * 32, lz, 0u);
    };
    // tiles w, w + NW, ... in pairs, each tile's A rows loaded while the one
    // before it is computed (two named buffers: no indexed register arrays)
    bf16x8_t a0[KS], a1[KS];
    if (w < ntiles) load_rows(w, a0);
#pragma unroll 1
    for (int tile = w; tile < ntiles; tile += 2 * NW) {
        if (tile + NW < ntiles) load_rows(tile + NW, a1);
        process(tile, a0);
        if (tile + NW >= ntiles) break;
        if (tile + 2 * NW < ntiles) load_rows(tile + 2 * NW, a0);
        process(tile + NW, a1);
    }
}

// ---------------------------------------------------------------------------
// Row-wise output normalisation (Norm of LASP Sec. 3.1, Eq. 2, read as
// o / sqrt(mean_j o_j^2 + eps) per row of d features), over all B*H*N rows;
// each row is handled by D/VEC lanes (16 bytes each) that reduce by shuffles.
//   forward  (float32 path; the bf16 sweep does this in its store):
//            O <- O r in place, rstd[row] = r
//   backward preparation: dOn = r (dYn - Yn mean(dYn . Yn)), the gradient of
//            the un-normalised output, which the backward then consumes as dO.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void store16(T *dst, const float *f);
template <>
__device__ __forceinline__ void store16<float>(float *dst, const float *f) {
    *(float4 *)dst = make_float4(f[0], f[1], f[2], f[3]);
}
template <>
__device__ __forceinline__ void store16<bf16>(bf16 *dst, const float *f) {
    *(bf16x8_t *)dst = pack8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
}

template <typename T, int D, bool BWD>
__global__ __launch_bounds__(NTHR) void k_rownorm(Params p) {
    constexpr int V = Tr<T>::VEC, LPR = D / V;   // lanes per row (a power of two <= 64)
    const int64_t nrows = (int64_t)p.B * p.H * p.N;
    const int64_t row = ((int64_t)blockIdx.x * NTHR + threadIdx.x) / LPR;
    const int64_t off = row * D + (threadIdx.x % LPR) * V;
    const bool ok = row < nrows;
    float a[V], b[V];
    float s = 0.f;
    if (ok) {
        if (BWD) {
            load16((const T *)p.Yn + off, a);
            load16((const T *)p.dYn + off, b);
#pragma unroll
            for (int e = 0; e < V; ++e) s += a[e] * b[e];
        } else {
            load16((const T *)p.O + off, a);
#pragma unroll
            for (int e = 0; e < V; ++e) s += a[e] * a[e];
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);   // every lane takes part
    if (!ok) return;
    if (BWD) {
        const float r = p.rstd_in[row], mean = s * (1.f / D);
#pragma unroll
        for (int e = 0; e < V; ++e) a[e] = r * (b[e] - a[e] * mean);
        store16((T *)p.dOn + off, a);
    } else {
        const float r = rsqrtf(s * (1.f / D) + kNormEps);
#pragma unroll
        for (int e = 0; e < V; ++e) a[e] *= r;
        store16((T *)p.O + off, a);
        if (threadIdx.x % LPR == 0) p.rstd[row] = r;
    }
}

template <typename T, int D, bool BWD>
static hipError_t rownorm_launch(const Params &p, hipStream_t st) {
    constexpr int LPR = D / Tr<T>::VEC;
    const int64_t threads = (int64_t)p.B * p.H * p.N * LPR;
    if (threads == 0) return hipSuccess;
    return launch_k(k_rownorm<T, D, BWD>, dim3((unsigned)((threads + NTHR - 1) / NTHR)), dim3(NTHR),
                    st, p);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline int round8(int n) { return (n + 7) & ~7; }

// Token block: 64, except float32 with d = 128 where 32 keeps LDS under 160 KB.
template <typename T, int D> struct Block {
    static constexpr int BT = (sizeof(T) == 4 && D == 128) ? 32 : 64;
};

// ---------------------------------------------------------------------------
// Scratch memory of the allocation-free forward entry point: a file-scope
// device array, one copy on every GPU the library runs on (held until the
// process ends).  Host code never passes `scratch` itself to a kernel (its
// host-side name is not a device address): the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept in a small table.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(hipStream_t st, void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    hipDevice_t dev = 0;
    LASP_TRY(hipStreamGetDevice(st, &dev));
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        LASP_TRY(hipGetDevice(&cur));
        if (cur != dev) LASP_TRY(hipSetDevice(dev));
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) LASP_TRY(hipSetDevice(cur));
        LASP_TRY(e);
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_setup(const Params &p, hipStream_t st) {
    return launch_k(k_setup, dim3(1), dim3(NTHR), st, p);
}

template <typename T, int D>
static hipError_t fwd_impl(const Params &p, bool with_output, hipStream_t st, hipEvent_t *ev) {
    constexpr int BT = Block<T, D>::BT;
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY(launch_k(k_fwd_local<T, D, BT>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_fwd_segscan<D, T>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    if (with_output) {
        LASP_TRY(launch_k(k_fwd_out<T, D, BT>, dim3(round8(p.n_chunks_ub * p.H)), dim3(NTHR), st, p));
        if (p.rstd) LASP_TRY((rownorm_launch<T, D, false>(p, st)));
    }
    return rec_event(ev, 3, st);
}

template <typename T, int D>
static hipError_t bwd_impl(const Params &p, hipStream_t st, hipEvent_t *ev) {
    constexpr int BT = Block<T, D>::BT;
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY(launch_k(k_bwd_local<T, D, BT>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_bwd_segscan<D, T>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    LASP_TRY(launch_k(k_bwd_grads<T, D, BT>, dim3(round8(p.n_chunks_ub * p.H)), dim3(NTHR), st, p));
    return rec_event(ev, 3, st);
}

// bf16: segment totals, segment scan, sweep.
template <int D, int C, int KIND>
static hipError_t sweep_launch(const Params &p, hipStream_t st) {
    const int roles = KIND == SWEEP_GRADS ? 3 : 1;
    const dim3 grid(round8(p.n_segs_ub * p.H * roles)), block(SweepCfg<C>::NT);
    if (KIND == SWEEP_OUT && p.rstd) {   // normalised output rows
        if (p.decay) return launch_k(k_sweep_bf16<D, C, SWEEP_OUT_NORM, true>, grid, block, st, p);
        return launch_k(k_sweep_bf16<D, C, SWEEP_OUT_NORM, false>, grid, block, st, p);
    }
    if (p.decay || (KIND == SWEEP_GRADS && p.dq_forward)) {
        if constexpr (KIND == SWEEP_GRADS) {
            if constexpr (C >= 128) {   // dV and dK in one launch (C = 64: it spills SGPRs)
                LASP_TRY(launch_k(k_sweep_bf16<D, C, SWEEP_DVDK, true>,
                                  dim3(round8(p.n_segs_ub * p.H * 2)), block, st, p));
            } else {
                LASP_TRY(launch_k(k_sweep_bf16<D, C, SWEEP_DV, true>, dim3(round8(p.n_segs_ub * p.H)),
                                  block, st, p));
                LASP_TRY(launch_k(k_sweep_bf16<D, C, SWEEP_DK, true>, dim3(round8(p.n_segs_ub * p.H)),
                                  block, st, p));
            }
            return launch_k(k_sweep_bf16<D, C, SWEEP_DQ, true>, dim3(round8(p.n_segs_ub * p.H)), block,
                            st, p);
        } else {
            return launch_k(k_sweep_bf16<D, C, KIND, true>, grid, block, st, p);
        }
    }
    return launch_k(k_sweep_bf16<D, C, KIND, false>, grid, block, st, p);
}

// ---------------------------------------------------------------------------
// Row-block products of the unmasked form in float32: the same products as
// k_rowmat_bf16 (Out = A X over the rows of a segment part, X = the summed
// state Pfin or Rfin, or its transpose), as 32x32x2 f32 MFMAs with both
// operands staged in LDS with the contracted feature contiguous.  Its
// template arguments are those of the float32 causal kernels.
// ---------------------------------------------------------------------------
template <int D, int KIND>
__global__ __launch_bounds__(NTHR) void k_rowmat_f32(Params p) {
    constexpr int BT = (D == 128) ? 32 : 64;        // rows per block
    constexpr int V = Tr<float>::VEC;
    constexpr int PD = D + V;                        // LDS pitch
    constexpr int nprod = KIND == RM_BWD ? 3 : 1;
    __shared__ __attribute__((aligned(16))) float X_s[D * PD];   // [n][k]
    __shared__ __attribute__((aligned(16))) float A_s[BT * PD];  // [row][k]
    using TO = Tiles<BT / 32, D / 32>;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int prod = lid % nprod, rest0 = lid / nprod;
    const int part = rest0 % p.parts, rest = rest0 / p.parts;
    const int h = rest % p.H, gs = rest / p.H;
    Seq s;
    int sl;
    if (!seg_seq(p, gs, s, sl)) return;
    const int t0 = sl * p.G, t1 = min(min(t0 + p.G, s.T), p.n_chunks_ub - s.c0);
    if (t1 <= t0) return;
    const int seg_rows = min(t1 * p.C, s.len) - t0 * p.C;
    const int bpp = ((seg_rows + BT - 1) / BT + p.parts - 1) / p.parts;   // blocks per part
    const int row0 = t0 * p.C + part * bpp * BT;
    const int nrows = min(seg_rows - part * bpp * BT, bpp * BT);
    if (nrows <= 0) return;
    const int64_t rbase = (row_base(p, s, h) + row0) * D;
    const float *X = (KIND == RM_FWD || prod == 0 ? p.Pfin : p.Rfin) + ((int64_t)s.i * p.H + h) * D * D;
    const bool trans = KIND == RM_BWD && prod != 1;            // dQ, dK use the transpose
    const float *A;
    float *Out;
    if (KIND == RM_FWD) {
        A = (const float *)p.Q + rbase; Out = (float *)p.O + rbase;
    } else if (prod == 0) {
        A = (const float *)p.dO + rbase; Out = (float *)p.dQ + rbase;
    } else if (prod == 1) {
        A = (const float *)p.K + rbase; Out = (float *)p.dV + rbase;
    } else {
        A = (const float *)p.V + rbase; Out = (float *)p.dK + rbase;
    }
    // X_s[n][k] = X[n][k], or X[k][n] for the transpose (reads of X rows
    // coalesced either way)
    for (int e = threadIdx.x; e < D * D; e += NTHR) {
        const int r = e / D, c = e % D;
        const float x = X[e];
        if (trans) X_s[c * PD + r] = x;
        else X_s[r * PD + c] = x;
    }
    for (int b0 = 0; b0 < nrows; b0 += BT) {
        const int nv = min(BT, nrows - b0);
        __syncthreads();   // X_s written; A_s free
        stage_rows<float, BT, D>(A_s, PD, A + (int64_t)b0 * D, nv);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TO::PER_WAVE; ++k) {
            int mi, ni;
            if (!TO::get(k, mi, ni)) continue;
            f32x16 acc;
            zero(acc);
            gemm<float, D>(acc, A_s, PD, mi * 32, X_s, PD, ni * 32);
            store_rows(acc, Out + (int64_t)b0 * D, D, mi * 32, ni * 32, nv);
        }
    }
}

template <int D, int KIND>
static hipError_t segtot_launch(const Params &p, hipStream_t st) {
    const dim3 grid(round8(p.n_segs_ub * p.H)), block(SegTotCfg<D>::NT);
    if (p.decay) return launch_k(k_segtot_bf16<D, KIND, true>, grid, block, st, p);
    return launch_k(k_segtot_bf16<D, KIND, false>, grid, block, st, p);
}

template <int D, int KIND>
static hipError_t sweep_dispatch(const Params &p, hipStream_t st) {
    switch (p.C) {
    case 64: return sweep_launch<D, 64, KIND>(p, st);
    case 128: return sweep_launch<D, 128, KIND>(p, st);
    default: return sweep_launch<D, 256, KIND>(p, st);
    }
}

template <int D>
static hipError_t fwd_bf16(const Params &p0, bool with_output, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    Params p = p0;
    p.end_by_sweep = with_output ? 1 : 0;   // the output sweep writes Pfin and M_out
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY((segtot_launch<D, TOT_F>(p, st)));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_fwd_segscan<D, float>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    if (with_output) LASP_TRY((sweep_dispatch<D, SWEEP_OUT>(p, st)));
    return rec_event(ev, 3, st);
}

template <int D>
static hipError_t bwd_bf16(const Params &p0, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    Params p = p0;
    p.end_by_sweep = 1;   // the dV sweep writes Rfin and dM_in
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    LASP_TRY((segtot_launch<D, TOT_B>(p, st)));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_bwd_segscan<D, float>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    LASP_TRY((sweep_dispatch<D, SWEEP_GRADS>(p, st)));
    return rec_event(ev, 3, st);
}

template <int D, int KIND>
static hipError_t rowmat_launch(const Params &p0, bool bf, hipStream_t st) {
    const int prods = KIND == RM_BWD ? 3 : 1;
    // about 1024 workgroups (four per CU), parts of at least 8 tiles
    Params p = p0;
    const int64_t wg = (int64_t)p.n_segs_ub * p.H * prods;
    const int by_wg = (int)((1024 + wg - 1) / wg);
    const int by_rows = (p.G * p.C / 32) / 8;
    p.parts = by_wg < 1 ? 1 : (by_wg < by_rows ? by_wg : (by_rows < 1 ? 1 : by_rows));
    if (!bf) return launch_k(k_rowmat_f32<D, KIND>, dim3(round8(wg * p.parts)), dim3(NTHR), st, p);
    return launch_k(k_rowmat_bf16<D, KIND>, dim3(round8(wg * p.parts)), dim3(64 * RM_NW), st, p);
}

// The summed states come from the causal path's totals and scans (bf16:
// segment totals; float32: the per-chunk local kernels, whose chunk states go
// unused here), then one row-block product launch.
template <int D>
static hipError_t fwd_bidir(const Params &p, bool bf, bool with_output, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    constexpr int BT = Block<float, D>::BT;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    if (bf)
        LASP_TRY((segtot_launch<D, TOT_F>(p, st)));
    else
        LASP_TRY(launch_k(k_fwd_local<float, D, BT>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_fwd_segscan<D, float>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    if (with_output) LASP_TRY((rowmat_launch<D, RM_FWD>(p, bf, st)));
    return rec_event(ev, 3, st);
}

template <int D>
static hipError_t bwd_bidir(const Params &p, bool bf, hipStream_t st, hipEvent_t *ev) {
    constexpr int NB = (D * D + NTHR - 1) / NTHR;
    constexpr int BT = Block<float, D>::BT;
    if (p.varlen) LASP_TRY(launch_setup(p, st));
    LASP_TRY(rec_event(ev, 0, st));
    if (bf)
        LASP_TRY((segtot_launch<D, TOT_B>(p, st)));
    else
        LASP_TRY(launch_k(k_bwd_local<float, D, BT>, dim3(p.n_segs_ub * p.H), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 1, st));
    LASP_TRY(launch_k(k_bwd_segscan<D, float>, dim3(p.nseq * p.H * NB), dim3(NTHR), st, p));
    LASP_TRY(rec_event(ev, 2, st));
    LASP_TRY((rowmat_launch<D, RM_BWD>(p, bf, st)));
    return rec_event(ev, 3, st);
}

hipError_t launch_fwd_bidir(const Params &p, bool bf, bool with_output, hipStream_t st, hipEvent_t *ev) {
    if (p.decay || !p.Pfin || (!bf && !p.Lc)) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return fwd_bidir<32>(p, bf, with_output, st, ev);
    case 64: return fwd_bidir<64>(p, bf, with_output, st, ev);
    case 128: return fwd_bidir<128>(p, bf, with_output, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_bidir(const Params &p, bool bf, hipStream_t st, hipEvent_t *ev) {
    if (p.decay || !p.Pfin || !p.Rfin || (!bf && !p.Rc)) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bwd_bidir<32>(p, bf, st, ev);
    case 64: return bwd_bidir<64>(p, bf, st, ev);
    case 128: return bwd_bidir<128>(p, bf, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_norm_bwd_prep(const Params &p, bool bf, hipStream_t st) {
    if (!p.Yn || !p.dYn || !p.rstd_in || !p.dOn) return hipErrorInvalidValue;
    switch (p.D) {
    case 32: return bf ? rownorm_launch<bf16, 32, true>(p, st) : rownorm_launch<float, 32, true>(p, st);
    case 64: return bf ? rownorm_launch<bf16, 64, true>(p, st) : rownorm_launch<float, 64, true>(p, st);
    case 128: return bf ? rownorm_launch<bf16, 128, true>(p, st) : rownorm_launch<float, 128, true>(p, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const Params &p, bool bf, bool with_output, hipStream_t st, hipEvent_t *ev) {
    switch (p.D) {
    case 32: return bf ? fwd_bf16<32>(p, with_output, st, ev) : fwd_impl<float, 32>(p, with_output, st, ev);
    case 64: return bf ? fwd_bf16<64>(p, with_output, st, ev) : fwd_impl<float, 64>(p, with_output, st, ev);
    case 128: return bf ? fwd_bf16<128>(p, with_output, st, ev) : fwd_impl<float, 128>(p, with_output, st, ev);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const Params &p, bool bf, hipStream_t st, hipEvent_t *ev) {
    switch (p.D) {
    case 32: return bf ? bwd_bf16<32>(p, st, ev) : bwd_impl<float, 32>(p, st, ev);
    case 64: return bf ? bwd_bf16<64>(p, st, ev) : bwd_impl<float, 64>(p, st, ev);
    case 128: return bf ? bwd_bf16<128>(p, st, ev) : bwd_impl<float, 128>(p, st, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace lasp

