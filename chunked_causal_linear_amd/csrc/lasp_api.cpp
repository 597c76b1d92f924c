// C ABI of the chunked causal linear attention library: argument checks,
// workspace / state-cache layout and kernel launches (declared in include/lasp.h).
#include "../../include/lasp.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "lasp_internal.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Text of the last HIP error seen by a call on this thread (for
// lasp_status_string); the only state the library keeps between calls.
thread_local std::string g_hip_error;

// Sizes derived from the shape.  G (chunks per segment) is a pure function of
// the shape, or the caller's explicit segment_chunks, so that lasp_fwd and
// lasp_bwd agree on the state-cache layout whenever they get the same arguments.
struct Plan {
    int D, C, G, H, nseq, T_fixed, S_fixed, n_chunks_ub, n_segs_ub;
    bool varlen;
    size_t esz;          // element size of Q/K/V
    size_t table_b;      // packed-batch tables
    size_t local_b;      // per-chunk local states (Lc or Rc)
    size_t seg_b;        // per-segment f32 states (Pseg, Z, Rseg or W)
    size_t fin_b;        // per-sequence f32 final states (Pfin)
    size_t chunk_v;      // gated backward: per-chunk f32 vectors of D (Tq)
    size_t ck_b;         // gated backward: forward states at checkpoints inside segments (Pck)
    size_t gate_s;       // gated form: per-segment f32 gate products (Gs)
    size_t cache_b;      // state cache = [Lc][Pseg][Pfin][Gs]
};

// gated: the per-channel gated form (its kernels use chunks of 64 tokens
// whatever shape->chunk names).  seg_chunks: 0, or the number of chunks per
// segment to use instead of the library's choice.
int make_plan(const lasp_shape *s, lasp_dtype dt, Plan &pl, bool gated = false,
              int seg_chunks = 0) {
    if (!s) return LASP_EINVAL;
    if (s->B <= 0 || s->H <= 0 || s->N <= 0 || s->d <= 0 || s->chunk <= 0 || s->nseq < 0)
        return LASP_EINVAL;
    if (s->nseq > 0 && s->B != 1) return LASP_EINVAL;
    if (dt != LASP_FP32 && dt != LASP_BF16) return LASP_EUNSUPPORTED;
    if (s->d != 32 && s->d != 64 && s->d != 128) return LASP_EUNSUPPORTED;
    if (s->chunk != 64 && s->chunk != 128 && s->chunk != 256) return LASP_EUNSUPPORTED;
    if (seg_chunks < 0 || seg_chunks > (1 << 20)) return LASP_EINVAL;
    // the gated kernels always work on chunks of 64 tokens (the result does
    // not depend on the chunking; shape->chunk only names a supported length)
    const int chunk = gated ? 64 : s->chunk;
    pl.D = s->d;
    pl.C = chunk;
    pl.H = s->H;
    pl.varlen = s->nseq > 0;
    pl.nseq = pl.varlen ? s->nseq : s->B;
    pl.esz = dt == LASP_BF16 ? 2 : 4;
    const int64_t per_seq_chunks = ((int64_t)s->N + chunk - 1) / chunk;
    int64_t chunks_ub = pl.varlen ? (int64_t)s->N / chunk + s->nseq
                                  : per_seq_chunks * (int64_t)s->B;
    // Segments of G chunks: one sweep workgroup each per (segment, head, role),
    // one resident per CU (256 CUs on MI355X), each taking a time about
    // G + 2 chunks (the 2: its start-up).  G minimizes (G + 2) x (rounds of the
    // one-role launches + rounds of the three-role backward launch), the
    // larger G on ties (fewer segment states, cheaper scans).  Packed batches
    // count one extra partial segment per sequence.  Measured at B1 H32 N131072 C256:
    // G = 16, 32, 48, 64 -> 4.30, 4.24, 5.09, 4.25 ms per forward+backward
    // (48 leaves the second round nearly empty).
    if (gated) {
        // the gated walks take G chunks per (segment, head): about 1024 of
        // them (two rounds of two workgroups per CU at d = 128; measured at
        // B1 H32 N131072 d128: G = 16, 32, 64, 128 -> 14.42, 14.20, 13.98,
        // 14.00 ms per forward+backward), segments of 1 to 64 chunks
        const int64_t g = chunks_ub * s->H / 1024;
        pl.G = (int)(g < 1 ? 1 : (g > 64 ? 64 : g));
    } else {
        const int64_t seqs = pl.varlen ? 1 : s->B;
        const int64_t T = pl.varlen ? chunks_ub : per_seq_chunks;   // chunks per sequence (packed: all)
        const int64_t extra = pl.varlen ? s->nseq : 0;              // packed: one partial segment per sequence
        int64_t best_cost = -1;
        for (int g = 1; g <= 256; ++g) {
            const int64_t wg = seqs * s->H * ((T + g - 1) / g + extra);
            const int64_t cost = (int64_t)(g + 2) * ((wg + 255) / 256 + (3 * wg + 255) / 256);
            if (best_cost < 0 || cost <= best_cost) {
                best_cost = cost;
                pl.G = g;
            }
        }
    }
    if (seg_chunks > 0) pl.G = seg_chunks;
    int64_t segs_ub;
    if (pl.varlen) {
        segs_ub = chunks_ub / pl.G + s->nseq;
        pl.T_fixed = pl.S_fixed = 0;
    } else {
        pl.T_fixed = (int)per_seq_chunks;
        pl.S_fixed = (int)((per_seq_chunks + pl.G - 1) / pl.G);
        segs_ub = (int64_t)pl.S_fixed * s->B;
    }
    // grid and index limits (grids are 1-D: chunks * H workgroups)
    if (chunks_ub * s->H > (int64_t)0x3fffffff || (int64_t)s->B * s->H * s->N > ((int64_t)1 << 40))
        return LASP_EINVAL;
    pl.n_chunks_ub = (int)chunks_ub;
    pl.n_segs_ub = (int)segs_ub;
    const size_t dd = (size_t)pl.D * pl.D;
    pl.table_b = pl.varlen ? align_up(2 * sizeof(int32_t) * ((size_t)pl.nseq + 1)) : 0;
    // per-chunk local states: only the float32 causal path keeps them (the bf16
    // path and the gated walks carry chunk states in registers)
    pl.local_b = (dt == LASP_BF16 || gated)
                     ? 0 : align_up((size_t)pl.n_chunks_ub * pl.H * dd * pl.esz);
    pl.seg_b = align_up((size_t)pl.n_segs_ub * pl.H * dd * sizeof(float));
    // final states: the bf16 backward starts its subtraction walk of dQ from
    // them, the unmasked form's row products read them, and the gated
    // backward's log-gate gradient of a sequence's last segment (both dtypes)
    pl.fin_b = align_up((size_t)pl.nseq * pl.H * dd * sizeof(float));
    pl.chunk_v = gated ? align_up((size_t)pl.n_chunks_ub * pl.H * pl.D * sizeof(float)) : 0;
    pl.ck_b = gated ? align_up((size_t)pl.n_segs_ub * pl.H * ((pl.G - 1) / lasp::GATED_CK) * dd * sizeof(float))
                    : 0;
    pl.gate_s = gated ? align_up((size_t)pl.n_segs_ub * pl.H * pl.D * sizeof(float)) : 0;
    pl.cache_b = pl.local_b + pl.seg_b + pl.fin_b + pl.gate_s;
    return LASP_OK;
}

size_t fwd_ws(const Plan &pl, bool cache) {
    return pl.table_b + pl.seg_b /*Z*/ + (cache ? 0 : pl.cache_b);
}
size_t bwd_ws(const Plan &pl, bool cache) {
    return pl.table_b + pl.local_b /*Rc*/ + 2 * pl.seg_b /*Rseg, W*/ + pl.fin_b /*Rfin*/ +
           pl.chunk_v /*Tq*/ + pl.ck_b /*Pck*/ +
           (cache ? 0 : pl.cache_b + pl.seg_b /*Lc, Pseg, Pfin, Z*/);
}

// bytes of one [B, H, N, d] token array, aligned
size_t norm_bwd_extra(const lasp_shape *s, const Plan &pl) {
    return align_up((size_t)s->B * s->H * s->N * s->d * pl.esz);
}

bool misaligned(const void *p, size_t a) { return p && ((uintptr_t)p % a) != 0; }

struct Range {
    const void *p;
    size_t n;
};
bool overlap(Range a, Range b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}
// Every output range must be disjoint from every other listed range.
bool any_overlap(const Range *outs, int no, const Range *ins, int ni) {
    for (int i = 0; i < no; ++i) {
        for (int j = 0; j < ni; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}

void fill_common(lasp::Params &p, const lasp_shape *s, const Plan &pl, const int32_t *cu,
                 const float *decay) {
    memset(&p, 0, sizeof(p));
    p.B = s->B;
    p.H = s->H;
    p.N = s->N;
    p.nseq = pl.nseq;
    p.D = pl.D;
    p.C = pl.C;
    p.G = pl.G;
    p.varlen = pl.varlen ? 1 : 0;
    p.T_fixed = pl.T_fixed;
    p.S_fixed = pl.S_fixed;
    p.n_chunks_ub = pl.n_chunks_ub;
    p.n_segs_ub = pl.n_segs_ub;
    p.cu = cu;
    p.decay = decay;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return LASP_OK;
    g_hip_error = hipGetErrorString(e);
    return LASP_EHIP;
}

}  // namespace

extern "C" {

size_t lasp_state_cache_bytes(const lasp_shape *shape, lasp_dtype dtype) {
    Plan pl;
    return make_plan(shape, dtype, pl) == LASP_OK ? pl.cache_b : 0;
}

size_t lasp_gated_state_cache_bytes(const lasp_shape *shape, lasp_dtype dtype) {
    Plan pl;
    return make_plan(shape, dtype, pl, true) == LASP_OK ? pl.cache_b : 0;
}

size_t lasp_gated_fwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                      int with_state_cache) {
    Plan pl;
    return make_plan(shape, dtype, pl, true) == LASP_OK ? fwd_ws(pl, with_state_cache != 0) : 0;
}

size_t lasp_gated_bwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                      int with_state_cache) {
    Plan pl;
    return make_plan(shape, dtype, pl, true) == LASP_OK ? bwd_ws(pl, with_state_cache != 0) : 0;
}

size_t lasp_fwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype, int with_state_cache) {
    Plan pl;
    return make_plan(shape, dtype, pl) == LASP_OK ? fwd_ws(pl, with_state_cache != 0) : 0;
}

size_t lasp_bwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype, int with_state_cache) {
    Plan pl;
    return make_plan(shape, dtype, pl) == LASP_OK ? bwd_ws(pl, with_state_cache != 0) : 0;
}

int lasp_query_sizes(const lasp_shape *shape, lasp_dtype dtype, int form, int segment_chunks,
                     lasp_sizes *out) {
    if (!out || form < 0 || form > 2 || (form == 2 && segment_chunks != 0)) return LASP_EINVAL;
    Plan pl;
    const int rc = make_plan(shape, dtype, pl, form == 1, segment_chunks);
    if (rc != LASP_OK) return rc;
    // the normalised form's backward also holds the un-normalised output's
    // gradient (one token array)
    const size_t extra = form == 2 ? norm_bwd_extra(shape, pl) : 0;
    out->state_cache = pl.cache_b;
    out->fwd_workspace[0] = fwd_ws(pl, false);
    out->fwd_workspace[1] = fwd_ws(pl, true);
    out->bwd_workspace[0] = bwd_ws(pl, false) + extra;
    out->bwd_workspace[1] = bwd_ws(pl, true) + extra;
    out->segment_chunks = pl.G;
    return LASP_OK;
}

// With LASP_DEBUG=1 in the environment, the contents of a packed batch's
// cu_seqlens and of the decay array are copied to the host (after the work
// already on the stream) and checked: cu[0] = 0, non-decreasing, cu[nseq] = N;
// every lambda in [0, 1].  Otherwise their contents are trusted.
static int debug_check(const lasp_shape *shape, const int32_t *cu, const float *decay,
                       hipStream_t stream) {
    const char *e = getenv("LASP_DEBUG");
    if ((!cu && !decay) || !e || strcmp(e, "1") != 0) return LASP_OK;
    std::vector<int32_t> h(cu ? (size_t)shape->nseq + 1 : 0);
    std::vector<float> lam(decay ? (size_t)shape->H : 0);
    hipError_t err = hipSuccess;
    if (cu)
        err = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                             stream);
    if (err == hipSuccess && decay)
        err = hipMemcpyAsync(lam.data(), decay, lam.size() * sizeof(float), hipMemcpyDeviceToHost,
                             stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) return hip_status(err);
    if (cu) {
        if (h[0] != 0 || h.back() != shape->N) return LASP_EINVAL;
        for (size_t i = 1; i < h.size(); ++i)
            if (h[i] < h[i - 1]) return LASP_EINVAL;
    }
    for (float x : lam)
        if (!(x >= 0.f && x <= 1.f)) return LASP_EINVAL;   // NaN fails too
    return LASP_OK;
}

}  // extern "C"

namespace {

enum Mode { CAUSAL, BIDIR, GATED, NORM };

int fwd_common(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
               const void *V, const float *decay, const float *log_g,
               const int32_t *cu_seqlens, const float *M_in, void *O, float *M_out,
               void *state_cache, void *workspace, size_t workspace_bytes, void *stream,
               void **events, int seg_chunks, Mode mode, float *rstd = nullptr) {
    Plan pl;
    int rc = make_plan(shape, dtype, pl, mode == GATED, seg_chunks);
    if (rc != LASP_OK) return rc;
    if (!Q || !K || !V || !O || (mode == GATED && !log_g) || (mode == NORM && !rstd))
        return LASP_EINVAL;
    if (misaligned(rstd, 4)) return LASP_EINVAL;
    if ((shape->nseq > 0) != (cu_seqlens != nullptr)) return LASP_EINVAL;
    const void *a16[] = {Q, K, V, O, M_in, M_out, state_cache, workspace, log_g};
    for (const void *ptr : a16)
        if (misaligned(ptr, 16)) return LASP_EINVAL;
    if (misaligned(decay, 4) || misaligned(cu_seqlens, 4)) return LASP_EINVAL;
    const bool cache = state_cache != nullptr;
    const size_t need = fwd_ws(pl, cache);
    if (workspace_bytes < need || (need && !workspace)) return LASP_EWORKSPACE;

    const size_t tens = (size_t)shape->B * shape->H * shape->N * shape->d * pl.esz;
    const size_t gates = (size_t)shape->B * shape->H * shape->N * shape->d * sizeof(float);
    const size_t st = (size_t)pl.nseq * pl.H * pl.D * pl.D * sizeof(float);
    const Range ins[] = {{Q, tens}, {K, tens}, {V, tens}, {M_in, st},
                         {decay, (size_t)pl.H * 4},
                         {cu_seqlens, cu_seqlens ? ((size_t)pl.nseq + 1) * 4 : 0},
                         {log_g, log_g ? gates : 0}};
    const size_t rows_b = (size_t)shape->B * shape->H * shape->N * sizeof(float);
    const Range outs[] = {{O, tens}, {M_out, st}, {state_cache, cache ? pl.cache_b : 0},
                          {workspace, need}, {rstd, rstd ? rows_b : 0}};
    if (any_overlap(outs, 5, ins, 7)) return LASP_EINVAL;
    if ((rc = debug_check(shape, cu_seqlens, decay, (hipStream_t)stream)) != LASP_OK) return rc;

    lasp::Params p;
    fill_common(p, shape, pl, cu_seqlens, decay);
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.O = O;
    p.M_in = M_in;
    p.M_out = M_out;
    p.rstd = rstd;
    char *w = (char *)workspace;
    if (pl.varlen) {
        p.chunk_prefix = (int32_t *)w;
        p.seg_prefix = p.chunk_prefix + (pl.nseq + 1);
        w += pl.table_b;
    }
    p.Z = (float *)w;
    w += pl.seg_b;
    char *c = cache ? (char *)state_cache : w;
    p.Lc = pl.local_b ? c : nullptr;
    p.Pseg = (float *)(c + pl.local_b);
    p.Pfin = pl.fin_b ? (float *)(c + pl.local_b + pl.seg_b) : nullptr;
    if (mode == BIDIR)
        return hip_status(lasp::launch_fwd_bidir(p, dtype == LASP_BF16, true, (hipStream_t)stream,
                                                 (hipEvent_t *)events));
    if (mode == GATED) {
        p.LG = log_g;
        p.Gs = (float *)(c + pl.local_b + pl.seg_b + pl.fin_b);
        return hip_status(lasp::launch_fwd_gated(p, dtype == LASP_BF16, true, (hipStream_t)stream,
                                                 (hipEvent_t *)events));
    }
    return hip_status(lasp::launch_fwd(p, dtype == LASP_BF16, true, (hipStream_t)stream,
                                       (hipEvent_t *)events));
}

}  // namespace

extern "C" {

int lasp_fwd_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                const void *V, const float *decay, const int32_t *cu_seqlens, const float *M_in,
                void *O, float *M_out, void *state_cache, void *workspace,
                size_t workspace_bytes, void *stream, void **events, int segment_chunks) {
    return fwd_common(shape, dtype, Q, K, V, decay, nullptr, cu_seqlens, M_in, O, M_out,
                      state_cache, workspace, workspace_bytes, stream, events, segment_chunks,
                      CAUSAL);
}

int lasp_fwd_bidir_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                      const void *V, const int32_t *cu_seqlens, const float *M_in, void *O,
                      float *M_out, void *state_cache, void *workspace, size_t workspace_bytes,
                      void *stream, void **events, int segment_chunks) {
    return fwd_common(shape, dtype, Q, K, V, nullptr, nullptr, cu_seqlens, M_in, O, M_out,
                      state_cache, workspace, workspace_bytes, stream, events, segment_chunks,
                      BIDIR);
}

int lasp_fwd_bidir(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                   const void *V, const int32_t *cu_seqlens, const float *M_in, void *O,
                   float *M_out, void *state_cache, void *workspace, size_t workspace_bytes,
                   void *stream) {
    return lasp_fwd_bidir_ex(shape, dtype, Q, K, V, cu_seqlens, M_in, O, M_out, state_cache,
                             workspace, workspace_bytes, stream, nullptr, 0);
}

int lasp_fwd_gated_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                      const void *V, const float *log_g, const int32_t *cu_seqlens,
                      const float *M_in, void *O, float *M_out, void *state_cache,
                      void *workspace, size_t workspace_bytes, void *stream, void **events,
                      int segment_chunks) {
    return fwd_common(shape, dtype, Q, K, V, nullptr, log_g, cu_seqlens, M_in, O, M_out,
                      state_cache, workspace, workspace_bytes, stream, events, segment_chunks,
                      GATED);
}

int lasp_fwd_gated(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                   const void *V, const float *log_g, const int32_t *cu_seqlens,
                   const float *M_in, void *O, float *M_out, void *state_cache, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return lasp_fwd_gated_ex(shape, dtype, Q, K, V, log_g, cu_seqlens, M_in, O, M_out,
                             state_cache, workspace, workspace_bytes, stream, nullptr, 0);
}

int lasp_fwd(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
             const void *V, const float *decay, const int32_t *cu_seqlens, const float *M_in,
             void *O, float *M_out, void *state_cache, void *workspace, size_t workspace_bytes,
             void *stream) {
    return lasp_fwd_ex(shape, dtype, Q, K, V, decay, cu_seqlens, M_in, O, M_out, state_cache,
                       workspace, workspace_bytes, stream, nullptr, 0);
}

int lasp_fwd_norm(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                  const void *V, const float *decay, const int32_t *cu_seqlens,
                  const float *M_in, void *Y, float *rstd, float *M_out, void *state_cache,
                  void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_common(shape, dtype, Q, K, V, decay, nullptr, cu_seqlens, M_in, Y, M_out,
                      state_cache, workspace, workspace_bytes, stream, nullptr, 0, NORM, rstd);
}

size_t lasp_noalloc_scratch_bytes(void) { return lasp::kStaticScratchBytes; }

int lasp_fwd_noalloc(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                     const void *V, const float *decay, const int32_t *cu_seqlens,
                     const float *M_in, void *O, float *M_out, void *state_cache, void *stream) {
    Plan pl;
    const int rc = make_plan(shape, dtype, pl);
    if (rc != LASP_OK) return rc;
    // the scratch takes what lasp_fwd's workspace would hold; checked before
    // the device is touched
    if (fwd_ws(pl, state_cache != nullptr) > lasp::kStaticScratchBytes) return LASP_ESCRATCH;
    void *ws = nullptr;
    const int st = hip_status(lasp::static_scratch((hipStream_t)stream, &ws));
    if (st != LASP_OK) return st;
    return fwd_common(shape, dtype, Q, K, V, decay, nullptr, cu_seqlens, M_in, O, M_out,
                      state_cache, ws, lasp::kStaticScratchBytes, stream, nullptr, 0, CAUSAL);
}

}  // extern "C"

namespace {

int bwd_common(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
               const void *V, const void *dO, const float *decay, const float *log_g,
               const int32_t *cu_seqlens, const float *M_in, const float *dM_out,
               const void *state_cache, void *dQ, void *dK, void *dV, float *dlog_g,
               float *dM_in, void *workspace, size_t workspace_bytes, void *stream,
               void **events, int seg_chunks, Mode mode, const void *Y = nullptr,
               const float *rstd = nullptr) {
    Plan pl;
    int rc = make_plan(shape, dtype, pl, mode == GATED, seg_chunks);
    if (rc != LASP_OK) return rc;
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return LASP_EINVAL;
    if (mode == GATED && (!log_g || !dlog_g)) return LASP_EINVAL;
    if (mode == NORM && (!Y || !rstd)) return LASP_EINVAL;
    if (misaligned(Y, 16) || misaligned(rstd, 4)) return LASP_EINVAL;
    if ((shape->nseq > 0) != (cu_seqlens != nullptr)) return LASP_EINVAL;
    const void *a16[] = {Q,  K,  V,  dO,    M_in,      dM_out, state_cache,
                         dQ, dK, dV, dM_in, workspace, log_g,  dlog_g};
    for (const void *ptr : a16)
        if (misaligned(ptr, 16)) return LASP_EINVAL;
    if (misaligned(decay, 4) || misaligned(cu_seqlens, 4)) return LASP_EINVAL;
    const bool cache = state_cache != nullptr;
    const size_t extra = mode == NORM ? norm_bwd_extra(shape, pl) : 0;
    const size_t need = bwd_ws(pl, cache) + extra;
    if (workspace_bytes < need || (need && !workspace)) return LASP_EWORKSPACE;

    const size_t tens = (size_t)shape->B * shape->H * shape->N * shape->d * pl.esz;
    const size_t gates = (size_t)shape->B * shape->H * shape->N * shape->d * sizeof(float);
    const size_t st = (size_t)pl.nseq * pl.H * pl.D * pl.D * sizeof(float);
    const size_t rows_b = (size_t)shape->B * shape->H * shape->N * sizeof(float);
    const Range ins[] = {{Q, tens}, {K, tens}, {V, tens}, {dO, tens}, {M_in, st}, {dM_out, st},
                         {state_cache, cache ? pl.cache_b : 0},
                         {decay, (size_t)pl.H * 4},
                         {cu_seqlens, cu_seqlens ? ((size_t)pl.nseq + 1) * 4 : 0},
                         {log_g, log_g ? gates : 0}, {Y, Y ? tens : 0},
                         {rstd, rstd ? rows_b : 0}};
    const Range outs[] = {{dQ, tens}, {dK, tens}, {dV, tens}, {dM_in, st}, {workspace, need},
                          {dlog_g, mode == GATED ? gates : 0}};
    if (any_overlap(outs, 6, ins, 12)) return LASP_EINVAL;
    if ((rc = debug_check(shape, cu_seqlens, decay, (hipStream_t)stream)) != LASP_OK) return rc;

    lasp::Params p;
    fill_common(p, shape, pl, cu_seqlens, decay);
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.dO = dO;
    p.dQ = dQ;
    p.dK = dK;
    p.dV = dV;
    p.M_in = M_in;
    p.dM_out = dM_out;
    p.dM_in = dM_in;
    char *w = (char *)workspace;
    if (pl.varlen) {
        p.chunk_prefix = (int32_t *)w;
        p.seg_prefix = p.chunk_prefix + (pl.nseq + 1);
        w += pl.table_b;
    }
    p.Rc = pl.local_b ? w : nullptr;
    w += pl.local_b;
    p.Rseg = (float *)w;
    w += pl.seg_b;
    p.W = (float *)w;
    w += pl.seg_b;
    p.Rfin = pl.fin_b ? (float *)w : nullptr;
    w += pl.fin_b;
    p.Tq = pl.chunk_v ? (float *)w : nullptr;
    w += pl.chunk_v;
    p.Pck = pl.ck_b ? (float *)w : nullptr;
    w += pl.ck_b;
    p.LG = log_g;
    p.dLG = dlog_g;
    const hipStream_t hs = (hipStream_t)stream;
    char *c = cache ? (char *)const_cast<void *>(state_cache) : w;
    p.Lc = pl.local_b ? c : nullptr;
    p.Pseg = (float *)(c + pl.local_b);
    p.Pfin = pl.fin_b ? (float *)(c + pl.local_b + pl.seg_b) : nullptr;
    if (mode == GATED) p.Gs = (float *)(c + pl.local_b + pl.seg_b + pl.fin_b);
    if (mode == NORM) {   // the gradient of the un-normalised output, into the workspace's end
        p.Yn = Y;
        p.dYn = dO;
        p.rstd_in = rstd;
        p.dOn = (char *)workspace + (need - extra);
        rc = hip_status(lasp::launch_norm_bwd_prep(p, dtype == LASP_BF16, hs));
        if (rc != LASP_OK) return rc;
        p.dO = p.dOn;
        p.dq_forward = 1;   // dO rows scaled by 1/rms of each output row: no subtraction walk
    }
    if (!cache) {   // recompute the forward states (no output, no M_out)
        p.Z = (float *)(w + pl.cache_b);
        const bool bf = dtype == LASP_BF16;
        rc = hip_status(mode == BIDIR   ? lasp::launch_fwd_bidir(p, bf, false, hs)
                        : mode == GATED ? lasp::launch_fwd_gated(p, bf, false, hs)
                                        : lasp::launch_fwd(p, bf, false, hs));
        if (rc != LASP_OK) return rc;
    }
    if (mode == BIDIR)
        return hip_status(lasp::launch_bwd_bidir(p, dtype == LASP_BF16, hs, (hipEvent_t *)events));
    if (mode == GATED)
        return hip_status(lasp::launch_bwd_gated(p, dtype == LASP_BF16, hs, (hipEvent_t *)events));
    return hip_status(lasp::launch_bwd(p, dtype == LASP_BF16, hs, (hipEvent_t *)events));
}

}  // namespace

extern "C" {

int lasp_bwd_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                const void *V, const void *dO, const float *decay, const int32_t *cu_seqlens,
                const float *M_in, const float *dM_out, const void *state_cache, void *dQ,
                void *dK, void *dV, float *dM_in, void *workspace, size_t workspace_bytes,
                void *stream, void **events, int segment_chunks) {
    return bwd_common(shape, dtype, Q, K, V, dO, decay, nullptr, cu_seqlens, M_in, dM_out,
                      state_cache, dQ, dK, dV, nullptr, dM_in, workspace, workspace_bytes, stream,
                      events, segment_chunks, CAUSAL);
}

int lasp_bwd_bidir_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                      const void *V, const void *dO, const int32_t *cu_seqlens,
                      const float *M_in, const float *dM_out, const void *state_cache, void *dQ,
                      void *dK, void *dV, float *dM_in, void *workspace, size_t workspace_bytes,
                      void *stream, void **events, int segment_chunks) {
    return bwd_common(shape, dtype, Q, K, V, dO, nullptr, nullptr, cu_seqlens, M_in, dM_out,
                      state_cache, dQ, dK, dV, nullptr, dM_in, workspace, workspace_bytes, stream,
                      events, segment_chunks, BIDIR);
}

int lasp_bwd_bidir(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                   const void *V, const void *dO, const int32_t *cu_seqlens, const float *M_in,
                   const float *dM_out, const void *state_cache, void *dQ, void *dK, void *dV,
                   float *dM_in, void *workspace, size_t workspace_bytes, void *stream) {
    return lasp_bwd_bidir_ex(shape, dtype, Q, K, V, dO, cu_seqlens, M_in, dM_out, state_cache,
                             dQ, dK, dV, dM_in, workspace, workspace_bytes, stream, nullptr, 0);
}

int lasp_bwd_gated_ex(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                      const void *V, const float *log_g, const void *dO,
                      const int32_t *cu_seqlens, const float *M_in, const float *dM_out,
                      const void *state_cache, void *dQ, void *dK, void *dV, float *dlog_g,
                      float *dM_in, void *workspace, size_t workspace_bytes, void *stream,
                      void **events, int segment_chunks) {
    return bwd_common(shape, dtype, Q, K, V, dO, nullptr, log_g, cu_seqlens, M_in, dM_out,
                      state_cache, dQ, dK, dV, dlog_g, dM_in, workspace, workspace_bytes, stream,
                      events, segment_chunks, GATED);
}

int lasp_bwd_gated(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                   const void *V, const float *log_g, const void *dO, const int32_t *cu_seqlens,
                   const float *M_in, const float *dM_out, const void *state_cache, void *dQ,
                   void *dK, void *dV, float *dlog_g, float *dM_in, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return lasp_bwd_gated_ex(shape, dtype, Q, K, V, log_g, dO, cu_seqlens, M_in, dM_out,
                             state_cache, dQ, dK, dV, dlog_g, dM_in, workspace, workspace_bytes,
                             stream, nullptr, 0);
}

int lasp_bwd_norm(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
                  const void *V, const void *Y, const float *rstd, const void *dY,
                  const float *decay, const int32_t *cu_seqlens, const float *M_in,
                  const float *dM_out, const void *state_cache, void *dQ, void *dK, void *dV,
                  float *dM_in, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_common(shape, dtype, Q, K, V, dY, decay, nullptr, cu_seqlens, M_in, dM_out,
                      state_cache, dQ, dK, dV, nullptr, dM_in, workspace, workspace_bytes, stream,
                      nullptr, 0, NORM, Y, rstd);
}

int lasp_bwd(const lasp_shape *shape, lasp_dtype dtype, const void *Q, const void *K,
             const void *V, const void *dO, const float *decay, const int32_t *cu_seqlens,
             const float *M_in, const float *dM_out, const void *state_cache, void *dQ, void *dK,
             void *dV, float *dM_in, void *workspace, size_t workspace_bytes, void *stream) {
    return lasp_bwd_ex(shape, dtype, Q, K, V, dO, decay, cu_seqlens, M_in, dM_out, state_cache,
                       dQ, dK, dV, dM_in, workspace, workspace_bytes, stream, nullptr, 0);
}

const char *lasp_status_string(int status) {
    switch (status) {
    case LASP_OK: return "ok";
    case LASP_EINVAL: return "invalid argument";
    case LASP_EUNSUPPORTED:
        return "unsupported configuration (d in {32,64,128}, chunk in {64,128,256}, dtype fp32/bf16; "
               "gated form: chunk 64; unmasked form: bf16)";
    case LASP_EWORKSPACE: return "workspace too small";
    case LASP_EHIP: return g_hip_error.empty() ? "HIP error" : g_hip_error.c_str();
    case LASP_ESCRATCH:
        return "the call needs more scratch than lasp_fwd_noalloc's static array holds "
               "(lasp_noalloc_scratch_bytes); use lasp_fwd with a workspace";
    }
    return "unknown status";
}

int lasp_version(void) { return 200; }

}  // extern "C"
