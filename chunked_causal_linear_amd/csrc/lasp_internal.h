// Internal interface between the C ABI (lasp_api.cpp) and the HIP kernels
// (lasp_kernels.hip).  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lasp {

// Gated backward: the forward state is kept at every GATED_CK-th chunk boundary
// inside a segment, where the log-gate gradient's running sum is reset to its
// exact value.
constexpr int GATED_CK = 8;

// Everything a kernel needs, by value in the kernel argument segment.
//
// Work decomposition (one head h of one sequence i, T chunks of length C, the
// last one possibly shorter):
//   chunks are numbered globally (over sequences) gc = c0(i) + t;
//   G consecutive chunks form a segment, numbered globally gs = s0(i) + t / G.
// State arrays are indexed [(global index) * H + h][D][D].
struct Params {
    int B, H, N;        // N: tokens per sequence (packed batch: total tokens)
    int nseq;           // number of sequences: B, or the packed count
    int D, C, G;        // head dim, chunk length, chunks per segment
    int varlen;         // 1: packed batch described by cu
    int T_fixed, S_fixed;          // chunks / segments per sequence (not packed)
    int n_chunks_ub, n_segs_ub;    // grid bounds (upper bounds when packed)
    const int32_t *cu;             // [nseq+1] device (packed)
    int32_t *chunk_prefix;         // [nseq+1] device (packed): first global chunk
    int32_t *seg_prefix;           // [nseq+1] device (packed): first global segment
    const float *decay;            // [H] device or null
    const void *Q, *K, *V, *dO;
    void *O, *dQ, *dK, *dV;
    const float *M_in, *dM_out;    // [nseq][H][D][D] or null
    float *M_out, *dM_in;          // [nseq][H][D][D] or null
    void *Lc;      // [chunks][H][D][D] elem: local prefix state entering each chunk, [dv][dk]
    float *Pseg;   // [segs][H][D][D] f32: state entering each segment, [dv][dk]
    float *Pfin;   // [nseq][H][D][D] f32 or null: state after each sequence's last token, [dv][dk]
    float *Z;      // [segs][H][D][D] f32: local state at each segment end, [dv][dk]
    void *Rc;      // [chunks][H][D][D] elem: local reverse state of each chunk, [dv][dk]
    float *Rseg;   // [segs][H][D][D] f32: reverse state entering each segment's last chunk
    float *W;      // [segs][H][D][D] f32: local reverse state at each segment start
    float *Rfin;   // [nseq][H][D][D] f32 or null: reverse state before each sequence's first token, [dv][dk]
    int parts;     // row-block products: workgroups per (segment, head, product)
    // output normalisation (Norm of LASP Eq. 2, read as a row-wise RMS norm)
    float *rstd;        // [B, H, N] f32: forward output 1/sqrt(mean(o^2) + eps) per row, or null
    const float *rstd_in;   // [B, H, N] f32: the forward's rstd (backward preparation)
    const void *Yn, *dYn;   // [B, H, N, d]: normalised output and its gradient
    void *dOn;              // [B, H, N, d]: gradient of the un-normalised output
    int dq_forward;         // 1: dQ walks forwards from the entering states even without
                            // decay (no subtraction walk; see the sweep kernel)
    int end_by_sweep;       // 1 (bf16 causal path): the sweeps write each sequence's end
                            // states (Pfin and M_out after the forward walk of its last
                            // segment, Rfin and dM_in after the dV walk of its first), so
                            // the totals of those segments are neither computed nor scanned
    // gated form
    const float *LG;   // [B, H, N, D] f32 log-gates (key channels)
    float *dLG;        // [B, H, N, D] f32 log-gate gradient
    float *Gs;         // [segs][H][D] f32: gate product of each segment
    float *Tq;         // [chunks][H][D] f32: per chunk, sum over its tokens of q . (2^b (dO P_t^T))
    float *Pck;        // [segs][H][(G-1)/GATED_CK][D][D] f32: forward states at every GATED_CK-th
                       // chunk boundary inside each segment, [dv][dk]
};

// Enqueue the forward kernels: (packed-batch tables), local chunk states,
// segment scan, and (if with_output) the output kernel.
// ev (nullable): 4 events recorded on the stream before the local-state kernel,
// before the scan, before the last kernel and after it.
hipError_t launch_fwd(const Params &p, bool bf16, bool with_output, hipStream_t stream,
                      hipEvent_t *ev = nullptr);
// Enqueue the backward kernels: (tables), reverse local states, reverse
// segment scan, gradient kernel.  The forward states (Lc, Pseg) must be valid.
hipError_t launch_bwd(const Params &p, bool bf16, hipStream_t stream, hipEvent_t *ev = nullptr);

// Unmasked (bidirectional) form, bf16, no decay.  Forward: (tables), segment
// totals, segment scan (Pfin = the summed state), O = Q M.  Backward: (tables),
// reverse totals, reverse scan (Rfin = the summed gradient state), then
// dQ = dO M^T, dV = K dM, dK = V dM^T; Pfin must be valid.
// Gated form (per-token, per-key-channel gates given as logs; chunk 64): segment
// totals, segment scan (Pseg, Pfin, with the segments' gate products Gs), the
// output walk; backward: reverse totals, reverse scan, the dQ walk (Tq, Pck),
// then the dV / dK / dlog_g walk, with the events of launch_fwd / launch_bwd
// (the two backward walks between the last two).
hipError_t launch_fwd_gated(const Params &p, bool bf16, bool with_output, hipStream_t stream,
                            hipEvent_t *ev = nullptr);
hipError_t launch_bwd_gated(const Params &p, bool bf16, hipStream_t stream, hipEvent_t *ev = nullptr);

// Bytes of the static scratch array used by lasp_fwd_noalloc, and the device
// address of the copy on the stream's GPU (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(hipStream_t stream, void **ptr);

// Output normalisation: Norm(o) = o / sqrt(mean_j o_j^2 + kNormEps) per row.
constexpr float kNormEps = 1e-6f;
// dOn = rstd_in * (dYn - Yn * mean(dYn . Yn)) per row (before launch_bwd).
hipError_t launch_norm_bwd_prep(const Params &p, bool bf16, hipStream_t stream);

// Packed-batch tables (chunk_prefix, seg_prefix) on the stream.
hipError_t launch_setup(const Params &p, hipStream_t stream);

// ev as for launch_fwd / launch_bwd (totals, scan, row-block products).
hipError_t launch_fwd_bidir(const Params &p, bool bf16, bool with_output, hipStream_t stream,
                            hipEvent_t *ev = nullptr);
hipError_t launch_bwd_bidir(const Params &p, bool bf16, hipStream_t stream, hipEvent_t *ev = nullptr);

}  // namespace lasp
