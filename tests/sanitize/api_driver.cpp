// Host-only check of the C ABI's plan and workspace arithmetic, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
//
// The library's C ABI source is compiled in directly; the kernel launchers it
// calls are replaced by stubs that check, for every array the plan places in
// the caller's buffers (packed-batch tables, segment states, final states,
// per-chunk states and gate products), that its whole extent lies inside the
// buffer it was carved from and overlaps no other array.  The pointers are
// fake, aligned addresses that nothing dereferences, so no GPU is involved.
// The three HIP runtime calls the ABI makes itself are stubbed too: the debug
// path's device-to-host copy fills the host array from a table the driver sets.
//
// Exit status 0 and "ok <cases>" on success; a message and status 1 on the
// first failure; a sanitizer report aborts the process.
#include "../../chunked_causal_linear_amd/csrc/lasp_api.cpp"

#include <stdio.h>

#include <algorithm>
#include <utility>

namespace {

struct Buf {
    uintptr_t base;
    size_t bytes;
    const char *name;
};
std::vector<Buf> g_bufs;           // buffers the current call was given
int g_failures = 0;
int g_launches = 0;
std::vector<int32_t> g_cu_host;    // what the stubbed copy returns for cu_seqlens
std::vector<float> g_decay_host;   // and for decay

void fail(const char *what, const char *name) {
    fprintf(stderr, "FAIL: %s (%s)\n", what, name);
    ++g_failures;
}

struct Extent {
    uintptr_t a, n;
    const char *name;
};

// every array must lie inside one caller buffer; no two arrays may overlap
void check_extents(std::vector<Extent> ex) {
    for (const Extent &e : ex) {
        if (!e.n) continue;
        bool inside = false;
        for (const Buf &b : g_bufs)
            if (e.a >= b.base && e.a + e.n <= b.base + b.bytes) inside = true;
        if (!inside) fail("array outside every caller buffer", e.name);
    }
    for (size_t i = 0; i < ex.size(); ++i)
        for (size_t j = i + 1; j < ex.size(); ++j) {
            const Extent &x = ex[i], &y = ex[j];
            if (x.n && y.n && x.a < y.a + y.n && y.a < x.a + x.n) {
                fprintf(stderr, "overlap: %s and %s\n", x.name, y.name);
                fail("arrays overlap", x.name);
            }
        }
}

uintptr_t U(const void *p) { return (uintptr_t)p; }

// extents of the state arrays a forward (fwd = true) or backward launch uses
void check_params(const lasp::Params &p, bool fwd, bool bf16, bool gated, bool bidir) {
    ++g_launches;
    const size_t H = p.H, D = p.D, dd = D * D, esz = bf16 ? 2 : 4;
    const size_t chunks = p.n_chunks_ub, segs = p.n_segs_ub, nseq = p.nseq;
    std::vector<Extent> ex;
    if (p.varlen) {
        ex.push_back({U(p.chunk_prefix), (nseq + 1) * 4, "chunk_prefix"});
        ex.push_back({U(p.seg_prefix), (nseq + 1) * 4, "seg_prefix"});
        if (!p.chunk_prefix || !p.seg_prefix) fail("packed tables missing", "tables");
    }
    const bool local = !bf16 && !gated;   // float32 causal and unmasked forms
    if (local && !p.Lc) fail("per-chunk states missing", "Lc");
    ex.push_back({U(p.Lc), local ? chunks * H * dd * esz : 0, "Lc"});
    ex.push_back({U(p.Pseg), segs * H * dd * 4, "Pseg"});
    const bool fin = true;   // every form and dtype keeps the final states
    if (fin && !p.Pfin) fail("final states missing", "Pfin");
    ex.push_back({U(p.Pfin), fin ? nseq * H * dd * 4 : 0, "Pfin"});
    if (gated) {
        if (!p.Gs) fail("segment gate products missing", "Gs");
        ex.push_back({U(p.Gs), segs * H * D * 4, "Gs"});
    }
    if (fwd || p.Z) ex.push_back({U(p.Z), segs * H * dd * 4, "Z"});
    if (!fwd) {
        ex.push_back({U(p.Rc), local ? chunks * H * dd * esz : 0, "Rc"});
        ex.push_back({U(p.Rseg), segs * H * dd * 4, "Rseg"});
        ex.push_back({U(p.W), segs * H * dd * 4, "W"});
        ex.push_back({U(p.Rfin), fin ? nseq * H * dd * 4 : 0, "Rfin"});
        if (fin && !p.Rfin) fail("reverse final states missing", "Rfin");
        if (gated) {
            if (!p.Tq) fail("per-chunk sums missing", "Tq");
            ex.push_back({U(p.Tq), chunks * H * D * 4, "Tq"});
            ex.push_back({U(p.Pck), segs * H * ((p.G - 1) / lasp::GATED_CK) * dd * 4, "Pck"});
        }
    }
    // the chunk and segment bounds cover every split of the tokens
    const int64_t T = ((int64_t)p.N + p.C - 1) / p.C;
    if (!p.varlen) {
        if ((int64_t)p.T_fixed != T || (int64_t)chunks != T * p.B) fail("chunk count", "T");
        if ((int64_t)p.S_fixed != (T + p.G - 1) / p.G || (int64_t)segs != (int64_t)p.S_fixed * p.B)
            fail("segment count", "S");
    } else if ((int64_t)chunks < (int64_t)p.N / p.C + p.nseq ||
               (int64_t)segs < (int64_t)chunks / p.G + p.nseq) {
        fail("packed bounds", "ub");
    }
    if (bidir && !bf16) {   // float32 unmasked form: the per-chunk local kernels run
        if (!p.Lc) fail("unmasked float32 without chunk states", "Lc");
        if (!fwd && !p.Rc) fail("unmasked float32 without reverse chunk states", "Rc");
    }
    if (p.dOn) ex.push_back({U(p.dOn), (size_t)p.B * H * p.N * D * esz, "dOn"});
    check_extents(ex);
}

}  // namespace

namespace lasp {
hipError_t launch_fwd(const Params &p, bool bf16, bool, hipStream_t, hipEvent_t *) {
    check_params(p, true, bf16, false, false);
    return hipSuccess;
}
hipError_t launch_bwd(const Params &p, bool bf16, hipStream_t, hipEvent_t *) {
    check_params(p, false, bf16, false, false);
    return hipSuccess;
}
hipError_t launch_fwd_gated(const Params &p, bool bf16, bool, hipStream_t, hipEvent_t *) {
    check_params(p, true, bf16, true, false);
    return hipSuccess;
}
hipError_t launch_bwd_gated(const Params &p, bool bf16, hipStream_t, hipEvent_t *) {
    check_params(p, false, bf16, true, false);
    return hipSuccess;
}
hipError_t launch_setup(const Params &, hipStream_t) { return hipSuccess; }
hipError_t launch_norm_bwd_prep(const Params &p, bool, hipStream_t) {
    if (!p.Yn || !p.dYn || !p.rstd_in || !p.dOn) fail("norm preparation arguments", "dOn");
    return hipSuccess;
}
hipError_t static_scratch(hipStream_t, void **ptr) {
    *ptr = (void *)((uintptr_t)20 << 40);   // a fake device address for the static array
    return hipSuccess;
}
hipError_t launch_fwd_bidir(const Params &p, bool bf16, bool, hipStream_t, hipEvent_t *) {
    check_params(p, true, bf16, false, true);
    return hipSuccess;
}
hipError_t launch_bwd_bidir(const Params &p, bool bf16, hipStream_t, hipEvent_t *) {
    check_params(p, false, bf16, false, true);
    return hipSuccess;
}
}  // namespace lasp

// HIP runtime calls made by the ABI itself (debug path and error text)
const char *hipGetErrorString(hipError_t) { return "stubbed HIP error"; }
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t) {
    // the debug path copies cu_seqlens (int32) and decay (float32) to the host
    const std::vector<char> *from = nullptr;
    static std::vector<char> cu_b, dec_b;
    cu_b.assign((const char *)g_cu_host.data(), (const char *)(g_cu_host.data() + g_cu_host.size()));
    dec_b.assign((const char *)g_decay_host.data(),
                 (const char *)(g_decay_host.data() + g_decay_host.size()));
    if ((uintptr_t)src == 0x40000000u) from = &cu_b;
    else if ((uintptr_t)src == 0x50000000u) from = &dec_b;
    if (!from || from->size() < bytes) return hipErrorInvalidValue;
    memcpy(dst, from->data(), bytes);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace {

// fake device addresses: 1 TiB apart, 256-byte aligned
void *fake(int i) { return (void *)((uintptr_t)(i + 1) << 40); }
const void *CU = (const void *)(uintptr_t)0x40000000u;     // cu_seqlens (debug copies read it)
const void *DECAY = (const void *)(uintptr_t)0x50000000u;

int run_case(const lasp_shape &s, lasp_dtype dt, int form, int G, bool with_cache, bool decay) {
    lasp_sizes z;
    if (form == 3 && G) return LASP_OK;   // the normalised form has no segment knob
    int rc = lasp_query_sizes(&s, dt, form == 2 ? 0 : form == 3 ? 2 : form, G, &z);
    if (rc != LASP_OK) return rc;
    const size_t tens = (size_t)s.B * s.H * s.N * s.d * (dt == LASP_BF16 ? 2 : 4);
    const size_t nS = s.nseq ? s.nseq : s.B;
    const size_t st = nS * s.H * (size_t)s.d * s.d * 4;
    void *Q = fake(0), *K = fake(1), *V = fake(2), *dO = fake(3), *O = fake(4), *dQ = fake(5),
         *dK = fake(6), *dV = fake(7), *ws = fake(8), *cache = fake(9), *Min = fake(10),
         *Mout = fake(11), *dMout = fake(12), *dMin = fake(13), *LG = fake(14), *dLG = fake(15);
    const int32_t *cu = s.nseq ? (const int32_t *)CU : nullptr;
    const float *dec = decay ? (const float *)DECAY : nullptr;
    const size_t fw = z.fwd_workspace[with_cache], bw = z.bwd_workspace[with_cache];
    void *c = with_cache ? cache : nullptr;
    (void)tens;
    g_bufs = {{U(ws), fw, "fwd workspace"}, {U(cache), with_cache ? z.state_cache : 0, "cache"}};
    if (form == 3)
        rc = lasp_fwd_norm(&s, dt, Q, K, V, dec, cu, (float *)Min, O, (float *)fake(16),
                           (float *)Mout, c, ws, fw, nullptr);
    else if (form == 0)
        rc = lasp_fwd_ex(&s, dt, Q, K, V, dec, cu, (float *)Min, O, (float *)Mout, c, ws, fw, nullptr,
                         nullptr, G);
    else if (form == 1)
        rc = lasp_fwd_gated_ex(&s, dt, Q, K, V, (float *)LG, cu, (float *)Min, O, (float *)Mout, c,
                               ws, fw, nullptr, nullptr, G);
    else
        rc = lasp_fwd_bidir_ex(&s, dt, Q, K, V, cu, (float *)Min, O, (float *)Mout, c, ws, fw,
                               nullptr, nullptr, G);
    if (rc != LASP_OK) return rc;
    g_bufs = {{U(ws), bw, "bwd workspace"}, {U(cache), with_cache ? z.state_cache : 0, "cache"}};
    if (form == 3)
        rc = lasp_bwd_norm(&s, dt, Q, K, V, O, (const float *)fake(16), dO, dec, cu, (float *)Min,
                           (float *)dMout, c, dQ, dK, dV, (float *)dMin, ws, bw, nullptr);
    else if (form == 0)
        rc = lasp_bwd_ex(&s, dt, Q, K, V, dO, dec, cu, (float *)Min, (float *)dMout, c, dQ, dK, dV,
                         (float *)dMin, ws, bw, nullptr, nullptr, G);
    else if (form == 1)
        rc = lasp_bwd_gated_ex(&s, dt, Q, K, V, (float *)LG, dO, cu, (float *)Min, (float *)dMout,
                               c, dQ, dK, dV, (float *)dLG, (float *)dMin, ws, bw, nullptr, nullptr,
                               G);
    else
        rc = lasp_bwd_bidir_ex(&s, dt, Q, K, V, dO, cu, (float *)Min, (float *)dMout, c, dQ, dK,
                               dV, (float *)dMin, ws, bw, nullptr, nullptr, G);
    (void)st;
    return rc;
}

}  // namespace

int main() {
    int cases = 0;
    const lasp_shape shapes[] = {
        {1, 32, 131072, 128, 256, 0}, {4, 16, 8192, 128, 256, 0}, {2, 16, 32768, 128, 256, 0},
        {1, 32, 69632, 64, 128, 8},   {1, 2, 256, 32, 64, 0},     {3, 5, 1000, 64, 128, 0},
        {1, 4, 777, 32, 64, 5},       {1, 1, 1, 64, 64, 0},       {1, 3, 1, 128, 256, 1},
        {2, 64, 1 << 20, 128, 256, 0}, {1, 96, 1 << 21, 64, 64, 300}};
    for (const lasp_shape &s : shapes)
        for (int dti = 0; dti < 2; ++dti)
            for (int form = 0; form < 4; ++form)
                for (int G : {0, 1, 3, 64})
                    for (int wc = 0; wc < 2; ++wc)
                        for (int dec = 0; dec < 2; ++dec) {
                            const lasp_dtype dt = dti ? LASP_BF16 : LASP_FP32;
                            if (form != 0 && form != 3 && dec) continue;
                            const int rc = run_case(s, dt, form, G, wc, dec);
                            const bool expect_ok = true;
                            if (expect_ok != (rc == LASP_OK)) {
                                fprintf(stderr, "unexpected status %d: B%d H%d N%d d%d C%d nseq%d "
                                        "dt%d form%d G%d cache%d\n", rc, s.B, s.H, s.N, s.d,
                                        s.chunk, s.nseq, dti, form, G, wc);
                                ++g_failures;
                            }
                            ++cases;
                        }
    // allocation-free forward: the plan's arrays stay inside the static array;
    // a shape that needs more is refused before anything else happens
    for (const lasp_shape &s : shapes)
        for (int wc = 0; wc < 2; ++wc) {
            lasp_sizes z;
            if (lasp_query_sizes(&s, LASP_BF16, 0, 0, &z) != LASP_OK) continue;
            g_bufs = {{(uintptr_t)20 << 40, lasp_noalloc_scratch_bytes(), "static scratch"},
                      {U(fake(9)), wc ? z.state_cache : 0, "cache"}};
            const int rc = lasp_fwd_noalloc(&s, LASP_BF16, fake(0), fake(1), fake(2), nullptr,
                                            s.nseq ? (const int32_t *)CU : nullptr, nullptr,
                                            fake(4), nullptr, wc ? fake(9) : nullptr, nullptr);
            const bool fits = z.fwd_workspace[wc] <= lasp_noalloc_scratch_bytes();
            if (rc != (fits ? LASP_OK : LASP_ESCRATCH)) fail("noalloc status", "noalloc");
            ++cases;
        }
    // debug path: malformed cu_seqlens and decay are rejected, good ones pass
    setenv("LASP_DEBUG", "1", 1);
    const lasp_shape pk = {1, 2, 300, 64, 64, 3};
    g_decay_host = {0.5f, 1.0f};
    g_cu_host = {0, 100, 200, 300};
    if (run_case(pk, LASP_BF16, 0, 0, true, true) != LASP_OK) fail("debug: good input rejected", "cu");
    for (auto bad : {std::vector<int32_t>{1, 100, 200, 300}, std::vector<int32_t>{0, 200, 100, 300},
                     std::vector<int32_t>{0, 100, 200, 301}}) {
        g_cu_host = bad;
        if (run_case(pk, LASP_BF16, 0, 0, true, true) != LASP_EINVAL) fail("debug: bad cu accepted", "cu");
    }
    g_cu_host = {0, 100, 200, 300};
    for (auto bad : {std::vector<float>{-0.1f, 1.f}, std::vector<float>{0.5f, 1.5f},
                     std::vector<float>{0.5f, __builtin_nanf("")}}) {
        g_decay_host = bad;
        if (run_case(pk, LASP_BF16, 0, 0, true, true) != LASP_EINVAL)
            fail("debug: bad decay accepted", "decay");
    }
    unsetenv("LASP_DEBUG");
    if (g_failures) {
        fprintf(stderr, "%d failures\n", g_failures);
        return 1;
    }
    printf("ok %d cases, %d launches checked\n", cases, g_launches);
    return 0;
}
