/*
 * Runs the C float64 oracle (oracle/crecurrent.c, compiled in) on inputs read
 * from a file and writes every output to another, so that a sanitizer build
 * (AddressSanitizer + UndefinedBehaviorSanitizer, tests/test_host_sanitizers.py)
 * exercises it on ragged packed sequences, decay, M_in and dM_out.
 *
 * Input file (little-endian): int32 n, d, rows, do_bwd; int64 row_off[n],
 * len[n]; float64 lam[n]; float32 Q, K, V, dO [rows * d]; float64 m_in[n d d],
 * dm_out[n d d].  Output file: float64 O, dQ, dK, dV [rows * d], m_out[n d d],
 * dm_in[n d d].  Exit status 0 on success.
 */
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/crecurrent.c"

static void *rd(FILE *f, size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p || fread(p, 1, n, f) != n) {
        fprintf(stderr, "short read\n");
        exit(2);
    }
    return p;
}

int main(int argc, char **argv) {
    if (argc != 3) return 2;
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 2;
    int32_t hdr[4];
    if (fread(hdr, 4, 4, f) != 4) return 2;
    const int n = hdr[0], d = hdr[1], rows = hdr[2], bwd = hdr[3];
    const size_t dd = (size_t)d * d, rd_ = (size_t)rows * d;
    int64_t *off = rd(f, 8 * (size_t)n), *len = rd(f, 8 * (size_t)n);
    double *lam = rd(f, 8 * (size_t)n);
    float *Q = rd(f, 4 * rd_), *K = rd(f, 4 * rd_), *V = rd(f, 4 * rd_), *dO = rd(f, 4 * rd_);
    double *mi = rd(f, 8 * n * dd), *dmo = rd(f, 8 * n * dd);
    fclose(f);
    double *O = calloc(rd_ ? rd_ : 1, 8), *dQ = calloc(rd_ ? rd_ : 1, 8);
    double *dK = calloc(rd_ ? rd_ : 1, 8), *dV = calloc(rd_ ? rd_ : 1, 8);
    double *mo = calloc(n * dd ? n * dd : 1, 8), *dmi = calloc(n * dd ? n * dd : 1, 8);
    if (lasp_ref_run(n, off, len, lam, d, Q, K, V, dO, mi, dmo, O, mo, dQ, dK, dV, dmi, bwd))
        return 3;
    FILE *g = fopen(argv[2], "wb");
    if (!g) return 2;
    fwrite(O, 8, rd_, g);
    fwrite(dQ, 8, rd_, g);
    fwrite(dK, 8, rd_, g);
    fwrite(dV, 8, rd_, g);
    fwrite(mo, 8, n * dd, g);
    fwrite(dmi, 8, n * dd, g);
    fclose(g);
    free(off); free(len); free(lam); free(Q); free(K); free(V); free(dO); free(mi); free(dmo);
    free(O); free(dQ); free(dK); free(dV); free(mo); free(dmi);
    return 0;
}
