/*
 * oracle_sanitize.c -- runs the CPU oracle on a problem read from a file, for
 * a build with the address and undefined-behaviour sanitizers (test
 * infrastructure; see test_oracle_sanitize.py).
 *
 * The oracle source is compiled into this program, so the sanitizer runtime
 * is linked into an executable of its own and every buffer below is a heap
 * block of exactly the size the oracle may touch: a read or write past any of
 * them, an uninitialised shift or an overflowing integer stops the program.
 *
 * Usage: oracle_sanitize <problem file> <result file>
 * Problem file (native byte order): int64 kind, then
 *   kind 0 (core):  int64 B Nv M D L Nq K; int64 shapes[2L], lsi[L];
 *                   double value[B Nv M D]; float loc[2P]; double attn[P];
 *                   double grad_out[B Nq M D]                  (P = B Nq M L K)
 *   kind 1 (fused): int64 B Nv M D L Nq K; int64 shapes[2L], lsi[L];
 *                   double value; float ref[B Nq L 2], off[2P], logits[P];
 *                   double grad_out
 *   kind 2 (DCNv3): int64 B H W G D kh kw sh sw ph pw dh dw Ho Wo;
 *                   double input[B H W G D]; float offset[2P]; double mask[P];
 *                   double grad_out[B Ho Wo G D]               (P = B Ho Wo G kh kw)
 * Result file: every output of the forward and the backward of that kind,
 * followed by their absolute term sums, as doubles, in argument order.
 */
#include "../oracle/msda_oracle.c"

#include <stdio.h>

static FILE *in_f, *out_f;

static void *take(size_t n, size_t elem) {
    void *p = malloc(n * elem > 0 ? n * elem : 1);
    if (!p) exit(2);
    if (n && fread(p, elem, n, in_f) != n) exit(3);
    return p;
}

static double *room(size_t n) {
    double *p = (double *)malloc(n > 0 ? n * sizeof(double) : 1);
    if (!p) exit(2);
    return p;
}

static void give(const double *p, size_t n) {
    if (n && fwrite(p, sizeof(double), n, out_f) != n) exit(4);
}

int main(int argc, char **argv) {
    if (argc != 3) return 1;
    in_f = fopen(argv[1], "rb");
    out_f = fopen(argv[2], "wb");
    if (!in_f || !out_f) return 1;
    int64_t kind;
    if (fread(&kind, sizeof kind, 1, in_f) != 1) return 3;
    int rc = 0;
    if (kind == 0 || kind == 1) {
        int64_t d[7];
        if (fread(d, sizeof(int64_t), 7, in_f) != 7) return 3;
        const int64_t B = d[0], Nv = d[1], M = d[2], D = d[3], L = d[4], Nq = d[5], K = d[6];
        const size_t P = (size_t)(B * Nq * M * L * K), T = (size_t)(B * Nq * M);
        const size_t nv = (size_t)(B * Nv * M * D), no = T * (size_t)D;
        int64_t *shapes = (int64_t *)take((size_t)(2 * L), sizeof(int64_t));
        int64_t *lsi = (int64_t *)take((size_t)L, sizeof(int64_t));
        double *value = (double *)take(nv, sizeof(double));
        if (kind == 0) {
            float *loc = (float *)take(2 * P, sizeof(float));
            double *attn = (double *)take(P, sizeof(double));
            double *g = (double *)take(no, sizeof(double));
            double *o = room(no), *oa = room(no), *gv = room(nv), *gva = room(nv);
            double *gl = room(2 * P), *gla = room(2 * P), *ga = room(P), *gaa = room(P);
            rc |= msda_oracle_forward(B, Nv, M, D, L, Nq, K, value, shapes, lsi, loc, attn, o, oa);
            rc |= msda_oracle_backward(B, Nv, M, D, L, Nq, K, value, shapes, lsi, loc, attn, g,
                                       gv, gl, ga, gva, gla, gaa);
            give(o, no); give(gv, nv); give(gl, 2 * P); give(ga, P);
            give(oa, no); give(gva, nv); give(gla, 2 * P); give(gaa, P);
            free(loc); free(attn); free(g); free(o); free(oa); free(gv); free(gva);
            free(gl); free(gla); free(ga); free(gaa);
        } else {
            const size_t nr = (size_t)(B * Nq * L * 2);
            float *ref = (float *)take(nr, sizeof(float));
            float *off = (float *)take(2 * P, sizeof(float));
            float *z = (float *)take(P, sizeof(float));
            double *g = (double *)take(no, sizeof(double));
            double *o = room(no), *oa = room(no), *gv = room(nv), *gva = room(nv);
            double *gr = room(nr), *gra = room(nr), *go = room(2 * P), *goa = room(2 * P);
            double *gz = room(P), *gza = room(P);
            rc |= msda_oracle_forward_fused(B, Nv, M, D, L, Nq, K, value, shapes, lsi, ref, off,
                                            z, o, oa);
            rc |= msda_oracle_backward_fused(B, Nv, M, D, L, Nq, K, value, shapes, lsi, ref, off,
                                             z, g, gv, gr, go, gz, gva, gra, goa, gza);
            give(o, no); give(gv, nv); give(gr, nr); give(go, 2 * P); give(gz, P);
            give(oa, no); give(gva, nv); give(gra, nr); give(goa, 2 * P); give(gza, P);
            free(ref); free(off); free(z); free(g); free(o); free(oa); free(gv); free(gva);
            free(gr); free(gra); free(go); free(goa); free(gz); free(gza);
        }
        free(shapes); free(lsi); free(value);
    } else if (kind == 2) {
        int64_t d[15];
        if (fread(d, sizeof(int64_t), 15, in_f) != 15) return 3;
        const int64_t B = d[0], H = d[1], W = d[2], G = d[3], D = d[4], kh = d[5], kw = d[6];
        const int64_t Ho = d[13], Wo = d[14];
        const size_t P = (size_t)(B * Ho * Wo * G * kh * kw);
        const size_t ni = (size_t)(B * H * W * G * D), no = (size_t)(B * Ho * Wo * G * D);
        double *x = (double *)take(ni, sizeof(double));
        float *off = (float *)take(2 * P, sizeof(float));
        double *mask = (double *)take(P, sizeof(double));
        double *g = (double *)take(no, sizeof(double));
        double *o = room(no), *oa = room(no), *gi = room(ni), *gia = room(ni);
        double *go = room(2 * P), *goa = room(2 * P), *gm = room(P), *gma = room(P);
        rc |= msda_oracle_dcn_forward(B, H, W, G, D, kh, kw, d[7], d[8], d[9], d[10], d[11],
                                      d[12], Ho, Wo, x, off, mask, o, oa);
        rc |= msda_oracle_dcn_backward(B, H, W, G, D, kh, kw, d[7], d[8], d[9], d[10], d[11],
                                       d[12], Ho, Wo, x, off, mask, g, gi, go, gm, gia, goa, gma);
        give(o, no); give(gi, ni); give(go, 2 * P); give(gm, P);
        give(oa, no); give(gia, ni); give(goa, 2 * P); give(gma, P);
        free(x); free(off); free(mask); free(g); free(o); free(oa); free(gi); free(gia);
        free(go); free(goa); free(gm); free(gma);
    } else {
        return 1;
    }
    fclose(in_f);
    fclose(out_f);
    return rc ? 5 : 0;
}
