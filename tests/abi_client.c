/*
 * A plain C99 client of the C ABI (include/msda.h), with no PyTorch: it
 * reads one problem from files, allocates device memory with the HIP
 * runtime, runs msda_forward and msda_backward on the default stream and
 * writes the results back. tests/test_gpu_abi_client.py drives it and checks
 * the results against the CPU oracle.
 *
 *   abi_client DIR     DIR holds dims.txt ("B Nv M D L Nq K"), value.bin
 *                      (f32 [B,Nv,M,D]), shapes.bin and lsi.bin (int64),
 *                      loc.bin, attn.bin and gout.bin (f32); the client
 *                      writes out.bin, gvalue.bin, gloc.bin and gattn.bin.
 *   abi_client         prints msda_version() and exits (no GPU call).
 *
 * Exit status 0 on success; otherwise the failing call is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "msda.h"

static int fail_hip(hipError_t e, const char *what) {
    fprintf(stderr, "abi_client: %s: %s\n", what, hipGetErrorString(e));
    return 1;
}

static int fail_msda(msda_status_t s, const char *what) {
    fprintf(stderr, "abi_client: %s: %s\n", what, msda_status_string(s));
    return 1;
}

/* n bytes of DIR/name into a fresh host buffer (NULL on a short read) */
static void *read_file(const char *dir, const char *name, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *p = malloc(n ? n : 1);
    if (p && fread(p, 1, n, f) != n) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int write_file(const char *dir, const char *name, const void *p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 1;
    const int bad = fwrite(p, 1, n, f) != n;
    return fclose(f) != 0 || bad;
}

/* device copy of a host buffer */
static hipError_t upload(void **dev, const void *host, size_t n) {
    hipError_t e = hipMalloc(dev, n ? n : 1);
    if (e == hipSuccess && n) e = hipMemcpy(*dev, host, n, hipMemcpyHostToDevice);
    return e;
}

int main(int argc, char **argv) {
    if (argc < 2) {
        printf("%d\n", msda_version());
        return 0;
    }
    const char *dir = argv[1];
    msda_dims_t d;
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/dims.txt", dir);
        FILE *f = fopen(path, "r");
        long long v[7];
        if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld %lld", &v[0], &v[1], &v[2], &v[3],
                         &v[4], &v[5], &v[6]) != 7) {
            fprintf(stderr, "abi_client: cannot read %s\n", path);
            return 1;
        }
        fclose(f);
        d.B = v[0], d.Nv = v[1], d.M = v[2], d.D = v[3], d.L = v[4], d.Nq = v[5], d.K = v[6];
    }
    const size_t n_value = (size_t)(d.B * d.Nv * d.M * d.D);
    const size_t n_pts = (size_t)(d.B * d.Nq * d.M * d.L * d.K);
    const size_t n_out = (size_t)(d.B * d.Nq * d.M * d.D);
    const size_t f4 = sizeof(float), i8 = sizeof(int64_t);

    void *h_value = read_file(dir, "value.bin", n_value * f4);
    void *h_shapes = read_file(dir, "shapes.bin", (size_t)d.L * 2 * i8);
    void *h_lsi = read_file(dir, "lsi.bin", (size_t)d.L * i8);
    void *h_loc = read_file(dir, "loc.bin", n_pts * 2 * f4);
    void *h_attn = read_file(dir, "attn.bin", n_pts * f4);
    void *h_gout = read_file(dir, "gout.bin", n_out * f4);
    if (!h_value || !h_shapes || !h_lsi || !h_loc || !h_attn || !h_gout) {
        fprintf(stderr, "abi_client: missing or short input file in %s\n", dir);
        return 1;
    }

    /* the library checks the level tables only on the host side, on request */
    msda_status_t s = msda_check_tables((const int64_t *)h_shapes, (const int64_t *)h_lsi, d.L,
                                        d.Nv);
    if (s != MSDA_SUCCESS) return fail_msda(s, "msda_check_tables");

    void *value, *shapes, *lsi, *loc, *attn, *gout, *out, *gvalue, *gloc, *gattn, *ws = NULL;
    hipError_t e;
    if ((e = upload(&value, h_value, n_value * f4)) != hipSuccess ||
        (e = upload(&shapes, h_shapes, (size_t)d.L * 2 * i8)) != hipSuccess ||
        (e = upload(&lsi, h_lsi, (size_t)d.L * i8)) != hipSuccess ||
        (e = upload(&loc, h_loc, n_pts * 2 * f4)) != hipSuccess ||
        (e = upload(&attn, h_attn, n_pts * f4)) != hipSuccess ||
        (e = upload(&gout, h_gout, n_out * f4)) != hipSuccess ||
        (e = hipMalloc(&out, n_out * f4 + 1)) != hipSuccess ||
        (e = hipMalloc(&gvalue, n_value * f4 + 1)) != hipSuccess ||
        (e = hipMalloc(&gloc, n_pts * 2 * f4 + 1)) != hipSuccess ||
        (e = hipMalloc(&gattn, n_pts * f4 + 1)) != hipSuccess)
        return fail_hip(e, "device buffers");

    s = msda_forward(&d, MSDA_DTYPE_F32, value, (const int64_t *)shapes, (const int64_t *)lsi,
                     (const float *)loc, (const float *)attn, (float *)out, NULL);
    if (s != MSDA_SUCCESS) return fail_msda(s, "msda_forward");

    size_t ws_bytes = 0;
    s = msda_backward_workspace_size(&d, MSDA_DTYPE_F32, &ws_bytes);
    if (s != MSDA_SUCCESS) return fail_msda(s, "msda_backward_workspace_size");
    if (ws_bytes && (e = hipMalloc(&ws, ws_bytes)) != hipSuccess)
        return fail_hip(e, "workspace");
    s = msda_backward(&d, MSDA_DTYPE_F32, value, (const int64_t *)shapes, (const int64_t *)lsi,
                      (const float *)loc, (const float *)attn, (const float *)gout,
                      (float *)gvalue, (float *)gloc, (float *)gattn, ws, ws_bytes, NULL);
    if (s != MSDA_SUCCESS) return fail_msda(s, "msda_backward");
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");

    void *h = malloc((n_value > 2 * n_pts ? n_value : 2 * n_pts) * f4 + n_out * f4 + 1);
    if (!h) return 1;
    struct {
        const char *name;
        void *dev;
        size_t bytes;
    } outs[4] = {{"out.bin", out, n_out * f4},
                 {"gvalue.bin", gvalue, n_value * f4},
                 {"gloc.bin", gloc, n_pts * 2 * f4},
                 {"gattn.bin", gattn, n_pts * f4}};
    for (int i = 0; i < 4; ++i) {
        if (outs[i].bytes &&
            (e = hipMemcpy(h, outs[i].dev, outs[i].bytes, hipMemcpyDeviceToHost)) != hipSuccess)
            return fail_hip(e, outs[i].name);
        if (write_file(dir, outs[i].name, h, outs[i].bytes)) {
            fprintf(stderr, "abi_client: cannot write %s\n", outs[i].name);
            return 1;
        }
    }
    printf("abi_client: ok (version %d, workspace %zu bytes)\n", msda_version(), ws_bytes);
    return 0;
}
