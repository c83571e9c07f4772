/* A plain C caller of the C-ABI library, for the GPU test that checks the boundary from outside
 * Python: reads a bf16 pre-attention problem from raw files, runs dit_pre_attn_bf16 on a stream
 * of its own, and writes the workspace and the output back.  It also checks two error paths
 * (a non-positive eps, a NULL weight), which must return their status without launching.
 *
 * usage: pre_attn_caller <dir>; <dir> holds meta.txt ("M rows S eps qk_eps") and x.bin, xw.bin,
 * scale.bin, shift.bin, idx.bin, w.bin, qw.bin, kw.bin, cs.bin (row-major, bf16 as uint16,
 * indices int64); writes ws.bin and out.bin there.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dit.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void* p = malloc(bytes);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

#define HIP_OK(call)                                                                    \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) { fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_)); exit(3); } \
    } while (0)

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s <dir>\n", argv[0]); return 2; }
    const char* dir = argv[1];
    long long M, rows, S;
    float eps, qk_eps;
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/meta.txt", dir);
        FILE* f = fopen(path, "r");
        if (!f || fscanf(f, "%lld %lld %lld %f %f", &M, &rows, &S, &eps, &qk_eps) != 5) {
            fprintf(stderr, "bad meta.txt\n");
            return 2;
        }
        fclose(f);
    }
    const size_t H = DIT_HIDDEN, row_b = H * 2;
    const size_t out_b = (size_t)M * DIT_HEADS * 3 * DIT_HEAD_DIM * 2;
    void* x = to_device(read_file(dir, "x.bin", (size_t)M * row_b), (size_t)M * row_b);
    void* xw = to_device(read_file(dir, "xw.bin", row_b), row_b);
    void* sc = to_device(read_file(dir, "scale.bin", (size_t)rows * row_b), (size_t)rows * row_b);
    void* sh = to_device(read_file(dir, "shift.bin", (size_t)rows * row_b), (size_t)rows * row_b);
    void* idx = to_device(read_file(dir, "idx.bin", (size_t)M * 8), (size_t)M * 8);
    void* w = to_device(read_file(dir, "w.bin", (size_t)DIT_QKV_ROWS * row_b), (size_t)DIT_QKV_ROWS * row_b);
    void* qw = to_device(read_file(dir, "qw.bin", DIT_HEAD_DIM * 2), DIT_HEAD_DIM * 2);
    void* kw = to_device(read_file(dir, "kw.bin", DIT_HEAD_DIM * 2), DIT_HEAD_DIM * 2);
    void* cs = to_device(read_file(dir, "cs.bin", (size_t)S * DIT_ROPE_COLS * 2), (size_t)S * DIT_ROPE_COLS * 2);
    void *ws = NULL, *out = NULL;
    HIP_OK(hipMalloc(&ws, (size_t)M * row_b));
    HIP_OK(hipMalloc(&out, out_b));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const dit_bf16_table tsc = {sc, rows, (int64_t)H}, tsh = {sh, rows, (int64_t)H};

    /* error paths: reported, nothing launched */
    dit_status st = dit_pre_attn_bf16(x, M, xw, tsc, tsh, (const int64_t*)idx, w, qw, kw, cs, S, NULL, 1, -1.0f,
                                      qk_eps, ws, out, stream);
    if (st != DIT_ERR_VALUE) { fprintf(stderr, "eps -1: %s\n", dit_status_string(st)); return 4; }
    st = dit_pre_attn_bf16(x, M, xw, tsc, tsh, (const int64_t*)idx, NULL, qw, kw, cs, S, NULL, 1, eps, qk_eps, ws,
                           out, stream);
    if (st != DIT_ERR_NULL) { fprintf(stderr, "NULL weight: %s\n", dit_status_string(st)); return 4; }

    st = dit_pre_attn_bf16(x, M, xw, tsc, tsh, (const int64_t*)idx, w, qw, kw, cs, S, NULL, 1, eps, qk_eps, ws, out,
                           stream);
    if (st != DIT_OK) { fprintf(stderr, "dit_pre_attn_bf16: %s\n", dit_status_string(st)); return 4; }
    HIP_OK(hipStreamSynchronize(stream));
    void* h_ws = malloc((size_t)M * row_b);
    void* h_out = malloc(out_b);
    HIP_OK(hipMemcpy(h_ws, ws, (size_t)M * row_b, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_out, out, out_b, hipMemcpyDeviceToHost));
    write_file(dir, "ws.bin", h_ws, (size_t)M * row_b);
    write_file(dir, "out.bin", h_out, out_b);
    HIP_OK(hipStreamDestroy(stream));
    printf("ok\n");
    return 0;
}
