/* Native caller of libmuon_rocm: one optimizer step on one matrix with device memory
 * from hipMalloc, no Python or torch. Used by the GPU tests to check the C ABI from a
 * native program against the float64 oracle.
 *
 * usage: muon_c_driver IN OUT
 *   IN:  int64 rows, cols, step, period_k, entry (0 = muon_step, 1 = rownorm_update),
 *        then W, M, G as rows * cols fp32 each
 *   OUT: W, M after the step (fp32), then the float update_rms monitor value
 * Exit status: 0 on success, otherwise the library status (negated) or 100+ for I/O. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "muon_rocm.h"

static int check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 100;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 101;
    int64_t hdr[5];
    if (fread(hdr, sizeof(int64_t), 5, in) != 5) return 102;
    const int64_t rows = hdr[0], cols = hdr[1], step = hdr[2], period_k = hdr[3], entry = hdr[4];
    const size_t n = (size_t)rows * (size_t)cols, bytes = n * sizeof(float);
    float* host = (float*)malloc(3 * bytes + sizeof(float));
    if (!host || fread(host, sizeof(float), 3 * n, in) != 3 * n) return 103;
    fclose(in);

    float *w = NULL, *m = NULL, *g = NULL, *rms = NULL;
    void* ws = NULL;
    size_t ws_bytes = 0;
    if (muon_workspace_bytes(&rows, &cols, 1, &ws_bytes) != MUON_OK) return 104;
    if (check_hip(hipMalloc((void**)&w, bytes), "hipMalloc w") || check_hip(hipMalloc((void**)&m, bytes), "hipMalloc m") ||
        check_hip(hipMalloc((void**)&g, bytes), "hipMalloc g") || check_hip(hipMalloc((void**)&rms, sizeof(float)), "hipMalloc rms") ||
        check_hip(hipMalloc(&ws, ws_bytes ? ws_bytes : 256), "hipMalloc workspace"))
        return 105;
    if (check_hip(hipMemcpy(w, host, bytes, hipMemcpyHostToDevice), "copy w") ||
        check_hip(hipMemcpy(m, host + n, bytes, hipMemcpyHostToDevice), "copy m") ||
        check_hip(hipMemcpy(g, host + 2 * n, bytes, hipMemcpyHostToDevice), "copy g"))
        return 106;

    muon_hparams hp;
    muon_default_hparams(&hp);
    hp.period_k = (int32_t)period_k;
    muon_matrix mat;
    mat.rows = rows;
    mat.cols = cols;
    mat.w = w;
    mat.m = m;
    mat.g = g;
    hipStream_t stream = NULL;
    if (check_hip(hipStreamCreate(&stream), "hipStreamCreate")) return 107;
    const int rc = entry == 0 ? muon_step(&mat, 1, &hp, step, ws, ws_bytes, rms, stream)
                              : rownorm_update(&mat, 1, &hp, ws, ws_bytes, rms, stream);
    if (rc != MUON_OK) {
        fprintf(stderr, "status %d: %s (%s)\n", rc, muon_status_str(rc), muon_last_error());
        return -rc;
    }
    if (check_hip(hipStreamSynchronize(stream), "sync")) return 108;
    if (check_hip(hipMemcpy(host, w, bytes, hipMemcpyDeviceToHost), "copy back w") ||
        check_hip(hipMemcpy(host + n, m, bytes, hipMemcpyDeviceToHost), "copy back m") ||
        check_hip(hipMemcpy(host + 2 * n, rms, sizeof(float), hipMemcpyDeviceToHost), "copy back rms"))
        return 109;
    FILE* out = fopen(argv[2], "wb");
    if (!out || fwrite(host, sizeof(float), 2 * n + 1, out) != 2 * n + 1) return 110;
    fclose(out);
    (void)hipStreamDestroy(stream);
    (void)hipFree(w);
    (void)hipFree(m);
    (void)hipFree(g);
    (void)hipFree(rms);
    (void)hipFree(ws);
    free(host);
    printf("muon_c_driver: %s step %lld on [%lld, %lld] ok\n", entry == 0 ? "muon_step" : "rownorm_update",
           (long long)step, (long long)rows, (long long)cols);
    return 0;
}
