/*
 * A C program that uses librmsq through include/rmsq.h alone (no Python, no
 * torch): it shows the boundary is plain C and checks it from C.
 *
 *   rmsq_c_check errors          argument errors only; no GPU work.  Prints
 *                                "errors ok" when every call returns the
 *                                status include/rmsq.h documents.
 *   rmsq_c_check run IN OUT      reads rows, hidden, x, residual, gamma (bf16
 *                                bits) and a global scale from IN, runs
 *                                residual_rmsnorm_fp8 (e4m3fn, fp32 scales),
 *                                rmsnorm_fp8 (e4m3fnuz, bf16 scales) and
 *                                rmsnorm_fp4 on a stream of its own, and
 *                                writes every output to OUT.
 *
 * IN : int64 rows, int64 hidden, uint16 x[rows*hidden], uint16 r[rows*hidden],
 *      uint16 gamma[hidden], float global_scale.
 * OUT: uint8 codes[rows*hidden], float scales[rows], uint16 residual_out
 *      [rows*hidden], uint8 codes_fnuz[rows*hidden], uint16 scales_bf16[rows],
 *      uint8 fp4[rows*hidden/2], uint8 fp4_scales[rows*hidden/16].
 * All little-endian, back to back.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rmsq.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d (%s)\n", what, got, rmsq_status_string(got), want,
                rmsq_status_string(want));
        ++failures;
    }
}

/* Fake device addresses: these calls fail their checks before any HIP call,
 * so nothing is dereferenced.  As a second guard, a forced launch shape (one
 * wave, one vector per lane: 512 16-bit elements) cannot hold these
 * 1024-element rows, so a call that passed every check would return
 * RMSQ_ERR_UNSUPPORTED rather than launch. */
static int errors(void) {
    expect("forced shape", rmsq_set_tuning(1, 1, 0), RMSQ_OK);
    void* const a = (void*)(uintptr_t)0x100000000ull;
    void* const b = (void*)(uintptr_t)0x200000000ull;
    void* const c = (void*)(uintptr_t)0x300000000ull;
    void* const d = (void*)(uintptr_t)0x400000000ull;
    void* const e = (void*)(uintptr_t)0x500000000ull;
    void* const f = (void*)(uintptr_t)0x600000000ull;
    expect("abi version", rmsq_abi_version(), RMSQ_ABI_VERSION);
    expect("null x", rmsnorm_fp8(4, 1024, RMSQ_BF16, NULL, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32, d, NULL),
           RMSQ_ERR_NULL);
    expect("bad dtype", rmsnorm_fp8(4, 1024, 7, a, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32, d, NULL),
           RMSQ_ERR_DTYPE);
    expect("bad format", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 1200.0f, 9, c, RMSQ_F32, d, NULL),
           RMSQ_ERR_DTYPE);
    expect("negative rows", rmsnorm_fp8(-1, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32, d,
                                        NULL),
           RMSQ_ERR_SHAPE);
    expect("negative eps", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, -1.0f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32, d,
                                       NULL),
           RMSQ_ERR_VALUE);
    expect("zero scale_ub", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 0.0f, RMSQ_E4M3FN, c, RMSQ_F32, d,
                                        NULL),
           RMSQ_ERR_VALUE);
    expect("misaligned scales", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32,
                                            (char*)d + 2, NULL),
           RMSQ_ERR_ALIGN);
    expect("codes over x", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, (char*)a + 16,
                                       RMSQ_F32, d, NULL),
           RMSQ_ERR_ALIAS);
    expect("zero rows", rmsnorm_fp8(0, 1024, RMSQ_BF16, NULL, NULL, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, NULL, RMSQ_F32,
                                    NULL, NULL),
           RMSQ_OK);
    expect("residual_out over gamma",
           residual_rmsnorm_fp8(4, 1024, RMSQ_BF16, a, e, b, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32, d,
                                NULL),
           RMSQ_ERR_ALIAS);
    expect("fp4 hidden not a multiple of 16",
           rmsnorm_fp4(4, 1000, RMSQ_BF16, a, b, 1e-6f, 0.0f, NULL, (uint8_t*)c, (uint8_t*)d, NULL), RMSQ_ERR_SHAPE);
    expect("fp4 unknown dtype", rmsnorm_fp4(4, 1024, 5, a, b, 1e-6f, 0.0f, NULL, (uint8_t*)c, (uint8_t*)d, NULL),
           RMSQ_ERR_DTYPE);
    expect("all checks passed", rmsnorm_fp8(4, 1024, RMSQ_BF16, a, b, 1e-6f, 0.0f, 1200.0f, RMSQ_E4M3FN, c, RMSQ_F32,
                                            d, NULL),
           RMSQ_ERR_UNSUPPORTED);
    expect("fp4 misaligned x", rmsnorm_fp4(4, 1024, RMSQ_BF16, (char*)a + 8, b, 1e-6f, 0.0f, NULL, (uint8_t*)c,
                                           (uint8_t*)f, NULL),
           RMSQ_ERR_ALIGN);
    if (strcmp(rmsq_status_string(RMSQ_OK), "ok") != 0) {
        fprintf(stderr, "status string of RMSQ_OK\n");
        ++failures;
    }
    expect("automatic shape", rmsq_set_tuning(0, 0, 0), RMSQ_OK);
    if (failures) return 1;
    printf("errors ok\n");
    return 0;
}

#define HIP_CHECK(call)                                                                  \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            exit(1);                                                                     \
        }                                                                                \
    } while (0)

#define RMSQ_CHECK(call)                                                                 \
    do {                                                                                 \
        int s_ = (call);                                                                 \
        if (s_ != RMSQ_OK) {                                                             \
            fprintf(stderr, "%s returned %d (%s), hip error %d\n", #call, s_,            \
                    rmsq_status_string(s_), rmsq_last_hip_error());                      \
            exit(1);                                                                     \
        }                                                                                \
    } while (0)

static void* read_exact(FILE* fp, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, fp) != bytes) {
        fprintf(stderr, "short input file\n");
        exit(1);
    }
    return p;
}

static void* to_device(const void* h, size_t bytes) {
    void* d = NULL;
    HIP_CHECK(hipMalloc(&d, bytes));
    HIP_CHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void* device_buffer(size_t bytes) {
    void* d = NULL;
    HIP_CHECK(hipMalloc(&d, bytes));
    return d;
}

static void write_back(FILE* fp, const void* d, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) exit(1);
    HIP_CHECK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, bytes, fp) != bytes) {
        fprintf(stderr, "write failed\n");
        exit(1);
    }
    free(h);
}

static int run(const char* in_path, const char* out_path) {
    FILE* fp = fopen(in_path, "rb");
    if (!fp) {
        fprintf(stderr, "cannot open %s\n", in_path);
        return 1;
    }
    int64_t dims[2];
    if (fread(dims, sizeof(int64_t), 2, fp) != 2) {
        fprintf(stderr, "short input file\n");
        return 1;
    }
    const int64_t rows = dims[0], hidden = dims[1], n = rows * hidden;
    if (rows <= 0 || hidden <= 0 || hidden % 16 != 0) {
        fprintf(stderr, "bad shape\n");
        return 1;
    }
    void* hx = read_exact(fp, (size_t)n * 2);
    void* hr = read_exact(fp, (size_t)n * 2);
    void* hg = read_exact(fp, (size_t)hidden * 2);
    float* hgs = (float*)read_exact(fp, sizeof(float));
    fclose(fp);

    void* x = to_device(hx, (size_t)n * 2);
    void* r = to_device(hr, (size_t)n * 2);
    void* g = to_device(hg, (size_t)hidden * 2);
    float* gs = (float*)to_device(hgs, sizeof(float));
    void* codes = device_buffer((size_t)n);
    void* scales = device_buffer((size_t)rows * 4);
    void* ro = device_buffer((size_t)n * 2);
    void* codes2 = device_buffer((size_t)n);
    void* scales2 = device_buffer((size_t)rows * 2);
    void* fp4 = device_buffer((size_t)n / 2);
    void* fp4s = device_buffer((size_t)n / 16);

    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    RMSQ_CHECK(residual_rmsnorm_fp8(rows, hidden, RMSQ_BF16, x, r, ro, g, 1e-5f, 0.0f, 1200.0f, RMSQ_E4M3FN, codes,
                                    RMSQ_F32, scales, stream));
    RMSQ_CHECK(rmsnorm_fp8(rows, hidden, RMSQ_BF16, x, g, 1e-6f, 1.0f, 1e4f, RMSQ_E4M3FNUZ, codes2, RMSQ_BF16, scales2,
                           stream));
    RMSQ_CHECK(rmsnorm_fp4(rows, hidden, RMSQ_BF16, x, g, 1e-6f, 0.0f, gs, (uint8_t*)fp4, (uint8_t*)fp4s, stream));
    HIP_CHECK(hipStreamSynchronize(stream));
    HIP_CHECK(hipStreamDestroy(stream));

    FILE* out = fopen(out_path, "wb");
    if (!out) {
        fprintf(stderr, "cannot open %s\n", out_path);
        return 1;
    }
    write_back(out, codes, (size_t)n);
    write_back(out, scales, (size_t)rows * 4);
    write_back(out, ro, (size_t)n * 2);
    write_back(out, codes2, (size_t)n);
    write_back(out, scales2, (size_t)rows * 2);
    write_back(out, fp4, (size_t)n / 2);
    write_back(out, fp4s, (size_t)n / 16);
    fclose(out);

    void* bufs[] = {x, r, g, gs, codes, scales, ro, codes2, scales2, fp4, fp4s};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_CHECK(hipFree(bufs[i]));
    free(hx);
    free(hr);
    free(hg);
    free(hgs);
    printf("run ok\n");
    return 0;
}

int main(int argc, char** argv) {
    if (argc == 2 && strcmp(argv[1], "errors") == 0) return errors();
    if (argc == 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
    fprintf(stderr, "usage: %s errors | run IN OUT\n", argv[0]);
    return 2;
}
