/*
 * head_consumer.c -- a plain C consumer of libdust's C ABI (test
 * infrastructure): it reads an LM-head problem from a file, runs
 * dust_head_estimate on device memory it allocates with the HIP runtime, and
 * writes g_hat and G_W back.  No C++, no Python, no torch: what a C caller of
 * include/dust.h does.
 *
 * Usage: head_consumer <input> <output>
 * Input (native byte order): int64 T, V, d, seq_len, K; float sigma, gamma;
 * uint64 seed; uint32 stream; int32 logits_dtype (DUST_F32 or DUST_BF16) and
 * x_dtype; then logits [T][V] (4 or 2 bytes each), int32 targets [T],
 * X [T][d] (4 or 2 bytes each).
 * Output: float g_hat [T][V], then float G_W [V][d].
 * Exit status 0 on success; otherwise the failing step is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dust.h"

static int fail(const char* what) {
    fprintf(stderr, "head_consumer: %s\n", what);
    return 1;
}

#define READ(ptr, size, n)                                   \
    do {                                                     \
        if (fread((ptr), (size), (size_t)(n), in) != (size_t)(n)) \
            return fail("short input file");                 \
    } while (0)

#define HIP_OK(call)                                         \
    do {                                                     \
        if ((call) != hipSuccess) return fail(#call);        \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 3) return fail("usage: head_consumer <input> <output>");
    FILE* in = fopen(argv[1], "rb");
    if (!in) return fail("cannot open the input");
    int64_t T, V, d, seq_len, K;
    float sigma, gamma;
    uint64_t seed;
    uint32_t stream;
    int32_t zdt, xdt;
    READ(&T, 8, 1); READ(&V, 8, 1); READ(&d, 8, 1); READ(&seq_len, 8, 1); READ(&K, 8, 1);
    READ(&sigma, 4, 1); READ(&gamma, 4, 1); READ(&seed, 8, 1); READ(&stream, 4, 1);
    READ(&zdt, 4, 1); READ(&xdt, 4, 1);
    if (T <= 0 || V <= 0 || d <= 0 || T > (1 << 20) || V > DUST_N_MAX || d > (1 << 16))
        return fail("sizes out of this consumer's range");
    const size_t zes = zdt == DUST_BF16 ? 2 : 4, xes = xdt == DUST_BF16 ? 2 : 4;
    const size_t zbytes = (size_t)T * (size_t)V * zes, xbytes = (size_t)T * (size_t)d * xes;
    void* hz = malloc(zbytes);
    int32_t* hy = (int32_t*)malloc((size_t)T * 4);
    void* hx = malloc(xbytes);
    float* hg = (float*)malloc((size_t)T * (size_t)V * 4);
    float* hG = (float*)malloc((size_t)V * (size_t)d * 4);
    if (!hz || !hy || !hx || !hg || !hG) return fail("host allocation");
    READ(hz, 1, zbytes);
    READ(hy, 4, T);
    READ(hx, 1, xbytes);
    fclose(in);

    void *dz, *dx, *dws;
    int32_t* dy;
    float *dg, *dG;
    const size_t ws = dust_head_workspace_size(T, V, d, K, gamma);
    HIP_OK(hipMalloc(&dz, zbytes));
    HIP_OK(hipMalloc((void**)&dy, (size_t)T * 4));
    HIP_OK(hipMalloc(&dx, xbytes));
    HIP_OK(hipMalloc((void**)&dg, (size_t)T * (size_t)V * 4));
    HIP_OK(hipMalloc((void**)&dG, (size_t)V * (size_t)d * 4));
    HIP_OK(hipMalloc(&dws, ws));
    HIP_OK(hipMemcpy(dz, hz, zbytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy, hy, (size_t)T * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dx, hx, xbytes, hipMemcpyHostToDevice));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    const dust_status st = dust_head_estimate(dz, (dust_dtype)zdt, dy, dx, (dust_dtype)xdt, T, V, d,
                                              seq_len, sigma, K, gamma, seed, stream, dg, dG,
                                              NULL, dws, ws, (dust_stream_t)s, NULL);
    if (st != DUST_OK) {
        fprintf(stderr, "head_consumer: dust_head_estimate: %s\n", dust_status_string(st));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(hg, dg, (size_t)T * (size_t)V * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hG, dG, (size_t)V * (size_t)d * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipFree(dz)); HIP_OK(hipFree(dy)); HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dg)); HIP_OK(hipFree(dG)); HIP_OK(hipFree(dws));

    FILE* out = fopen(argv[2], "wb");
    if (!out) return fail("cannot open the output");
    if (fwrite(hg, 4, (size_t)T * (size_t)V, out) != (size_t)T * (size_t)V ||
        fwrite(hG, 4, (size_t)V * (size_t)d, out) != (size_t)V * (size_t)d)
        return fail("short write");
    fclose(out);
    free(hz); free(hy); free(hx); free(hg); free(hG);
    printf("head_consumer: %s, T=%lld V=%lld d=%lld K=%lld: ok\n", dust_version(), (long long)T,
           (long long)V, (long long)d, (long long)K);
    return 0;
}
