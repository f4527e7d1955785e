/*
 * A plain C consumer of libdca (no C++, no Python, no torch): it builds a
 * small bf16 problem from a counter-based generator, sizes and allocates the
 * workspace, runs dca_prefill on the null stream, checks one rejected call,
 * and writes out and lse to a file for the GPU test to compare with the
 * Python binding's result on the same inputs.
 *
 *     c_abi_example OUTPUT_FILE
 *
 * Compiled by position_extrapolation_amd/build.py with gcc against
 * include/dca.h and the HIP runtime.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dca.h"

enum { B = 1, HQ = 4, HKV = 2, D = 128, S = 3000, C = 1024, W = 128 };

/* splitmix64 of seed + i: a value in [-0.5, 0.5) with 24 random bits */
static float input_value(uint64_t seed, uint64_t i) {
    uint64_t z = seed + i * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)(z >> 40) * (1.0f / 16777216.0f) - 0.5f;
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int fail(const char *what, int status) {
    fprintf(stderr, "%s: %s (%s)\n", what, dca_status_str(status), dca_last_error());
    return 1;
}

#define HIP_CHECK(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
            return 1;                                                                \
        }                                                                            \
    } while (0)

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
        return 2;
    }
    const size_t nq = (size_t)B * HQ * S * D, nk = (size_t)B * HKV * S * D, nl = (size_t)B * HQ * S;
    uint16_t *hq = malloc(nq * 2), *hk = malloc(nk * 2), *hv = malloc(nk * 2), *ho = malloc(nq * 2);
    float *hl = malloc(nl * 4);
    if (!hq || !hk || !hv || !ho || !hl) return 1;
    for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16(input_value(1, i));
    for (size_t i = 0; i < nk; ++i) hk[i] = to_bf16(input_value(2, i));
    for (size_t i = 0; i < nk; ++i) hv[i] = to_bf16(input_value(3, i));

    void *q, *k, *v, *out, *ws;
    float *lse;
    HIP_CHECK(hipMalloc(&q, nq * 2));
    HIP_CHECK(hipMalloc(&k, nk * 2));
    HIP_CHECK(hipMalloc(&v, nk * 2));
    HIP_CHECK(hipMalloc(&out, nq * 2));
    HIP_CHECK(hipMalloc((void **)&lse, nl * 4));
    HIP_CHECK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice));

    const dca_shape shape = {B, HQ, HKV, D, DCA_BF16, 0.0f};
    const double rope_base = 1e7;
    const float yarn = (float)(0.1 * log((double)S / C) + 1.0);
    size_t bytes = 0;
    int st = dca_workspace_size(S, C, W, &shape, NULL, &bytes);
    if (st != DCA_OK) return fail("dca_workspace_size", st);
    HIP_CHECK(hipMalloc(&ws, bytes));

    /* a workspace one byte short is rejected before anything is enqueued */
    st = dca_prefill(q, k, v, out, lse, S, C, W, rope_base, yarn, NULL, &shape, ws, bytes - 1, NULL);
    if (st != DCA_E_WORKSPACE || dca_last_error()[0] == '\0') {
        fprintf(stderr, "short workspace: expected DCA_E_WORKSPACE, got %d\n", st);
        return 1;
    }
    st = dca_prefill(q, k, v, out, lse, S, C, W, rope_base, yarn, NULL, &shape, ws, bytes, NULL);
    if (st != DCA_OK) return fail("dca_prefill", st);
    HIP_CHECK(hipDeviceSynchronize());
    HIP_CHECK(hipMemcpy(ho, out, nq * 2, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(hl, lse, nl * 4, hipMemcpyDeviceToHost));

    FILE *f = fopen(argv[1], "wb");
    if (!f || fwrite(ho, 2, nq, f) != nq || fwrite(hl, 4, nl, f) != nl || fclose(f) != 0) {
        fprintf(stderr, "cannot write %s\n", argv[1]);
        return 1;
    }
    printf("c_abi_example: dca_prefill bf16 S=%d C=%d W=%d, workspace %zu bytes: ok\n", S, C, W, bytes);
    hipFree(q); hipFree(k); hipFree(v); hipFree(out); hipFree(lse); hipFree(ws);
    free(hq); free(hk); free(hv); free(ho); free(hl);
    return 0;
}
