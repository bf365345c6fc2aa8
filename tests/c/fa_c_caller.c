/*
 * fa_c_caller.c -- a plain C99 caller of the attention library's C ABI (include/fa_fwd.h):
 * device memory and copies through the HIP runtime API, one fa_fwd call, no C++ and no
 * Python.  Test infrastructure: tests/test_gpu_c_caller.py runs it and compares what it
 * writes with the fp64 oracle.
 *
 * Usage: fa_c_caller OUTPUT_FILE
 * The problem: B=1, Hq=4, Hkv=2, Sq=70, Skv=130, D=64, bf16, causal, input_pos=60,
 * scale=0.125.  Inputs: element n of tensor t (q=0, k=1, v=2) is hash(n, t) mapped to
 * [-1, 1) and rounded to bf16 (round to nearest even) -- a formula the test repeats.
 * Output file: out as raw bf16 bits (B*Hq*Sq*D uint16), then lse (B*Hq*Sq float32).
 * Exit status 0 on success; 1 on any HIP or library error (printed).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa_fwd.h"

enum { B = 1, HQ = 4, HKV = 2, SQ = 70, SKV = 130, D = 64, INPUT_POS = 60 };

static uint32_t mix(uint32_t n, uint32_t t) {
    uint32_t h = n * 2654435761u + t * 0x9E3779B9u;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    return h;
}

static uint16_t to_bf16(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    bits += 0x7FFFu + ((bits >> 16) & 1u);
    return (uint16_t)(bits >> 16);
}

static void fill(uint16_t* dst, size_t n, uint32_t t) {
    for (size_t i = 0; i < n; ++i)
        dst[i] = to_bf16((float)(mix((uint32_t)i, t) & 0xFFFFFFu) / 8388608.0f - 1.0f);
}

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
        return 1;
    }
    const size_t nq = (size_t)B * HQ * SQ * D, nk = (size_t)B * HKV * SKV * D, nl = (size_t)B * HQ * SQ;
    uint16_t* hq = malloc(nq * 2);
    uint16_t* hk = malloc(nk * 2);
    uint16_t* hv = malloc(nk * 2);
    uint16_t* ho = malloc(nq * 2);
    float* hl = malloc(nl * 4);
    if (!hq || !hk || !hv || !ho || !hl) return 1;
    fill(hq, nq, 0);
    fill(hk, nk, 1);
    fill(hv, nk, 2);

    void *q, *k, *v, *out;
    float* lse;
    HIP_OK(hipMalloc(&q, nq * 2));
    HIP_OK(hipMalloc(&k, nk * 2));
    HIP_OK(hipMalloc(&v, nk * 2));
    HIP_OK(hipMalloc(&out, nq * 2));
    HIP_OK(hipMalloc((void**)&lse, nl * 4));
    HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice));

    /* An invalid head dim is rejected on the host, before any launch. */
    int rc = fa_fwd(q, k, v, out, lse, B, HQ, HKV, SQ, SKV, 96, 0.125f, 1, INPUT_POS,
                    FA_DTYPE_BF16, NULL);
    if (rc != FA_ERR_UNSUPPORTED_HEAD_DIM) {
        fprintf(stderr, "expected FA_ERR_UNSUPPORTED_HEAD_DIM, got %d\n", rc);
        return 1;
    }
    printf("head dim 96: %d (%s)\n", rc, fa_strerror(rc));

    const int cfg = fa_select_config(B, HQ, HKV, SQ, SKV, D, 1, INPUT_POS, FA_DTYPE_BF16);
    printf("configuration %d: %s (of %d)\n", cfg, cfg >= 0 ? fa_config_name(cfg) : "?",
           fa_num_configs());
    rc = fa_fwd(q, k, v, out, lse, B, HQ, HKV, SQ, SKV, D, 0.125f, 1, INPUT_POS, FA_DTYPE_BF16,
                NULL);
    if (rc != FA_OK) {
        fprintf(stderr, "fa_fwd: %d (%s)\n", rc, fa_strerror(rc));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(ho, out, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, lse, nl * 4, hipMemcpyDeviceToHost));

    FILE* f = fopen(argv[1], "wb");
    if (!f || fwrite(ho, 2, nq, f) != nq || fwrite(hl, 4, nl, f) != nl || fclose(f) != 0) {
        fprintf(stderr, "cannot write %s\n", argv[1]);
        return 1;
    }
    HIP_OK(hipFree(q));
    HIP_OK(hipFree(k));
    HIP_OK(hipFree(v));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(lse));
    free(hq);
    free(hk);
    free(hv);
    free(ho);
    free(hl);
    printf("fa_fwd ok: %zu outputs written\n", nq + nl);
    return 0;
}
