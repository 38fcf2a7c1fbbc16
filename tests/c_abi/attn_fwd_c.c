/*
 * attn_fwd_c.c -- one call of libtos.so through its C ABI alone (HIP runtime
 * for device memory and the stream; no Python, no torch).  Test program: it
 * draws seeded inputs, runs tos_attn_fwd and writes inputs and outputs to a
 * file that the parity test checks against the oracle.
 *
 *   attn_fwd_c B H N d causal dtype seed out.bin
 *
 * dtype: 0 = f32, 1 = bf16, 3 = f16 (tos_dtype values).  Output file: six
 * int64 (B, H, N, d, causal, dtype), then q, k, v and o as stored (element
 * size of the dtype; o as the library writes it), then lse as float32.
 * Exit status 0 on success; the tos_status or HIP error is printed otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tos.h"

/* xorshift64* -> uniform in [-2, 2) */
static uint64_t state;
static float next_uniform(void) {
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    const uint64_t r = state * 0x2545F4914F6CDD1DULL;
    return (float)((double)(r >> 11) * (1.0 / 9007199254740992.0) * 4.0 - 2.0);
}

/* float32 -> bfloat16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* float32 -> float16 bits, round to nearest even, for |x| < 65504 and normal
 * results (the generator's range) */
static uint16_t to_f16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const int32_t e = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
    uint32_t m = u & 0x7FFFFFu;
    if (e <= 0) return (uint16_t)sign;   /* below 2^-14: flush (rare in [-2, 2)) */
    uint32_t h = ((uint32_t)e << 10) | (m >> 13);
    const uint32_t rest = m & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1;
    return (uint16_t)(sign | h);
}

static int check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 9) {
        fprintf(stderr, "usage: %s B H N d causal dtype seed out.bin\n", argv[0]);
        return 2;
    }
    const int64_t B = atoll(argv[1]), H = atoll(argv[2]), N = atoll(argv[3]), d = atoll(argv[4]);
    const int causal = atoi(argv[5]), dtype = atoi(argv[6]);
    state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)atoll(argv[7]);
    if (dtype != TOS_F32 && dtype != TOS_BF16 && dtype != TOS_F16) {
        fprintf(stderr, "dtype must be 0, 1 or 3\n");
        return 2;
    }
    const size_t n = (size_t)(B * H * N * d), esz = dtype == TOS_F32 ? 4 : 2;
    const size_t nl = (size_t)(B * H * N);
    unsigned char* host[4];
    for (int t = 0; t < 4; ++t) host[t] = (unsigned char*)malloc(n * esz);
    float* lse = (float*)malloc(nl * sizeof(float));
    for (int t = 0; t < 3; ++t)
        for (size_t i = 0; i < n; ++i) {
            const float x = next_uniform();
            if (dtype == TOS_F32) ((float*)host[t])[i] = x;
            else if (dtype == TOS_BF16) ((uint16_t*)host[t])[i] = to_bf16(x);
            else ((uint16_t*)host[t])[i] = to_f16(x);
        }

    void* dev[4];
    float* dlse;
    hipStream_t stream;
    if (check_hip(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
    for (int t = 0; t < 4; ++t)
        if (check_hip(hipMalloc(&dev[t], n * esz), "hipMalloc")) return 1;
    if (check_hip(hipMalloc((void**)&dlse, nl * sizeof(float)), "hipMalloc")) return 1;
    for (int t = 0; t < 3; ++t)
        if (check_hip(hipMemcpy(dev[t], host[t], n * esz, hipMemcpyHostToDevice), "hipMemcpy")) return 1;

    tos_fwd_opts opts;
    if (tos_fwd_opts_default(&opts) != TOS_OK) return 1;
    const float scale = 1.0f / sqrtf((float)d);
    const tos_status st = tos_attn_fwd(dev[0], dev[1], dev[2], dev[3], dlse, B, H, N, d, causal,
                                       scale, (tos_dtype)dtype, &opts, (void*)stream);
    if (st != TOS_OK) {
        fprintf(stderr, "tos_attn_fwd: %s\n", tos_status_string(st));
        return 1;
    }
    if (check_hip(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;
    if (check_hip(hipMemcpy(host[3], dev[3], n * esz, hipMemcpyDeviceToHost), "hipMemcpy")) return 1;
    if (check_hip(hipMemcpy(lse, dlse, nl * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy")) return 1;

    FILE* f = fopen(argv[8], "wb");
    if (!f) {
        perror(argv[8]);
        return 1;
    }
    const int64_t hdr[6] = {B, H, N, d, causal, dtype};
    fwrite(hdr, sizeof(hdr), 1, f);
    for (int t = 0; t < 4; ++t) fwrite(host[t], esz, n, f);
    fwrite(lse, sizeof(float), nl, f);
    fclose(f);
    for (int t = 0; t < 4; ++t) {
        hipFree(dev[t]);
        free(host[t]);
    }
    hipFree(dlse);
    free(lse);
    hipStreamDestroy(stream);
    printf("tos_attn_fwd: %s (library version %d)\n", tos_status_string(st), tos_version());
    return 0;
}
