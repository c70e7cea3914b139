/*
 * The library driven from plain C (C99, built with gcc), through include/df11.h
 * and the HIP runtime API only: no Python, no PyTorch.  It encodes three
 * seeded tensors on the host, validates the containers, builds one plan,
 * uploads the containers, decodes them in one batched launch on a stream
 * of its own, checks the plan's flag, compares every word with its source,
 * then encodes the same words on the GPU and compares those containers with
 * the host encoder's byte for byte.  Exit status 0 when everything matches,
 * 1 otherwise (with the failing call on stderr).
 *
 * The method it exercises (mlx-dfloat project page, introduction and its
 * 16-bit weight diagram): each BF16 word's exponent byte is stored as a
 * prefix code, its sign and fraction as one raw byte, and decoding gives
 * back every word bit for bit.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "df11.h"

#define DF11_TRY(call)                                                                       \
    do {                                                                                     \
        df11_status s_ = (call);                                                             \
        if (s_ != DF11_OK) {                                                                 \
            fprintf(stderr, "%s: %s (%s)\n", #call, df11_status_str(s_), df11_last_error()); \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)
#define HIP_TRY(call)                                                    \
    do {                                                                 \
        hipError_t e_ = (call);                                          \
        if (e_ != hipSuccess) {                                          \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_)); \
            return 1;                                                    \
        }                                                                \
    } while (0)

enum { N_TENSORS = 3 };

/* splitmix64 (Steele, Lea and Flood, 2014): seeded 64-bit words */
static uint64_t next_u64(uint64_t *s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* BF16 words with weight-like exponents (118 + a binomial(8, 1/2) draw, one
 * word in 64 a zero), random sign and fraction */
static void make_words(uint16_t *w, uint64_t n, uint64_t seed) {
    uint64_t s = seed;
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t r = next_u64(&s);
        const unsigned e = 118u + (unsigned)__builtin_popcountll(r & 0xFFu);
        const unsigned low = (unsigned)(r >> 8) & 0xFFu;
        w[i] = ((r >> 16) & 63u) == 0 ? 0 : (uint16_t)(((low & 0x80u) << 8) | (e << 7) | (low & 0x7Fu));
    }
}

int main(void) {
    const uint64_t n[N_TENSORS] = {100000, 4 * 32768 + 77, 5};
    uint16_t *words[N_TENSORS];
    uint8_t *conts[N_TENSORS];
    uint64_t cont_bytes[N_TENSORS];
    size_t meta_bytes[N_TENSORS];
    const void *metas[N_TENSORS];
    void *d_conts[N_TENSORS], *d_outs[N_TENSORS], *d_words[N_TENSORS], *d_encs[N_TENSORS];
    uint64_t enc_caps[N_TENSORS], enc_bytes[N_TENSORS], dims[8 * N_TENSORS];
    int ndims[N_TENSORS];
    if (df11_abi_version() != DF11_ABI_VERSION) {
        fprintf(stderr, "library ABI %d, header ABI %d\n", df11_abi_version(), DF11_ABI_VERSION);
        return 1;
    }

    /* encode on the host, validate */
    for (int t = 0; t < N_TENSORS; ++t) {
        words[t] = (uint16_t *)malloc(n[t] * 2);
        const uint64_t cap = df11_container_bound(n[t]);
        conts[t] = (uint8_t *)malloc(cap);
        if (!words[t] || !conts[t]) return 1;
        make_words(words[t], n[t], 1000u + (uint64_t)t);
        DF11_TRY(df11_encode(words[t], n[t], 1, &n[t], conts[t], cap, &cont_bytes[t], 0));
        df11_tensor_info info;
        DF11_TRY(df11_validate(conts[t], cont_bytes[t], &info));
        if (info.n_elems != n[t] || info.container_bytes != cont_bytes[t]) {
            fprintf(stderr, "tensor %d: validate describes %llu elements, %llu bytes\n", t,
                    (unsigned long long)info.n_elems, (unsigned long long)info.container_bytes);
            return 1;
        }
        metas[t] = conts[t];
        meta_bytes[t] = (size_t)cont_bytes[t];
    }

    /* one plan, the containers in device memory, one batched decode */
    df11_plan_t plan = NULL;
    DF11_TRY(df11_plan(metas, meta_bytes, N_TENSORS, 0, 0, &plan));
    hipStream_t stream;
    HIP_TRY(hipStreamCreate(&stream));
    for (int t = 0; t < N_TENSORS; ++t) {
        HIP_TRY(hipMalloc(&d_conts[t], cont_bytes[t]));
        HIP_TRY(hipMalloc(&d_outs[t], n[t] * 2));
        HIP_TRY(hipMemcpy(d_conts[t], conts[t], cont_bytes[t], hipMemcpyHostToDevice));
    }
    DF11_TRY(df11_decode_batch(plan, (const void *const *)d_conts, (void *const *)d_outs, stream));
    DF11_TRY(df11_check(plan, stream));
    uint64_t words_checked = 0;
    for (int t = 0; t < N_TENSORS; ++t) {
        uint16_t *back = (uint16_t *)malloc(n[t] * 2);
        if (!back) return 1;
        HIP_TRY(hipMemcpy(back, d_outs[t], n[t] * 2, hipMemcpyDeviceToHost));
        if (memcmp(back, words[t], n[t] * 2) != 0) {
            fprintf(stderr, "tensor %d: decoded words differ from the source\n", t);
            return 1;
        }
        words_checked += n[t];
        free(back);
    }

    /* the GPU encoder on the same words: the host encoder's bytes */
    for (int t = 0; t < N_TENSORS; ++t) {
        HIP_TRY(hipMalloc(&d_words[t], n[t] * 2));
        HIP_TRY(hipMemcpy(d_words[t], words[t], n[t] * 2, hipMemcpyHostToDevice));
        enc_caps[t] = df11_container_bound(n[t]);
        HIP_TRY(hipMalloc(&d_encs[t], enc_caps[t]));
        ndims[t] = 1;
        dims[8 * t] = n[t];
    }
    DF11_TRY(df11_encode_device_batch(N_TENSORS, (const void *const *)d_words, n, ndims, dims,
                                      (void *const *)d_encs, enc_caps, enc_bytes, 0, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    for (int t = 0; t < N_TENSORS; ++t) {
        if (enc_bytes[t] != cont_bytes[t]) {
            fprintf(stderr, "tensor %d: GPU container %llu bytes, host %llu\n", t,
                    (unsigned long long)enc_bytes[t], (unsigned long long)cont_bytes[t]);
            return 1;
        }
        uint8_t *back = (uint8_t *)malloc(enc_bytes[t]);
        if (!back) return 1;
        HIP_TRY(hipMemcpy(back, d_encs[t], enc_bytes[t], hipMemcpyDeviceToHost));
        if (memcmp(back, conts[t], enc_bytes[t]) != 0) {
            fprintf(stderr, "tensor %d: GPU container differs from the host encoder's\n", t);
            return 1;
        }
        free(back);
    }

    for (int t = 0; t < N_TENSORS; ++t) {
        HIP_TRY(hipFree(d_conts[t]));
        HIP_TRY(hipFree(d_outs[t]));
        HIP_TRY(hipFree(d_words[t]));
        HIP_TRY(hipFree(d_encs[t]));
        free(words[t]);
        free(conts[t]);
    }
    df11_plan_destroy(plan);
    HIP_TRY(hipStreamDestroy(stream));
    printf("ok: %d tensors, %llu words decoded bit-exact, GPU containers equal the host encoder's\n", N_TENSORS,
           (unsigned long long)words_checked);
    return 0;
}
