/*
 * A torch-free caller of libkvevict on the GPU: plain C with the HIP runtime's
 * C API for device memory and copies.  The small parity configuration (one
 * layer of H KV heads, head dim 128, float32 keys, one 1024-token prefill
 * block, budget 512, 4 sinks, no recent window, keep the lowest L2 norms) runs
 * two ways:
 *   block:  qf_score_keys, kv_evict_topk and kv_compact_gather over the block;
 *   decode: the same 1024 tokens one at a time, qf_score_keys then
 *           kv_evict_one_inplace.
 * Both are compared with the CPU oracle (oracle/kvx_oracle.c, linked as a
 * test library: orc_score, orc_select) -- scores within 1e-5 of the norm, kept
 * positions, stored scores and K/V bytes bit for bit -- and with each other
 * (the L2Norm page's block-versus-token path independence).  Prints one
 * "name value" line per check; the pytest wrapper compares them.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvevict.h"

/* the oracle's C entry points (test library) */
int orc_score(const void *k, int dtype, int64_t n, int64_t D, int mode, const float *f, int sign, float *out);
int orc_select(const float *s, int64_t n_total, int64_t budget, int64_t n_sink, int64_t recent, int keep_low,
               int64_t *keep_idx, int64_t *n_out);

enum { H = 3, D = 128, T = 1024, BUDGET = 512, SINK = 4 };

#define CHECK_HIP(x)                                                      \
    do {                                                                  \
        if ((x) != hipSuccess) {                                          \
            printf("hip_error %s line %d\n", #x, __LINE__);               \
            return 1;                                                     \
        }                                                                 \
    } while (0)
#define CHECK_KVX(x)                                                      \
    do {                                                                  \
        int rc_ = (x);                                                    \
        if (rc_ != KVX_OK) {                                              \
            printf("kvx_error %d %s: %s\n", rc_, #x, kvx_last_error());   \
            return 1;                                                     \
        }                                                                 \
    } while (0)

/* xorshift64* and the sum of four uniforms: a seeded, roughly normal key */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float next_value(void) {
    float acc = 0.0f;
    for (int i = 0; i < 4; ++i) {
        rng_state ^= rng_state >> 12;
        rng_state ^= rng_state << 25;
        rng_state ^= rng_state >> 27;
        acc += (float)((rng_state * 0x2545F4914F6CDD1Dull) >> 40) / (float)(1 << 24) - 0.5f;
    }
    return acc * 1.7320508f;
}

int main(void) {
    const size_t row = D * sizeof(float);
    float *K = malloc((size_t)H * T * row), *V = malloc((size_t)H * T * row);
    for (size_t i = 0; i < (size_t)H * T * D; ++i) K[i] = next_value();
    for (size_t i = 0; i < (size_t)H * T * D; ++i) V[i] = next_value();
    const kvx_shape sh = {1, 1, H, D, KVX_F32};
    const kvx_evict_params p = {BUDGET, SINK, 0, KVX_KEEP_LOW};

    void *k_new, *v_new, *kb[2], *vb[2];
    float *s_new, *sb[2];
    int32_t *pb[2], *idx;
    CHECK_HIP(hipMalloc(&k_new, (size_t)H * T * row));
    CHECK_HIP(hipMalloc(&v_new, (size_t)H * T * row));
    CHECK_HIP(hipMalloc((void **)&s_new, (size_t)H * T * sizeof(float)));
    CHECK_HIP(hipMalloc((void **)&idx, (size_t)H * BUDGET * sizeof(int32_t)));
    for (int b = 0; b < 2; ++b) {
        CHECK_HIP(hipMalloc(&kb[b], (size_t)H * BUDGET * row));
        CHECK_HIP(hipMalloc(&vb[b], (size_t)H * BUDGET * row));
        CHECK_HIP(hipMalloc((void **)&sb[b], (size_t)H * BUDGET * sizeof(float)));
        CHECK_HIP(hipMalloc((void **)&pb[b], (size_t)H * BUDGET * sizeof(int32_t)));
    }
    CHECK_HIP(hipMemcpy(k_new, K, (size_t)H * T * row, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v_new, V, (size_t)H * T * row, hipMemcpyHostToDevice));

    /* block: an empty cache (buffer set 0) absorbs all T rows into buffer set 1 */
    CHECK_KVX(qf_score_keys(k_new, sh, T, KVX_SCORE_L2, NULL, 1, s_new, NULL));
    CHECK_KVX(kv_evict_topk(sb[0], s_new, sh, 0, T, p, idx, NULL, 0, NULL));
    CHECK_KVX(kv_compact_gather(kb[0], vb[0], sb[0], pb[0], k_new, v_new, s_new, 0, idx, sh, 0, T, p, kb[1], vb[1],
                                sb[1], pb[1], NULL));
    CHECK_HIP(hipDeviceSynchronize());
    float *s_gpu = malloc((size_t)H * T * sizeof(float));
    CHECK_HIP(hipMemcpy(s_gpu, s_new, (size_t)H * T * sizeof(float), hipMemcpyDeviceToHost));

    /* decode: token t of every group is row t of a [H, T, D] tensor, so one
       token's rows are strided; copy them into a [H, 1, D] staging buffer */
    void *k_tok, *v_tok;
    float *s_tok;
    CHECK_HIP(hipMalloc(&k_tok, (size_t)H * row));
    CHECK_HIP(hipMalloc(&v_tok, (size_t)H * row));
    CHECK_HIP(hipMalloc((void **)&s_tok, (size_t)H * sizeof(float)));
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            CHECK_HIP(hipMemcpy((char *)k_tok + h * row, K + ((size_t)h * T + t) * D, row, hipMemcpyHostToDevice));
            CHECK_HIP(hipMemcpy((char *)v_tok + h * row, V + ((size_t)h * T + t) * D, row, hipMemcpyHostToDevice));
        }
        CHECK_KVX(qf_score_keys(k_tok, sh, 1, KVX_SCORE_L2, NULL, 1, s_tok, NULL));
        CHECK_KVX(kv_evict_one_inplace(kb[0], vb[0], sb[0], pb[0], k_tok, v_tok, s_tok, t, sh,
                                       t < BUDGET ? t : BUDGET, p, NULL));
    }
    CHECK_HIP(hipDeviceSynchronize());

    float *kout[2], *vout[2], *sout[2];
    int32_t *pout[2];
    for (int b = 0; b < 2; ++b) {
        kout[b] = malloc((size_t)H * BUDGET * row);
        vout[b] = malloc((size_t)H * BUDGET * row);
        sout[b] = malloc((size_t)H * BUDGET * sizeof(float));
        pout[b] = malloc((size_t)H * BUDGET * sizeof(int32_t));
        CHECK_HIP(hipMemcpy(kout[b], kb[b], (size_t)H * BUDGET * row, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(vout[b], vb[b], (size_t)H * BUDGET * row, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(sout[b], sb[b], (size_t)H * BUDGET * sizeof(float), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(pout[b], pb[b], (size_t)H * BUDGET * sizeof(int32_t), hipMemcpyDeviceToHost));
    }

    /* oracle on the host: scores, then the kept rows chosen on the GPU's scores */
    int scores_ok = 1, block_ok = 1, decode_ok = 1, same_ok = 1;
    float *s_ref = malloc((size_t)T * sizeof(float));
    int64_t *keep = malloc((size_t)T * sizeof(int64_t));
    for (int h = 0; h < H; ++h) {
        const float *Kh = K + (size_t)h * T * D, *Vh = V + (size_t)h * T * D;
        if (orc_score(Kh, 0, T, D, 0, NULL, 1, s_ref) != 0) return 1;
        for (int t = 0; t < T; ++t)
            if (fabs((double)s_gpu[(size_t)h * T + t] - (double)s_ref[t]) > 1e-5 * (double)s_ref[t]) scores_ok = 0;
        int64_t n_out = 0;
        if (orc_select(s_gpu + (size_t)h * T, T, BUDGET, SINK, 0, 1, keep, &n_out) != 0 || n_out != BUDGET) return 1;
        for (int b = 0; b < 2; ++b) {
            int ok = 1;
            for (int j = 0; j < BUDGET; ++j) {
                const size_t o = (size_t)h * BUDGET + j;
                const int64_t r = keep[j];
                ok &= pout[b == 0 ? 1 : 0][o] == r;
                ok &= sout[b == 0 ? 1 : 0][o] == s_gpu[(size_t)h * T + r];
                ok &= memcmp(kout[b == 0 ? 1 : 0] + o * D, Kh + r * D, row) == 0;
                ok &= memcmp(vout[b == 0 ? 1 : 0] + o * D, Vh + r * D, row) == 0;
            }
            if (b == 0) block_ok &= ok;
            else decode_ok &= ok;
        }
    }
    same_ok = memcmp(kout[0], kout[1], (size_t)H * BUDGET * row) == 0 &&
              memcmp(pout[0], pout[1], (size_t)H * BUDGET * sizeof(int32_t)) == 0;
    printf("scores_within_tolerance %d\n", scores_ok);
    printf("block_equals_oracle %d\n", block_ok);
    printf("decode_equals_oracle %d\n", decode_ok);
    printf("block_equals_decode %d\n", same_ok);
    return 0;
}
