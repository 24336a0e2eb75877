/*
 * Drives every oracle entry point on small seeded inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).
 * Prints "ok" when every output is finite; any out-of-bounds access, leak or
 * undefined operation aborts the run instead.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oscar_oracle.h"

static uint32_t rng_state = 12345u;
static float urand(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)((rng_state >> 8) & 0xffffu) / 65536.0f - 0.5f;
}

static uint16_t *fp16_vec(size_t n, float scale)
{
    uint16_t *x = malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; i++)
        x[i] = orc_f32_to_f16(scale * urand());
    return x;
}

static int all_finite(const float *x, size_t n)
{
    for (size_t i = 0; i < n; i++)
        if (!isfinite(x[i]))
            return 0;
    return 1;
}

/* prefill sequence 0 with n_prefill tokens, leave sequence 1 empty, then
 * n_append appends to both and one decode step */
static int run_cache(int hq, int hkv, int scope, int flush, int n_prefill, int n_append, int mb)
{
    const int B = 2, P = B * mb, D = ORC_D;
    const size_t nh = scope == ORC_NORM_HEAD ? (size_t)hkv : 1;
    orc_cache c;
    memset(&c, 0, sizeof c);
    c.batch = B;
    c.num_q_heads = hq;
    c.num_kv_heads = hkv;
    c.norm_scope = scope;
    c.max_blocks_per_seq = mb;
    c.num_physical_blocks = P;
    c.flush_tokens = flush;
    c.pool = calloc((size_t)P * hkv * ORC_REC_BYTES, 1);
    c.pool_norm = calloc((size_t)P * nh * ORC_G, sizeof(uint16_t));
    c.res_k = calloc((size_t)B * hkv * ORC_R * D, sizeof(uint16_t));
    c.res_v = calloc((size_t)B * hkv * D * ORC_R, sizeof(uint16_t));
    c.res_norm = calloc((size_t)B * nh * ORC_R, sizeof(uint16_t));
    int32_t *table = malloc((size_t)B * mb * sizeof(int32_t));
    for (int i = 0; i < B * mb; i++)
        table[i] = (i * 7) % P;
    c.block_table = table;
    c.seq_state = calloc((size_t)B * 2, sizeof(int32_t));
    c.error_flag = calloc(1, sizeof(int32_t));

    uint16_t *k = fp16_vec((size_t)n_prefill * hkv * D, 8.0f);
    uint16_t *v = fp16_vec((size_t)n_prefill * hkv * D, 2.0f);
    if (n_prefill)
        orc_prefill(&c, 0, k, v, n_prefill, ORC_FP16);
    for (int s = 0; s < n_append; s++) {
        uint16_t *kn = fp16_vec((size_t)B * hkv * D, 8.0f);
        uint16_t *vn = fp16_vec((size_t)B * hkv * D, 2.0f);
        orc_append(&c, kn, vn, ORC_FP16);
        free(kn);
        free(vn);
    }
    uint16_t *q = fp16_vec((size_t)B * hq * D, 2.0f);
    float *qr = malloc((size_t)B * hq * D * sizeof(float));
    float *out = malloc((size_t)B * hq * D * sizeof(float));
    float *lse = malloc((size_t)B * hq * sizeof(float));
    orc_rotate_query(q, ORC_FP16, (size_t)B * hq, qr);
    orc_decode_attn(&c, qr, out, lse);
    int ok = all_finite(out, (size_t)B * hq * D);
    free(k);
    free(v);
    free(q);
    free(qr);
    free(out);
    free(lse);
    free(c.pool);
    free(c.pool_norm);
    free(c.res_k);
    free(c.res_v);
    free(c.res_norm);
    free(table);
    free(c.seq_state);
    free(c.error_flag);
    return ok;
}

int main(void)
{
    int ok = 1;
    /* rotation and scaling, both norm scopes; a zero token */
    {
        const int T = 40, H = 3, D = ORC_D;
        uint16_t *k = fp16_vec((size_t)T * H * D, 4.0f);
        memset(k, 0, (size_t)H * D * sizeof(uint16_t));
        uint16_t *khat = malloc((size_t)T * H * D * sizeof(uint16_t));
        uint16_t *norm = malloc((size_t)T * H * sizeof(uint16_t));
        orc_rotate_scale_key(k, ORC_FP16, T, H, ORC_NORM_TOKEN, khat, norm);
        orc_rotate_scale_key(k, ORC_BF16, T, H, ORC_NORM_HEAD, khat, norm);
        /* stateless quantizer over the first 32 tokens, both scopes */
        uint8_t *rec = malloc((size_t)H * ORC_REC_BYTES);
        uint16_t *pn = malloc((size_t)H * ORC_G * sizeof(uint16_t));
        orc_quant_pack(khat, norm, k, 1, H, ORC_NORM_HEAD, rec, pn);
        orc_rotate_scale_key(k, ORC_FP16, T, H, ORC_NORM_TOKEN, khat, norm);
        orc_quant_pack(khat, norm, k, 1, H, ORC_NORM_TOKEN, rec, pn);
        free(k);
        free(khat);
        free(norm);
        free(rec);
        free(pn);
    }
    /* the residual-window state machine and attention; flushes of 32 and
     * 128 tokens; a block table too short (capacity flag) */
    ok &= run_cache(4, 1, ORC_NORM_TOKEN, 32, 300, 70, 16);
    ok &= run_cache(8, 2, ORC_NORM_HEAD, 32, 129, 40, 12);
    ok &= run_cache(8, 8, ORC_NORM_TOKEN, 128, 257, 130, 20);
    ok &= run_cache(4, 1, ORC_NORM_TOKEN, 32, 160, 100, 4);
    /* more KV heads than any fixed-size buffer of 64 would hold */
    ok &= run_cache(80, 80, ORC_NORM_HEAD, 32, 40, 2, 4);
    ok &= run_cache(80, 80, ORC_NORM_TOKEN, 32, 40, 2, 4);
    /* values beyond fp16's range, non-finite and NaN inputs: saturated on
     * the way into the cache, no undefined conversion in the quantizer */
    {
        const int T = 64, H = 2, D = ORC_D;
        uint16_t *x = fp16_vec((size_t)T * H * D, 4.0f);
        const uint16_t odd[] = {0x7c00u, 0xfc00u, 0x7e00u, 0x7bffu, 0xfbffu};
        for (size_t i = 0; i < (size_t)T * H * D; i += 37)
            x[i] = odd[(i / 37) % 5];
        uint16_t *v16 = malloc((size_t)T * H * D * sizeof(uint16_t));
        orc_to_f16(x, ORC_FP16, (size_t)T * H * D, v16);
        uint8_t *rec = malloc((size_t)2 * H * ORC_REC_BYTES);
        uint16_t *pn = malloc((size_t)2 * H * ORC_G * sizeof(uint16_t));
        uint16_t *nrm = calloc((size_t)T * H, sizeof(uint16_t));
        orc_quant_pack(x, nrm, x, 2, H, ORC_NORM_HEAD, rec, pn);
        orc_quant_pack(v16, nrm, v16, 2, H, ORC_NORM_HEAD, rec, pn);
        free(x);
        free(v16);
        free(rec);
        free(pn);
        free(nrm);
    }
    /* unquantized attention (the bf16 baseline), including n = 0 */
    {
        const int n = 77, hq = 8, hkv = 2, D = ORC_D;
        float *q = malloc((size_t)hq * D * sizeof(float));
        float *k = malloc((size_t)n * hkv * D * sizeof(float));
        float *v = malloc((size_t)n * hkv * D * sizeof(float));
        float *out = malloc((size_t)hq * D * sizeof(float));
        float *lse = malloc((size_t)hq * sizeof(float));
        for (int i = 0; i < hq * D; i++)
            q[i] = urand();
        for (int i = 0; i < n * hkv * D; i++) {
            k[i] = 10.0f * urand();
            v[i] = urand();
        }
        orc_dense_attn(q, k, v, n, hq, hkv, out, lse);
        ok &= all_finite(out, (size_t)hq * D);
        orc_dense_attn(q, k, v, 0, hq, hkv, out, NULL);
        free(q);
        free(k);
        free(v);
        free(out);
        free(lse);
    }
    printf(ok ? "ok\n" : "non-finite output\n");
    return ok ? 0 : 1;
}
