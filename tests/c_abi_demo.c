/*
 * A plain C caller of the OScaR library: only include/oscar.h and the HIP
 * runtime, no Python and no torch.  Reads a sequence's Keys and Values, one
 * new token and the step's query from a binary file, then, through the C ABI:
 * cache layout, prefill, one append, decode attention.  Writes the attention
 * output, the log-sum-exp, {n, Q} and the error flag to a second file.
 *
 *   c_abi_demo IN OUT
 *   IN:  int32 hq, hkv, n_prefill, dtype; uint16 k[n][hkv][128], v[n][hkv][128],
 *        k_new[hkv][128], v_new[hkv][128], q[hq][128]
 *   OUT: float out[hq][128], lse[hq]; int32 n, Q, error_flag
 * Exit status 0 on success; a failing call prints its status string.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oscar.h"

#define CHECK_HIP(x)                                                      \
    do {                                                                  \
        if ((x) != hipSuccess) {                                          \
            fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);  \
            return 2;                                                     \
        }                                                                 \
    } while (0)
#define CHECK_OSCAR(x)                                                    \
    do {                                                                  \
        oscar_status s_ = (x);                                            \
        if (s_ != OSCAR_OK) {                                             \
            fprintf(stderr, "%s: %s\n", #x, oscar_status_str(s_));        \
            return 3;                                                     \
        }                                                                 \
    } while (0)

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    if (hipMalloc(&p, bytes ? bytes : 16) != hipSuccess)
        return NULL;
    if (hipMemset(p, 0, bytes ? bytes : 16) != hipSuccess)
        return NULL;
    return p;
}

static void *dev_copy(const void *host, size_t bytes)
{
    void *p = dev_alloc(bytes);
    if (p && bytes && hipMemcpy(p, host, bytes, hipMemcpyHostToDevice) != hipSuccess)
        return NULL;
    return p;
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f)
        return 1;
    int32_t hdr[4];
    if (fread(hdr, sizeof hdr, 1, f) != 1)
        return 1;
    const int hq = hdr[0], hkv = hdr[1], n = hdr[2];
    const oscar_dtype dtype = (oscar_dtype)hdr[3];
    const size_t row = (size_t)hkv * OSCAR_HEAD_DIM;
    uint16_t *k = malloc((size_t)n * row * 2), *v = malloc((size_t)n * row * 2);
    uint16_t *kn = malloc(row * 2), *vn = malloc(row * 2);
    uint16_t *q = malloc((size_t)hq * OSCAR_HEAD_DIM * 2);
    if (fread(k, 2, (size_t)n * row, f) != (size_t)n * row || fread(v, 2, (size_t)n * row, f) != (size_t)n * row ||
        fread(kn, 2, row, f) != row || fread(vn, 2, row, f) != row ||
        fread(q, 2, (size_t)hq * OSCAR_HEAD_DIM, f) != (size_t)hq * OSCAR_HEAD_DIM)
        return 1;
    fclose(f);

    const int max_ctx = n + 1;
    oscar_cache_geom g;
    memset(&g, 0, sizeof g);
    g.batch = 1;
    g.num_q_heads = hq;
    g.num_kv_heads = hkv;
    g.head_dim = OSCAR_HEAD_DIM;
    g.block_tokens = OSCAR_BLOCK_TOKENS;
    g.residual_tokens = OSCAR_RESIDUAL_TOKENS;
    g.v_group = OSCAR_V_GROUP;
    g.norm_scope = OSCAR_NORM_TOKEN;
    g.max_blocks_per_seq = max_ctx / OSCAR_BLOCK_TOKENS + 1;
    g.num_physical_blocks = g.max_blocks_per_seq;
    g.flush_tokens = 32;
    g.key_scale = OSCAR_SCALE_IEEE;
    oscar_cache_sizes sz;
    CHECK_OSCAR(oscar_cache_layout(&g, &sz));

    int32_t *table = malloc(sz.block_table);
    for (int i = 0; i < g.max_blocks_per_seq; i++)  /* physical blocks in reverse order */
        table[i] = g.max_blocks_per_seq - 1 - i;
    oscar_cache c;
    c.pool = dev_alloc(sz.pool);
    c.pool_norm = dev_alloc(sz.pool_norm);
    c.res_k = dev_alloc(sz.res_k);
    c.res_v = dev_alloc(sz.res_v);
    c.res_norm = dev_alloc(sz.res_norm);
    c.block_table = dev_copy(table, sz.block_table);
    c.seq_state = dev_alloc(sz.seq_state);
    c.error_flag = dev_alloc(sz.error_flag);
    c.append_sync = dev_alloc(sz.append_sync);
    c.rope = NULL;   /* inputs arrive rotated by position (rope_max_pos 0) */
    void *dk = dev_copy(k, (size_t)n * row * 2), *dv = dev_copy(v, (size_t)n * row * 2);
    void *dkn = dev_copy(kn, row * 2), *dvn = dev_copy(vn, row * 2);
    void *dq = dev_copy(q, (size_t)hq * OSCAR_HEAD_DIM * 2);
    float *dout = dev_alloc((size_t)hq * OSCAR_HEAD_DIM * sizeof(float));
    float *dlse = dev_alloc((size_t)hq * sizeof(float));
    if (!c.pool || !c.pool_norm || !c.res_k || !c.res_v || !c.res_norm || !c.block_table ||
        !c.seq_state || !c.error_flag || !c.append_sync || !dk || !dv || !dkn || !dvn || !dq || !dout || !dlse)
        return 2;

    CHECK_OSCAR(oscar_prefill_quantize(&g, &c, 0, dk, dv, n, dtype, NULL));
    CHECK_OSCAR(oscar_append_kv(&g, &c, dkn, dvn, dtype, NULL));
    int32_t splits = 0;
    size_t ws_bytes = 0;
    CHECK_OSCAR(oscar_decode_workspace_bytes(&g, max_ctx, 0, &splits, &ws_bytes));
    void *ws = dev_alloc(ws_bytes);
    if (!ws)
        return 2;
    CHECK_OSCAR(oscar_decode_attn(&g, &c, dq, dtype, dout, dlse, ws, ws_bytes, 0, max_ctx,
                                  OSCAR_ATTN_AUTO, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    float *out = malloc((size_t)hq * OSCAR_HEAD_DIM * sizeof(float));
    float *lse = malloc((size_t)hq * sizeof(float));
    int32_t st[3];
    CHECK_HIP(hipMemcpy(out, dout, (size_t)hq * OSCAR_HEAD_DIM * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse, dlse, (size_t)hq * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(st, c.seq_state, 2 * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(st + 2, c.error_flag, sizeof(int32_t), hipMemcpyDeviceToHost));
    f = fopen(argv[2], "wb");
    if (!f)
        return 1;
    fwrite(out, sizeof(float), (size_t)hq * OSCAR_HEAD_DIM, f);
    fwrite(lse, sizeof(float), (size_t)hq, f);
    fwrite(st, sizeof(int32_t), 3, f);
    fclose(f);

    void *bufs[] = {c.pool, c.pool_norm, c.res_k, c.res_v, c.res_norm, c.block_table,
                    c.seq_state, c.error_flag, dk, dv, dkn, dvn, dq, dout, dlse, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++)
        CHECK_HIP(hipFree(bufs[i]));
    free(k);
    free(v);
    free(kn);
    free(vn);
    free(q);
    free(table);
    free(out);
    free(lse);
    printf("ok: n=%d splits=%d\n", n + 1, splits);
    return 0;
}
