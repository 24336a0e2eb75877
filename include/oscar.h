/*
 * oscar.h -- C ABI of the MI355X (gfx950) OScaR INT2 KV-cache library.
 *
 * OScaR ("Omni-Scaled Canalized Rotation", arXiv 2605.19660) quantizes the KV
 * cache to 2 bits in three steps: an online 128-point Hadamard rotation of
 * each new Key and of the query, a per-token L2 normalisation of the rotated
 * Key whose norm is kept, and KIVI-style INT2 quantization (Keys per channel
 * over 32-token blocks, Values per token over 32-channel groups) with the
 * newest 128 tokens kept in fp16.  Decode attention dequantizes, undoes the
 * scaling and attends.  The three kernels of the method -- fused FHT +
 * scaling, quantization, fused dequant + inverse scaling + attention -- are
 * named in the structured summary "OScaR：面向大模型及多模态LLM极限KV缓存量化的
 * 奥卡姆剃刀" (paper.rainbus.top), section 方法步骤详情, and in the reading
 * notes "OScaR: The Occam's Razor for Extreme KV Cache Quantization in LLMs
 * and Beyond" (yingwang.github.io), section End-to-End Flow.
 *
 * Conventions for every entry point:
 *   - Plain pointers only.  "device" pointers are HIP device memory of the
 *     current device; "host" pointers are ordinary host memory.
 *   - The caller owns and allocates every buffer (sizes from
 *     oscar_cache_layout / oscar_decode_workspace_bytes).  The library never
 *     allocates, frees or synchronizes; its only memory of its own is the
 *     fixed per-GPU workspace of oscar_decode_attn_noalloc.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream).  Results are visible after the
 *     caller synchronizes that stream.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns OSCAR_EINVAL and enqueues nothing.  Device-side
 *     conditions (block-table capacity, prefill into a non-empty sequence)
 *     set sticky bits in *error_flag and skip the affected write.
 *   - Calls on one stream are ordered; calls on different streams that touch
 *     the same cache race.
 *   - Only gfx950 is supported (OSCAR_EUNSUPPORTED otherwise).
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define OSCAR_API __attribute__((visibility("default")))
#else
#define OSCAR_API
#endif

#define OSCAR_HEAD_DIM 128       /* d */
#define OSCAR_BLOCK_TOKENS 32    /* G: Key quantization block */
#define OSCAR_RESIDUAL_TOKENS 128 /* R: fp16 residual window */
#define OSCAR_V_GROUP 32         /* Value quantization group (channels) */
#define OSCAR_RECORD_BYTES 3072  /* one (physical block, KV head) record */

typedef enum {
    OSCAR_OK = 0,
    OSCAR_EINVAL = 1,       /* bad argument: null pointer, bad shape, misalignment */
    OSCAR_EUNSUPPORTED = 2, /* device is not gfx950, or option not built */
    OSCAR_ELAUNCH = 3,      /* the HIP runtime rejected a launch */
    OSCAR_EWORKSPACE = 4    /* workspace smaller than oscar_decode_workspace_bytes */
} oscar_status;

typedef enum { OSCAR_FP16 = 0, OSCAR_BF16 = 1, OSCAR_FP32 = 2 } oscar_dtype;
typedef enum { OSCAR_NORM_TOKEN = 0, OSCAR_NORM_HEAD = 1 } oscar_norm_scope;
typedef enum {
    OSCAR_ROT_QUERY = 0,
    OSCAR_ROT_KEY = 1,
    OSCAR_ROT_KEY_HW_RSQ = 2 /* KEY with the hardware reciprocal square root
                                (see oscar_key_scale) */
} oscar_rot_mode;
/* How the Omni-Token Scaling factor r = 1/||y|| is computed from the sum of
 * squares ss.  The popular-science article (三) replaces "L2 norm, then
 * reciprocal" by one hardware reciprocal-square-root instruction. */
typedef enum {
    OSCAR_SCALE_IEEE = 0,  /* r = 1 / sqrt(ss), each correctly rounded: k_hat,
                              norms and codes bit-exact with the reference */
    OSCAR_SCALE_HW_RSQ = 1 /* r = v_rsq_f32(ss) (about 1 ulp): k_hat within one
                              fp16 step of the IEEE result; the stored norm is
                              still the correctly rounded sqrt(ss) */
} oscar_key_scale;
typedef enum {
    OSCAR_ATTN_AUTO = 0, /* the fastest kernel built (the MFMA one) */
    OSCAR_ATTN_VALU = 1, /* scalar-FMA dot products on the vector ALUs */
    OSCAR_ATTN_MFMA = 2  /* GQA-group q.K^T and P.V tiles on the matrix cores */
} oscar_attn_variant;

/* error_flag bits */
#define OSCAR_FLAG_CAPACITY 1u  /* a block index reached max_blocks_per_seq */
#define OSCAR_FLAG_NONEMPTY 2u  /* prefill into a sequence with n != 0 */
#define OSCAR_FLAG_BADSTATE 4u  /* a block id outside the pool, or an inconsistent
                                   {n, Q}: the affected work is skipped */
#define OSCAR_FLAG_POSITION 8u  /* a token position at or beyond rope_max_pos:
                                   the append is dropped */

/* Cache geometry (host struct).  The method's fixed sizes are fields too,
 * so that a caller states them and a mismatch is an error rather than a
 * silent reinterpretation: the structured summary "OScaR：…" (方法步骤详情 and
 * 实验结果) fixes INT2 with 32-token Key blocks and 32-channel Value groups,
 * and the popular-science article (三) a 128-token fp16 residual window. */
typedef struct {
    int32_t batch;               /* B sequences */
    int32_t num_q_heads;         /* Hq */
    int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0, Hq/Hkv in {1,2,4,8} */
    int32_t head_dim;            /* must be 128 (OSCAR_HEAD_DIM) */
    int32_t block_tokens;        /* Key quantization block G: must be 32 */
    int32_t residual_tokens;     /* fp16 residual window R: must be 128 */
    int32_t v_group;             /* Value quantization group: must be 32 */
    int32_t norm_scope;          /* oscar_norm_scope: TOKEN (default) or HEAD,
                                    which sizes the two norm buffers below */
    int32_t max_blocks_per_seq;  /* block-table row length */
    int32_t num_physical_blocks; /* pool capacity */
    int32_t flush_tokens;        /* tokens quantized when the window is full:
                                    0 or 32 = one block (default), 128 = the
                                    whole window as four blocks */
    int32_t key_scale;           /* oscar_key_scale used by append and prefill:
                                    0 = IEEE (default), 1 = hardware rsqrt */
    int32_t rope_max_pos;        /* 0: queries and Keys arrive already rotated
                                    by position (RoPE applied by the caller);
                                    > 0: the library applies RoPE itself, from
                                    the table cache->rope of this many
                                    positions (see oscar_cache) */
} oscar_cache_geom;

/* Cache buffers (device pointers, caller-owned).  Layout, per the record
 * layout of the packed cache ("packed cache" + "residual cache", popular
 * science article on OScaR (animattoys.com), section 三):
 *   pool        [num_physical_blocks][Hkv][3072] bytes, 256-B aligned.  Record:
 *                 [0,1024)    K codes: channel c of token t at bits 2*(c&3) of
 *                             byte 32*t + (c>>2)
 *                 [1024,2048) V codes: slice 16*(t>>3) + (c&15) of 16 bytes at
 *                             1024 + 16*slice; 32-bit word c>>5 of it; bits
 *                             2m, 2m+1 with m = 8*((c>>4)&1) + s(t&7), s(k)
 *                             = k with its two low bits swapped
 *                 [2048,2304) K step (delta) fp16 [128]
 *                 [2304,2560) K zero point fp16 [128]
 *                 [2560,3072) V (step, zero) fp16 pairs, [4 groups][32 tokens]
 *   pool_norm   [num_physical_blocks][32] fp16 token norms (TOKEN scope), or
 *               [num_physical_blocks][Hkv][32] norms per (token, KV head) (HEAD)
 *   res_k       [B][Hkv][128 slots][128] fp16 rotated+scaled keys (k_hat)
 *   res_v       [B][Hkv][128 channels][128 slots] fp16 values
 *   res_norm    [B][128 slots] fp16 token norms (TOKEN), or [B][Hkv][128] (HEAD)
 *   block_table [B][max_blocks_per_seq] int32 physical block ids (caller fills)
 *   seq_state   [B][2] int32 = {n tokens, Q quantized tokens}; zero = empty
 *   error_flag  [1] int32 sticky bits (OSCAR_FLAG_*); caller zeroes it
 *   append_sync [B] int32, library-private (the per-sequence arrival
 *               counters of oscar_append_kv's and oscar_prefill_quantize's
 *               workgroups); caller zeroes it once, every call leaves it zero
 *   rope        NULL when geom->rope_max_pos == 0; else read-only
 *               [rope_max_pos][64][2] fp32 (cos, sin): the rotary position
 *               embedding of the model.  The popular-science article (五)
 *               names RoPE as the reason the Key and query rotation must run
 *               online: the library applies it right before the FHT, channel
 *               pairs (i, i + 64) of token position p rotated by the angle of
 *               row p, column i:  x_i <- x_i c - x_{i+64} s,
 *               x_{i+64} <- x_{i+64} c + x_i s  (fp32 products, then one add).
 *               Keys take the position of the token in its sequence (0 for
 *               the first), the query of a decode step the position of the
 *               step's own token (n - 1 after its append).
 * Token t of a sequence lives in block t/32 (t < Q) or ring slot t % 128
 * (Q <= t < n).  All buffers zero-initialised by the caller before first use. */
typedef struct {
    void *pool;
    void *pool_norm;
    void *res_k;
    void *res_v;
    void *res_norm;
    int32_t *block_table;
    int32_t *seq_state;
    int32_t *error_flag;
    int32_t *append_sync;
    const float *rope;
} oscar_cache;

/* Byte sizes of each cache buffer for a geometry. */
typedef struct {
    size_t pool, pool_norm, res_k, res_v, res_norm, block_table, seq_state, error_flag,
        append_sync;
} oscar_cache_sizes;

/* Host-only infrastructure (no defining passage: the pages fix no memory
 * layout).  Fills *out with the byte size of every cache buffer.
 * EINVAL on a null pointer or an unsupported geometry: head_dim != 128,
 * block_tokens != 32, residual_tokens != 128, v_group != 32, Hq % Hkv != 0,
 * Hq/Hkv outside {1,2,4,8}, Hkv outside 1..16, batch or block counts < 1,
 * an unknown norm_scope, flush_tokens outside {0,32,128}, an unknown
 * key_scale.  Every entry point taking a geometry validates it the same way. */
OSCAR_API oscar_status oscar_cache_layout(const oscar_cache_geom *geom, oscar_cache_sizes *out);

/* Canalized Rotation and Omni-Token Scaling on a batch of tokens (summary
 * "OScaR：…", 方法步骤详情 (1) and (2); reading notes §II Step One and
 * Step Two).
 *   x         device, [n_tokens][n_heads][128] fp16 or bf16 (dtype).
 *   mode      QUERY: q_out[n_tokens][n_heads][128] fp32 = FHT(x) per head,
 *                    exactly the oracle's fp32 butterfly (strides 1..64,
 *                    then x 1/sqrt(128)); khat_out, norm_out unused.
 *             KEY:   y = FHT(x) per head; ss = pairwise-tree sum of squares
 *                    over all heads (TOKEN) or per head (HEAD); khat_out
 *                    [n_tokens][n_heads][128] fp16 = fp16(y * (1/sqrt(ss)));
 *                    norm_out fp16 [n_tokens] (TOKEN) or [n_tokens][n_heads],
 *                    sqrt(ss) saturated at 65504.
 *             KEY_HW_RSQ: KEY with 1/sqrt(ss) from the hardware instruction
 *                    (OSCAR_SCALE_HW_RSQ).
 *   n_heads   >= 1 (QUERY), 1..16 (KEY: the norm spans all heads of a token).
 * No RoPE here: stateless inputs are taken as already rotated by position.
 * Errors: EINVAL (null, n_tokens < 0, n_heads out of range, bad dtype; for
 * KEY, x or khat_out not 16-byte aligned). */
OSCAR_API oscar_status oscar_rotate_scale(const void *x, oscar_dtype dtype, int32_t n_tokens,
                                int32_t n_heads, oscar_rot_mode mode,
                                oscar_norm_scope norm_scope, float *q_out,
                                void *khat_out, void *norm_out, void *stream);

/* Stateless INT2 quantize + pack of whole 32-token blocks (summary "OScaR：…",
 * 方法步骤详情 ②, the quantization kernel handling Keys and Values together).
 *   khat16, v16  device, [32*n_blocks][n_kv_heads][128] fp16; v16 16-byte
 *                aligned.
 *   knorm16      device, fp16 norms: [32*n_blocks] (TOKEN scope) or
 *                [32*n_blocks][n_kv_heads] (HEAD scope), as oscar_rotate_scale
 *                returns them.
 *   rec_out      device, [n_blocks][n_kv_heads][3072] records (layout above).
 *   norm_out     device, fp16 [n_blocks][32] (TOKEN) or [n_blocks][n_kv_heads][32]
 *                (HEAD).
 * Keys: per channel over the block's 32 tokens; Values: per token over each
 * 32-channel group; delta = (max-min)/3, zero = min, code =
 * clamp(rint((x-zero)/delta), 0, 3) in IEEE fp32, delta == 0 -> code 0.
 * Inputs must be finite (as every fp16 value the other entry points store
 * is); an infinite or NaN input gives unspecified codes and parameters.
 * Errors: EINVAL (null, counts out of range, rec_out or v16 not 16-byte
 * aligned). */
OSCAR_API oscar_status oscar_quant_pack(const void *khat16, const void *knorm16, const void *v16,
                              int32_t n_blocks, int32_t n_kv_heads,
                              oscar_norm_scope norm_scope, void *rec_out,
                              void *norm_out, void *stream);

/* One decode-step append for every sequence (popular-science article, 三:
 * residual cache of the newest tokens in fp16, quantized a block at a time;
 * summary 论文图表 (c)).  Per sequence b with state {n, Q}, F = flush_tokens
 * (32 by default, or 128):
 *   if n - Q == 128: quantize ring tokens Q..Q+F-1 into physical blocks
 *                    block_table[b][Q/32 ..] (or set OSCAR_FLAG_CAPACITY and
 *                    drop the append if (Q+F)/32 > max_blocks_per_seq); Q += F;
 *   rotate+scale k_new[b], store k_hat, norm and fp16(v_new[b]) in slot
 *   n % 128; n += 1.
 * One workgroup per (sequence, KV head) does that head's share (its part of
 * the flush, its row of the window); the last of a sequence's workgroups to
 * finish writes {n, Q}, counted in append_sync[b].
 * Stored fp16 values saturate: a Value entry or a norm beyond +-65504
 * (+-inf included) is stored as +-65504, a NaN Value as -65504; |k_hat| <= 1.
 *   k_new, v_new  device, [B][Hkv][128] fp16 or bf16; Keys must be finite
 *                 with a sum of squares below fp32's range.
 * Errors: EINVAL. */
OSCAR_API oscar_status oscar_append_kv(const oscar_cache_geom *geom, const oscar_cache *cache,
                             const void *k_new, const void *v_new, oscar_dtype dtype,
                             void *stream);

/* Bulk prefill of an empty sequence `seq` with n_tokens tokens (reading notes,
 * End-to-End Flow: prefill Keys pass FHT, per-token scaling and INT2
 * per-channel quantization before entering the cache).  The resulting cache
 * state is byte-identical, on its valid region, to n_tokens appends
 * (saturation included).
 *   k, v  device, [n_tokens][Hkv][128] fp16 or bf16, 16-byte aligned.
 * Errors: EINVAL (also when the blocks needed exceed max_blocks_per_seq, or
 * k / v are not 16-byte aligned);
 * device: OSCAR_FLAG_NONEMPTY if the sequence already holds tokens. */
OSCAR_API oscar_status oscar_prefill_quantize(const oscar_cache_geom *geom, const oscar_cache *cache,
                                    int32_t seq, const void *k, const void *v,
                                    int32_t n_tokens, oscar_dtype dtype, void *stream);

/* Infrastructure (no defining passage): the split count the library would
 * pick for max_ctx (num_splits == 0) and the workspace bytes decode attention
 * needs with that split count.  Host-only.
 * Errors: EINVAL (bad geometry, null bytes, max_ctx < 0, num_splits outside
 * 0..1024). */
OSCAR_API oscar_status oscar_decode_workspace_bytes(const oscar_cache_geom *geom, int32_t max_ctx,
                                          int32_t num_splits, int32_t *splits_out,
                                          size_t *bytes);

/* Split-K decode attention over the INT2 cache (summary "OScaR：…",
 * 方法步骤详情 ③: fused dequantization, inverse scaling and attention;
 * reading notes, End-to-End Flow).  For sequence b and query head i, with
 * KV head h = i / (Hq/Hkv) and the n cached tokens (the step's own token
 * included): out = softmax(q' K^T / sqrt(128)) V where q' = FHT(q) and
 * K, V are the dequantized, un-scaled rows in the rotated basis.
 *   q        device, [B][Hq][128]: fp16/bf16 raw queries (rotated in the
 *            kernel), or fp32 already-rotated q' (dtype OSCAR_FP32).
 *   out      device, [B][Hq][128] fp32 (rotated-V basis).
 *   lse      device, [B][Hq] fp32 log-sum-exp of the scaled scores, or NULL.
 *   workspace device, >= oscar_decode_workspace_bytes(...) bytes, 256-B aligned,
 *            zero-filled by the caller once, before its first use.  Its
 *            first 256 KiB hold one arrival counter per (sequence, KV head)
 *            for the cross-split merge that the launch does itself (B * Hkv
 *            <= 65536); every call leaves them zero again, so the workspace
 *            stays valid for any later call whose size fits (any geometry or
 *            split count).  The rest holds the per-split partials (m, l, o)
 *            and, for a batch of 2..1024 sequences, the launch order
 *            (sequences longest first, with their {n, Q}), rewritten by
 *            every call.  Two calls in flight at the same time
 *            must not share a workspace.
 *   num_splits  0 = pick from max_ctx; else 1..1024 splits per (b, KV head).
 *   variant  AUTO / MFMA: one launch (matrix-core attention; the last split
 *            of each (b, KV head) to finish merges all of them); VALU: the
 *            vector-ALU kernel and a separate merge launch.
 *   max_ctx  an upper bound on every sequence's n (used to size the split).
 * Errors: EINVAL (also B * Hkv > 65536), EWORKSPACE, ELAUNCH. */
OSCAR_API oscar_status oscar_decode_attn(const oscar_cache_geom *geom, const oscar_cache *cache,
                               const void *q, oscar_dtype q_dtype, float *out, float *lse,
                               void *workspace, size_t ws_bytes, int32_t num_splits,
                               int32_t max_ctx, oscar_attn_variant variant, void *stream);

/* One whole decode step in one launch: the same result as oscar_append_kv
 * (k_new, v_new) followed by oscar_decode_attn (q) on the same stream -- the
 * cache left byte for byte as the append leaves it, the same flags, and the
 * same out and lse -- for the steps the pages describe (popular-science
 * article, 三: the newest token joins the fp16 residual cache, a full window
 * is quantized a block at a time; summary "OScaR：…", 方法步骤详情 ③: fused
 * attention over the INT2 blocks and the window).  Inside the launch each
 * sequence's attention covers the state the append leaves: the workgroup
 * whose window chunk holds the new token rotates and scales it itself, a
 * block that a full window flushes is quantized by the workgroup whose
 * split holds it (and written to the pool before its copy), and the stores
 * that overwrite slots other workgroups read (the new token's window rows
 * and norm, {n, Q}) are made by the last of the sequence's workgroups to
 * finish those reads (counted in append_sync[b]).
 *   k_new, v_new, kv_dtype  as oscar_append_kv;
 *   q, q_dtype, out, lse, workspace, ws_bytes, num_splits, max_ctx, variant
 *            as oscar_decode_attn (max_ctx bounds n after the append).
 *            VALU: the append and then attention, two launches.
 * Errors: as oscar_append_kv and oscar_decode_attn. */
OSCAR_API oscar_status oscar_decode_step(const oscar_cache_geom *geom, const oscar_cache *cache,
                               const void *k_new, const void *v_new, oscar_dtype kv_dtype,
                               const void *q, oscar_dtype q_dtype, float *out, float *lse,
                               void *workspace, size_t ws_bytes, int32_t num_splits,
                               int32_t max_ctx, oscar_attn_variant variant, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation:
 * oscar_decode_attn with its workspace taken from a library-owned device
 * array (one per GPU, OSCAR_STATIC_WORKSPACE_BYTES = 8 MiB, held until the
 * process ends) instead of an argument.  Same arguments (less the
 * workspace), kernels and results as oscar_decode_attn.  Allocates nothing.
 * The array's merge counters are cleared by a fill kernel enqueued on
 * `stream` by the first call on each GPU, and every call leaves them zero.
 * Calls on one GPU share its array: calls that overlap in time on one GPU
 * (different streams, or one graph replayed on two streams) race.
 * Errors: as oscar_decode_attn, and OSCAR_EWORKSPACE when the workspace the
 * geometry and split count need (oscar_decode_workspace_bytes) exceeds
 * OSCAR_STATIC_WORKSPACE_BYTES (e.g. 48 sequences with 1024 splits). */
#define OSCAR_STATIC_WORKSPACE_BYTES ((size_t)8 << 20)
OSCAR_API oscar_status oscar_decode_attn_noalloc(const oscar_cache_geom *geom,
                                                 const oscar_cache *cache, const void *q,
                                                 oscar_dtype q_dtype, float *out, float *lse,
                                                 int32_t num_splits, int32_t max_ctx,
                                                 oscar_attn_variant variant, void *stream);

/* ---------------------------------------------------------------------------
 * The BF16 baseline: decode attention over an unquantized bf16 cache, the
 * comparison point of the pages' efficiency results (summary "OScaR：…",
 * 实验结果 and 论文图表: decode speed-up over BF16 FlashDecoding-v2 at long
 * context; popular-science article, 四: batch-48 memory and throughput).
 * Same split-K structure and log-sum-exp reduce as oscar_decode_attn; no
 * rotation, scaling or quantization.  The geometry's norm_scope and
 * flush_tokens are not used (any accepted value, e.g. 0, will do).
 *
 * Paged bf16 layout, per (physical block p, KV head h) of 32 tokens:
 *   k_pool  [P][Hkv][32 tokens][128 channels] bf16 (P = num_physical_blocks)
 *   v_pool  [P][Hkv][128 channels][32 tokens] bf16 (transposed per block)
 * Token t of sequence b lives in block block_table[b][t / 32], row t % 32.
 * ------------------------------------------------------------------------- */

/* Write tokens start .. start + n_tokens - 1 of sequence `seq` into the bf16
 * pools (a plain layout transform; the cache a model's attention layer would
 * write).
 *   k, v         device, [n_tokens][Hkv][128] bf16, 16-byte aligned.
 *   k_pool, v_pool device, 256-byte aligned; block_table device [B][max_blocks].
 *   error_flag   device int32: OSCAR_FLAG_BADSTATE for a block id outside
 *                [0, num_physical_blocks) (that token is skipped).
 * Errors: EINVAL (also when start + n_tokens > 32 * max_blocks_per_seq). */
OSCAR_API oscar_status oscar_dense_write_kv(const oscar_cache_geom *geom, void *k_pool, void *v_pool,
                                  const int32_t *block_table, int32_t seq, int32_t start,
                                  const void *k, const void *v, int32_t n_tokens,
                                  int32_t *error_flag, void *stream);

/* Infrastructure (no defining passage): the split count the bf16 kernel
 * would pick for max_ctx (num_splits == 0) and the workspace bytes it needs
 * with that split count.  Host-only; errors as for
 * oscar_decode_workspace_bytes. */
OSCAR_API oscar_status oscar_dense_workspace_bytes(const oscar_cache_geom *geom, int32_t max_ctx,
                                         int32_t num_splits, int32_t *splits_out,
                                         size_t *bytes);

/* out[b][i] = softmax(q[b][i] K_h^T / sqrt(128)) V_h over the ctx_lens[b]
 * tokens of sequence b, h = i / (Hq/Hkv).
 *   q          device, [B][Hq][128] bf16, 16-byte aligned (not rotated).
 *   ctx_lens   device, [B] int32 tokens per sequence (0 gives zeros and
 *              lse = -inf; above 32 * max_blocks_per_seq sets
 *              OSCAR_FLAG_BADSTATE and attends to nothing).
 *   out, lse, workspace, num_splits, max_ctx: as for oscar_decode_attn, with
 *              the workspace from oscar_dense_workspace_bytes.
 *   error_flag device int32 sticky bits: OSCAR_FLAG_BADSTATE for a block id
 *              outside the pool (block 0 is read instead).
 * Errors: EINVAL, EWORKSPACE, ELAUNCH. */
OSCAR_API oscar_status oscar_dense_decode_attn(const oscar_cache_geom *geom, const void *k_pool,
                                     const void *v_pool, const int32_t *block_table,
                                     const int32_t *ctx_lens, const void *q, float *out,
                                     float *lse, void *workspace, size_t ws_bytes,
                                     int32_t num_splits, int32_t max_ctx, int32_t *error_flag,
                                     void *stream);

/* Infrastructure (no defining passage): a static, never-freed string naming
 * a status code ("unknown status" for any other value).  Host-only. */
/* Offline absorption of the Value rotation into the projection weights
 * (reading notes §II Step One, query-side symmetric processing; summary
 * "OScaR：…", 方法步骤详情 (3)).  Keeping V' = H V per KV head in the cache
 * takes W_v' = H W_v, and the attention output, which is then H o per query
 * head, is turned back by W_o' = W_o H; after this one-time transform the
 * Value rotation costs nothing at decode time.  H is the 128-point Sylvester
 * Hadamard matrix times 1/sqrt(128) (symmetric, its own inverse), applied as
 * the plain fp32 butterfly, strides 1..64, then x fp32(1/sqrt(128)).
 *   w, out   device, row-major fp32 [rows][cols]; out may equal w (in place).
 *   axis 0   every column of every 128-row block is replaced by H times it:
 *            W_v' for W_v stored [Hkv*128][d_model] (nn.Linear layout).
 *   axis 1   every 128-column block of every row is replaced by it times H:
 *            W_o' for W_o stored [d_model][Hq*128]; also a Value bias b_v
 *            taken as [1][Hkv*128] (H b = b H).
 * Errors: EINVAL (null, negative sizes, axis not 0 or 1, rows (axis 0) or
 * cols (axis 1) not a multiple of 128, a grid beyond 2^31 - 1 blocks). */
OSCAR_API oscar_status oscar_absorb_value_rotation(const float *w, float *out, int64_t rows,
                                                   int64_t cols, int32_t axis, void *stream);

OSCAR_API const char *oscar_status_str(oscar_status s);

#ifdef __cplusplus
}
#endif
#endif
