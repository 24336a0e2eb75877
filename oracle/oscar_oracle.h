/*
 * oscar_oracle.h -- plain CPU oracle of the OScaR INT2 KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls it, and it shares no code with the GPU library.
 *
 * Sources (web pages about OScaR, arXiv 2605.19660), cited by tag:
 *   [RN]  reading notes "OScaR: The Occam's Razor for Extreme KV Cache
 *         Quantization in LLMs and Beyond" (yingwang.github.io paper-reads)
 *   [SUM] structured summary "OScaR：面向大模型及多模态LLM极限KV缓存量化的奥卡姆剃刀"
 *         (paper.rainbus.top)
 *   [POP] popular-science article on OScaR (animattoys.com), sections 一 to 五
 *   [ABS] abstract (chatpaper.ai)
 *
 * Fixed hyper-parameters: head dim d=128, INT2, Key block G=32 tokens,
 * Value group 32 channels, residual window R=128 ([SUM] 方法步骤详情 and
 * 实验结果; [POP] 三).
 */
#ifndef OSCAR_ORACLE_H
#define OSCAR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORC_D = 128,          /* head dim */
    ORC_G = 32,           /* Key quantization block, tokens */
    ORC_R = 128,          /* residual window, tokens */
    ORC_VG = 32,          /* Value quantization group, channels */
    ORC_REC_BYTES = 3072  /* one (physical block, KV head) record */
};
enum { ORC_FP16 = 0, ORC_BF16 = 1 };
enum { ORC_NORM_TOKEN = 0, ORC_NORM_HEAD = 1 };

/* Record layout, byte offsets inside one (physical block, KV head) record. */
enum {
    ORC_REC_KCODES = 0,     /* 1024 B: 32 tokens x 128 channels x 2 bit */
    ORC_REC_VCODES = 1024,  /* 1024 B: 32 tokens x 128 channels x 2 bit */
    ORC_REC_KDELTA = 2048,  /* 128 x fp16 step per channel */
    ORC_REC_KZERO = 2304,   /* 128 x fp16 zero point per channel */
    ORC_REC_VPARAM = 2560   /* [4 groups][32 tokens] x (step, zero) fp16 */
};

/* The cache state.  Every array is caller-owned, zero-initialised. */
typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, norm_scope;
    int32_t max_blocks_per_seq, num_physical_blocks;
    int32_t flush_tokens;   /* tokens quantized per flush: 32 (one block) or 128 */
    uint8_t *pool;          /* [num_physical_blocks][Hkv][3072] */
    uint16_t *pool_norm;    /* TOKEN: [num_physical_blocks][32]; HEAD: [..][Hkv][32] */
    uint16_t *res_k;        /* [B][Hkv][128 slots][128] fp16 */
    uint16_t *res_v;        /* [B][Hkv][128 channels][128 slots] fp16 */
    uint16_t *res_norm;     /* TOKEN: [B][128 slots]; HEAD: [B][Hkv][128 slots] */
    const int32_t *block_table; /* [B][max_blocks_per_seq] physical block ids */
    int32_t *seq_state;     /* [B][2] = {n tokens, Q quantized tokens} */
    int32_t *error_flag;    /* sticky bit 1: block table capacity exceeded;
                               bit 8: a position beyond the RoPE table */
    const float *rope;      /* NULL, or [rope_max_pos][64] (cos, sin) pairs:
                               Keys are rotated by position before the FHT */
    int32_t rope_max_pos;
} orc_cache;

/* number conversions */
uint16_t orc_f32_to_f16(float f);
uint16_t orc_f32_to_f16_sat(float f);  /* clamp to +-65504, then round */
float orc_f16_to_f32(uint16_t h);
float orc_bf16_to_f32(uint16_t b);
float orc_in_to_f32(uint16_t x, int dtype);
void orc_to_f16(const uint16_t *x, int dtype, size_t n, uint16_t *out);

/* Canalized Rotation */
float orc_fht_scale(void);
void orc_fht128(float *x);
void orc_rotate_query(const uint16_t *q, int dtype, size_t n_vec, float *out);

/* rotary position embedding of one 128-vector: pairs (i, i + 64) rotated by
 * the angle whose (cos, sin) is cs[2i], cs[2i + 1] */
void orc_rope(float *x, const float *cs);
void orc_rotate_query_pos(const uint16_t *q, int dtype, size_t n_vec,
                          const float *cs, float *out);

/* offline absorption of the Value rotation into weights: the FHT over every
 * 128-block along axis 0 (rows: W_v [H*128][cols]) or axis 1 (columns:
 * W_o [rows][H*128]) of a row-major fp32 matrix */
void orc_absorb_value_rotation(const float *w, float *out, int rows, int cols,
                               int axis);

/* Omni-Token Scaling */
float orc_tree_sumsq(const float *y, int n);
void orc_rotate_scale_key(const uint16_t *k, int dtype, int n_tokens, int hkv,
                          int norm_scope, uint16_t *khat, uint16_t *norm);
/* the same with RoPE first: token t at position pos0 + t, cos/sin from rope
 * ([positions][64] pairs; NULL = no RoPE) */
void orc_rotate_scale_key_pos(const uint16_t *k, int dtype, int n_tokens, int hkv,
                              int norm_scope, const float *rope, int pos0,
                              uint16_t *khat, uint16_t *norm);

/* INT2 quantizer on one group of 32 fp16 values taken with a stride */
void orc_quant_group32(const uint16_t *x16, size_t stride, float *delta,
                       float *zero, uint8_t *codes);

/* packed layout accessors */
size_t orc_kcode_byte(int t, int c);
int orc_kcode_shift(int t, int c);
size_t orc_vcode_byte(int t, int c);
int orc_vcode_shift(int t, int c);
int orc_kcode_get(const uint8_t *rec, int t, int c);
int orc_vcode_get(const uint8_t *rec, int t, int c);

/* Stateless block quantizer.  khat, v16: [32 * n_blocks][Hkv][128] fp16;
 * knorm: TOKEN [32 * n_blocks], HEAD [32 * n_blocks][Hkv].
 * rec_out: [n_blocks][Hkv][3072]; norm_out: TOKEN [n_blocks][32],
 * HEAD [n_blocks][Hkv][32]. */
void orc_quant_pack(const uint16_t *khat, const uint16_t *knorm,
                    const uint16_t *v16, int n_blocks, int hkv, int norm_scope,
                    uint8_t *rec_out, uint16_t *norm_out);

/* Residual-window state machine */
void orc_append(orc_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                int dtype);
void orc_append_one(orc_cache *c, int b, const uint16_t *k_tok,
                    const uint16_t *v_tok, int dtype);
int orc_prefill(orc_cache *c, int b, const uint16_t *k, const uint16_t *v,
                int n_tokens, int dtype);

/* dequantized cache rows (fp64) */
void orc_key_row(const orc_cache *c, int b, int h, int t, double *out);
void orc_value_row(const orc_cache *c, int b, int h, int t, double *out);

/* decode attention, fp64 accumulation */
void orc_decode_attn(const orc_cache *c, const float *qrot, float *out,
                     float *lse);
void orc_decode_attn_one(const orc_cache *c, const float *qrot, int b, int i,
                         float *out, float *lse);
/* split-K pieces: a partial (m, l, o) over tokens [t0, t1), and the merge */
void orc_decode_attn_partial(const orc_cache *c, const float *qrot, int b, int i,
                             int t0, int t1, double *m_out, double *l_out,
                             double *o_out);
void orc_lse_merge(int n_parts, const double *m, const double *l,
                   const double *o, float *out, float *lse);

/* unquantized decode attention of one sequence (the BF16 baseline), fp64:
 * q [Hq][128], k and v [n][Hkv][128], out [Hq][128], lse [Hq] or NULL */
void orc_dense_attn(const float *q, const float *k, const float *v, int n,
                    int hq, int hkv, float *out, float *lse);

#ifdef __cplusplus
}
#endif
#endif
