/*
 * oscar_oracle.c -- plain CPU oracle of the OScaR INT2 KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oscar_oracle.h): loaded by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Written for readability, not speed: scalar loops, one step at a time, in the
 * order the pages give them.  Build with gcc -O2 -ffp-contract=off and no
 * fast-math, so that every fp32 operation below is one IEEE operation with
 * round-to-nearest-even and nothing is fused.
 *
 * Where the pages leave a step open, the reading taken here is stated beside
 * the code.  Citation tags ([RN], [SUM], [POP]) are defined in the header.
 */
#include "oscar_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number conversions                                                        */
/* ------------------------------------------------------------------------ */

/* fp32 -> IEEE binary16, round to nearest, ties to even.  Written from the
 * binary16 definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; subnormals are multiples of 2^-24.  nearbyint() rounds ties to even
 * in the default rounding mode. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    double a = fabs((double)f);
    if (isnan(a))
        return (uint16_t)(sign | 0x7e00u);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);
    int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal range: value = m * 2^-24; m == 1024 becomes the
         * smallest normal number, whose bit pattern is exactly 0x0400 */
        double m = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    double m = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* fp32 -> binary16 for a stored value (a Value row entry, a token norm):
 * the value is first clamped to the finite binary16 range [-65504, 65504],
 * then rounded as above, so a stored value is never infinite.  The pages
 * only say the residual cache holds FP16 ([POP] 三); what happens to a bf16
 * input beyond FP16's range is a reading: it saturates.  fmaxf returns its
 * other operand for a NaN, so a NaN input is stored as -65504. */
uint16_t orc_f32_to_f16_sat(float f)
{
    return orc_f32_to_f16(fminf(fmaxf(f, -65504.0f), 65504.0f));
}

float orc_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);
}

/* bfloat16 is the top half of an fp32 bit pattern. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

float orc_in_to_f32(uint16_t x, int dtype)
{
    return dtype == ORC_BF16 ? orc_bf16_to_f32(x) : orc_f16_to_f32(x);
}

/* Values enter the cache in fp16 ([POP] 三: the residual cache holds full
 * precision FP16).  bf16/fp16 -> fp32 is exact; fp32 -> fp16 saturates and
 * rounds RNE (orc_f32_to_f16_sat). */
void orc_to_f16(const uint16_t *x, int dtype, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = orc_f32_to_f16_sat(orc_in_to_f32(x[i], dtype));
}

/* ------------------------------------------------------------------------ */
/* Canalized Rotation: the 128-point fast Hadamard transform                 */
/* ------------------------------------------------------------------------ */

/* fp32(1/sqrt(128)): the orthonormal Hadamard matrix has entries +-1/sqrt(d)
 * ([RN] §II Method, Step One: Canalized Rotation). */
float orc_fht_scale(void)
{
    return (float)(1.0 / sqrt(128.0));
}

/* In-place FHT of 128 fp32 values: butterflies with strides 1, 2, 4, ..., 64
 * (ascending), pair (j, j+h) -> (a+b, a-b), then one multiply by 1/sqrt(128).
 * The result is the Sylvester-ordered Hadamard matrix, normalised to be
 * orthonormal, applied to x; it costs O(d log d) ([SUM] 前置知识 on FHT;
 * [POP] 二; [RN] §II Step One).  The stride order is a reading: the pages do
 * not fix one, and any order gives the same matrix in exact arithmetic. */
void orc_fht128(float *x)
{
    for (int h = 1; h < ORC_D; h <<= 1) {
        for (int j = 0; j < ORC_D; j++) {
            if (j & h)
                continue;
            float a = x[j], b = x[j + h];
            x[j] = a + b;
            x[j + h] = a - b;
        }
    }
    const float c = orc_fht_scale();
    for (int i = 0; i < ORC_D; i++)
        x[i] = x[i] * c;
}

/* Query side: q' = H q for every query head, no scaling, so that the Key
 * rotation cancels inside q.k ([SUM] 方法步骤详情 (1); [POP] 二 and Q2;
 * [RN] §II, Query-side symmetric processing).  q: [n_vec][128], out fp32. */
void orc_rotate_query(const uint16_t *q, int dtype, size_t n_vec, float *out)
{
    for (size_t v = 0; v < n_vec; v++) {
        float *y = out + v * ORC_D;
        for (int c = 0; c < ORC_D; c++)
            y[c] = orc_in_to_f32(q[v * ORC_D + c], dtype);
        orc_fht128(y);
    }
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding (the reason the rotation must be online)       */
/* ------------------------------------------------------------------------ */

/* The model rotates queries and Keys by their position (RoPE) before they
 * reach the cache, which is why the Hadamard rotation cannot be folded into
 * the projection weights offline and has to run online after it ([POP] 五).
 * The pages do not give RoPE's form; this is the common "rotate half" form:
 * channels i and i + 64 (i < 64) form a pair rotated by an angle whose cosine
 * and sine are cs[2i], cs[2i + 1] (a caller-supplied table, so that every
 * implementation multiplies by the same numbers):
 *     x[i]      <- x[i] c - x[i + 64] s
 *     x[i + 64] <- x[i + 64] c + x[i] s
 * each product rounded to fp32, then one fp32 add or subtract. */
void orc_rope(float *x, const float *cs)
{
    for (int i = 0; i < ORC_D / 2; i++) {
        const float a = x[i], b = x[i + ORC_D / 2];
        const float c = cs[2 * i], s = cs[2 * i + 1];
        const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        x[i] = ac - bs;
        x[i + ORC_D / 2] = bc + as;
    }
}

/* Query side with RoPE: every vector at the position whose (cos, sin) row is
 * cs (NULL: no RoPE), then the FHT. */
void orc_rotate_query_pos(const uint16_t *q, int dtype, size_t n_vec,
                          const float *cs, float *out)
{
    for (size_t v = 0; v < n_vec; v++) {
        float *y = out + v * ORC_D;
        for (int c = 0; c < ORC_D; c++)
            y[c] = orc_in_to_f32(q[v * ORC_D + c], dtype);
        if (cs)
            orc_rope(y, cs);
        orc_fht128(y);
    }
}

/* The Value rotation is absorbed into the weights offline: V' = H V per KV
 * head means W_v' = H W_v (the FHT down each 128-row block of every column),
 * and the attention output o' = H o is turned back by W_o' = W_o H (the FHT
 * along each 128-column block of every row; H is symmetric) ([SUM]
 * 方法步骤详情 (3); [RN] §II Step One, Query-side symmetric processing).
 * w, out: row-major fp32 [rows][cols]; axis 0 needs rows % 128 == 0, axis 1
 * cols % 128 == 0. */
void orc_absorb_value_rotation(const float *w, float *out, int rows, int cols,
                               int axis)
{
    float x[ORC_D];
    if (axis == 0) {
        for (int h = 0; h < rows / ORC_D; h++)
            for (int j = 0; j < cols; j++) {
                for (int i = 0; i < ORC_D; i++)
                    x[i] = w[(size_t)(h * ORC_D + i) * cols + j];
                orc_fht128(x);
                for (int i = 0; i < ORC_D; i++)
                    out[(size_t)(h * ORC_D + i) * cols + j] = x[i];
            }
    } else {
        for (int r = 0; r < rows; r++)
            for (int h = 0; h < cols / ORC_D; h++) {
                for (int i = 0; i < ORC_D; i++)
                    x[i] = w[(size_t)r * cols + h * ORC_D + i];
                orc_fht128(x);
                for (int i = 0; i < ORC_D; i++)
                    out[(size_t)r * cols + h * ORC_D + i] = x[i];
            }
    }
}

/* ------------------------------------------------------------------------ */
/* Omni-Token Scaling                                                        */
/* ------------------------------------------------------------------------ */

/* Sum of squares of n fp32 values by a pairwise tree: square each value
 * (one fp32 multiply), zero-pad to a power of two, then at level s = 1, 2,
 * 4, ... set a[i] = a[i] + a[i+s] for every i that is a multiple of 2s.  The
 * pages only ask for the L2 norm; the tree fixes one summation order. */
float orc_tree_sumsq(const float *y, int n)
{
    int p = 1;
    while (p < n)
        p <<= 1;
    float *a = (float *)calloc((size_t)p, sizeof(float));
    for (int i = 0; i < n; i++)
        a[i] = y[i] * y[i];
    for (int s = 1; s < p; s <<= 1)
        for (int i = 0; i + s < p; i += 2 * s)
            a[i] = a[i] + a[i + s];
    float r = a[0];
    free(a);
    return r;
}

/* Key side: rotate each KV head's 128 values with the FHT, then divide the
 * token by its L2 norm and keep the norm ([RN] §II Step Two: the norm of k_i
 * is taken over all heads, k_i in R^{H*d_h}; [POP] 二: divide each token by
 * its own norm so its energy becomes 1, store the norm as a tag; [SUM]
 * 方法步骤详情 (2)).
 *   TOKEN scope (default): one norm over the token's Hkv*128 rotated values,
 *                          index h*128 + c.
 *   HEAD scope (variant):  one norm per KV head over its 128 values.
 * r = 1/sqrt(ss) with IEEE fp32 sqrt and divide; k_hat = fp16(y * r);
 * norm = fp16(sqrt(ss)), saturated at 65504 like every stored fp16 value
 * (|k_hat| <= 1 needs no clamp).  ss == 0 gives r = 0, k_hat = 0, norm = 0.
 * k: [n_tokens][hkv][128]; khat: same shape fp16; norm: TOKEN [n_tokens],
 * HEAD [n_tokens][hkv]. */
void orc_rotate_scale_key(const uint16_t *k, int dtype, int n_tokens, int hkv,
                          int norm_scope, uint16_t *khat, uint16_t *norm)
{
    orc_rotate_scale_key_pos(k, dtype, n_tokens, hkv, norm_scope, NULL, 0, khat, norm);
}

void orc_rotate_scale_key_pos(const uint16_t *k, int dtype, int n_tokens, int hkv,
                              int norm_scope, const float *rope, int pos0,
                              uint16_t *khat, uint16_t *norm)
{
    const int w = hkv * ORC_D;
    float *y = (float *)malloc(sizeof(float) * (size_t)w);
    for (int t = 0; t < n_tokens; t++) {
        const uint16_t *kt = k + (size_t)t * w;
        for (int i = 0; i < w; i++)
            y[i] = orc_in_to_f32(kt[i], dtype);
        for (int h = 0; h < hkv; h++) {
            if (rope)
                orc_rope(y + h * ORC_D, rope + (size_t)(pos0 + t) * ORC_D);
            orc_fht128(y + h * ORC_D);
        }
        int groups = norm_scope == ORC_NORM_TOKEN ? 1 : hkv;
        int glen = norm_scope == ORC_NORM_TOKEN ? w : ORC_D;
        for (int g = 0; g < groups; g++) {
            float ss = orc_tree_sumsq(y + g * glen, glen);
            float s = sqrtf(ss);
            float r = ss > 0.0f ? 1.0f / s : 0.0f;
            for (int i = 0; i < glen; i++)
                khat[(size_t)t * w + g * glen + i] = orc_f32_to_f16(y[g * glen + i] * r);
            norm[(size_t)t * groups + g] = orc_f32_to_f16_sat(s);
        }
    }
    free(y);
}

/* ------------------------------------------------------------------------ */
/* INT2 quantizer                                                            */
/* ------------------------------------------------------------------------ */

/* Asymmetric min-max INT2 over 32 fp16 values: delta = (max - min) / 3,
 * zero = min, code = clamp(round((x - zero) / delta), 0, 3) with round half
 * to even; delta == 0 (a constant group) gives code 0 everywhere.  This is
 * the per-channel (Key) / per-token (Value) quantizer of the KIVI paradigm
 * that OScaR keeps ([SUM] 前置知识 on per-channel quantization, 方法步骤详情
 * (2) and (3); [RN] §I: shared step delta and zero point z).  The pages do
 * not state the rounding rule or the delta == 0 case; both are readings. */
void orc_quant_group32(const uint16_t *x16, size_t stride, float *delta,
                       float *zero, uint8_t *codes)
{
    float x[32];
    for (int t = 0; t < 32; t++)
        x[t] = orc_f16_to_f32(x16[t * stride]);
    float mn = x[0], mx = x[0];
    for (int t = 1; t < 32; t++) {
        if (x[t] < mn)
            mn = x[t];
        if (x[t] > mx)
            mx = x[t];
    }
    /* -0 and +0 compare equal, so which of them a scan keeps depends on the
     * scan order; adding +0 turns a zero minimum or maximum into +0 (reading:
     * the stored zero point of a group whose minimum is zero is +0). */
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    float d = (mx - mn) / 3.0f;
    for (int t = 0; t < 32; t++) {
        int q = 0;
        if (d > 0.0f) {
            /* clamp to [0, 3]; fmaxf maps a NaN quotient (possible only for
             * non-finite inputs) to 0, so the conversion is always defined */
            float r = fminf(fmaxf(rintf((x[t] - mn) / d), 0.0f), 3.0f);
            q = (int)r;
        }
        codes[t] = (uint8_t)q;
    }
    *delta = d;
    *zero = mn;
}

/* ------------------------------------------------------------------------ */
/* Packed layout of one (physical block, KV head) record                     */
/* ------------------------------------------------------------------------ */
/*
 * K codes, bytes [0, 1024): token-major rows of 32 bytes; channel c of token
 *   t sits at bits 2*(c & 3) of byte 32*t + (c >> 2).
 * V codes, bytes [1024, 2048): 64 slices of 16 bytes.  Slice number
 *   16*(t >> 3) + (c & 15) holds tokens 8*(t>>3) .. +7 of channels
 *   c & 15, 16 + (c & 15), ..., 112 + (c & 15).  Inside a slice, 32-bit word
 *   d = c >> 5 holds the two 16-channel tiles 2d, 2d+1; the code of token
 *   slot k = t & 7 of tile e = (c >> 4) & 1 sits at position
 *   m = 8e + s(k) of that little-endian word (bits 2m, 2m+1), where s(k)
 *   swaps the two low bits of k: s = 0,2,1,3,4,6,5,7.
 *   (The layout is this code's own choice; the pages do not define one.  It
 *   puts the 8 codes of 8 consecutive tokens of one channel in one 16-bit
 *   half word, in the order in which splitting the word into even and odd
 *   2-bit fields yields consecutive token pairs.)
 * K step/zero: fp16 [128] each at 2048 / 2304.
 * V step/zero: fp16 pairs (step, zero) at 2560 + 4*(32*g + t), g = c >> 5
 *   (group-major, so the pairs of 8 consecutive tokens of one group are 32
 *   contiguous bytes).
 */
size_t orc_kcode_byte(int t, int c) { return (size_t)(32 * t + (c >> 2)); }
int orc_kcode_shift(int t, int c)
{
    (void)t;
    return 2 * (c & 3);
}

static int vcode_bit(int t, int c)
{
    int k = t & 7, e = (c >> 4) & 1;
    int sk = (k & 4) | ((k & 1) << 1) | ((k >> 1) & 1);
    return 2 * (8 * e + sk);
}

size_t orc_vcode_byte(int t, int c)
{
    int g = t >> 3, c16 = c & 15, d = c >> 5;
    int slice = 16 * g + c16;
    return (size_t)(ORC_REC_VCODES + 16 * slice + 4 * d + (vcode_bit(t, c) >> 3));
}
int orc_vcode_shift(int t, int c)
{
    return vcode_bit(t, c) & 7;
}

int orc_kcode_get(const uint8_t *rec, int t, int c)
{
    return (rec[orc_kcode_byte(t, c)] >> orc_kcode_shift(t, c)) & 3;
}
int orc_vcode_get(const uint8_t *rec, int t, int c)
{
    return (rec[orc_vcode_byte(t, c)] >> orc_vcode_shift(t, c)) & 3;
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* Quantize one 32-token block of one KV head into a record.
 *   khat_t(t, c), v_t(t, c): fp16 of token t (0..31), channel c.
 * Keys: per channel over the 32 tokens ([SUM] 方法步骤详情 (2), block size
 * G=32).  Values: per token over 32-channel groups ([SUM] 实验结果: group
 * size 32; [RN] §II: per-token Value quantization).  Steps and zero points
 * are stored fp16 (a reading: the pages do not give their precision); the
 * codes are decided from the fp32 step and zero point. */
static void quant_record(const uint16_t *khat, size_t k_tstride,
                         const uint16_t *v16, size_t v_tstride, size_t v_cstride,
                         uint8_t *rec)
{
    memset(rec, 0, ORC_REC_BYTES);
    uint8_t codes[32];
    float d, z;
    for (int c = 0; c < ORC_D; c++) {
        orc_quant_group32(khat + c, k_tstride, &d, &z, codes);
        for (int t = 0; t < 32; t++)
            rec[orc_kcode_byte(t, c)] |= (uint8_t)(codes[t] << orc_kcode_shift(t, c));
        put_u16(rec + ORC_REC_KDELTA + 2 * c, orc_f32_to_f16(d));
        put_u16(rec + ORC_REC_KZERO + 2 * c, orc_f32_to_f16(z));
    }
    for (int t = 0; t < 32; t++) {
        for (int g = 0; g < ORC_D / ORC_VG; g++) {
            const uint16_t *x = v16 + t * v_tstride + (size_t)(g * ORC_VG) * v_cstride;
            orc_quant_group32(x, v_cstride, &d, &z, codes);
            for (int i = 0; i < 32; i++) {
                int c = g * ORC_VG + i;
                rec[orc_vcode_byte(t, c)] |= (uint8_t)(codes[i] << orc_vcode_shift(t, c));
            }
            put_u16(rec + ORC_REC_VPARAM + 4 * (32 * g + t), orc_f32_to_f16(d));
            put_u16(rec + ORC_REC_VPARAM + 4 * (32 * g + t) + 2, orc_f32_to_f16(z));
        }
    }
}

void orc_quant_pack(const uint16_t *khat, const uint16_t *knorm,
                    const uint16_t *v16, int n_blocks, int hkv, int norm_scope,
                    uint8_t *rec_out, uint16_t *norm_out)
{
    const size_t w = (size_t)hkv * ORC_D;
    for (int j = 0; j < n_blocks; j++) {
        for (int h = 0; h < hkv; h++) {
            const uint16_t *kb = khat + (size_t)(32 * j) * w + (size_t)h * ORC_D;
            const uint16_t *vb = v16 + (size_t)(32 * j) * w + (size_t)h * ORC_D;
            quant_record(kb, w, vb, w, 1,
                         rec_out + ((size_t)j * hkv + h) * ORC_REC_BYTES);
        }
        for (int t = 0; t < 32; t++) {
            if (norm_scope == ORC_NORM_TOKEN)
                norm_out[(size_t)j * 32 + t] = knorm[(size_t)(32 * j + t)];
            else
                for (int h = 0; h < hkv; h++)
                    norm_out[((size_t)j * hkv + h) * 32 + t] =
                        knorm[(size_t)(32 * j + t) * hkv + h];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Residual window state machine                                             */
/* ------------------------------------------------------------------------ */
/*
 * Per sequence: n tokens appended, Q of them quantized (a multiple of 32);
 * the newest n - Q tokens sit in a ring of 128 fp16 slots, token t in slot
 * t mod 128 ([POP] 三: the residual cache holds the newest tokens not yet
 * forming a quantization block, FP16, and is quantized in batch once it holds
 * 128; [SUM] 论文图表 (c): new tokens enter the R=128 window and are
 * quantized a whole block at a time).
 * Reading taken: capacity 128, and an append that finds the window full
 * (n - Q == 128) first quantizes its oldest 32 tokens as block Q/32, then
 * stores the new token.  Hence Q(n) = 32*ceil(max(0, n - 128)/32).
 * Variant flush_tokens = 128 (the popular-science article's wording, 三:
 * the full window is quantized as one batch): the full window's 128 tokens
 * become blocks Q/32 .. Q/32 + 3 at once, so Q(n) = 128*floor((n-1)/128)
 * for n > 128.  Every block holds the same bytes in both variants.
 * A block index beyond the block table's capacity sets bit 1 of the error
 * flag and drops the append (state unchanged).
 */

static uint16_t *ring_k(const orc_cache *c, int b, int h, int slot)
{
    return c->res_k + (((size_t)b * c->num_kv_heads + h) * ORC_R + slot) * ORC_D;
}
static uint16_t *ring_v_ch(const orc_cache *c, int b, int h, int ch)
{
    return c->res_v + (((size_t)b * c->num_kv_heads + h) * ORC_D + ch) * ORC_R;
}
static uint16_t *ring_norm(const orc_cache *c, int b, int h, int slot)
{
    if (c->norm_scope == ORC_NORM_TOKEN)
        return c->res_norm + (size_t)b * ORC_R + slot;
    return c->res_norm + ((size_t)b * c->num_kv_heads + h) * ORC_R + slot;
}
static uint8_t *pool_rec(const orc_cache *c, int p, int h)
{
    return c->pool + ((size_t)p * c->num_kv_heads + h) * ORC_REC_BYTES;
}
static uint16_t *pool_norm(const orc_cache *c, int p, int h, int t)
{
    if (c->norm_scope == ORC_NORM_TOKEN)
        return c->pool_norm + (size_t)p * 32 + t;
    return c->pool_norm + ((size_t)p * c->num_kv_heads + h) * 32 + t;
}

/* Quantize the ring's 32 oldest tokens (token Q .. Q+31) as block Q/32. */
static void flush_block(orc_cache *c, int b, int Q)
{
    int j = Q / ORC_G;
    int p = c->block_table[(size_t)b * c->max_blocks_per_seq + j];
    int s0 = Q % ORC_R;
    for (int h = 0; h < c->num_kv_heads; h++) {
        quant_record(ring_k(c, b, h, s0), ORC_D, ring_v_ch(c, b, h, 0) + s0, 1,
                     ORC_R, pool_rec(c, p, h));
        for (int t = 0; t < 32; t++)
            *pool_norm(c, p, h, t) = *ring_norm(c, b, h, s0 + t);
    }
}

void orc_append_one(orc_cache *c, int b, const uint16_t *k_tok,
                    const uint16_t *v_tok, int dtype)
{
    int32_t *st = c->seq_state + 2 * b;
    int n = st[0], Q = st[1];
    const int hkv = c->num_kv_heads;
    if (c->rope && n >= c->rope_max_pos) {
        *c->error_flag |= 8;   /* no (cos, sin) for this position: dropped */
        return;
    }
    if (n - Q == ORC_R) {
        const int nf = c->flush_tokens == ORC_R ? ORC_R : ORC_G;   /* tokens per flush */
        if ((Q + nf) / ORC_G > c->max_blocks_per_seq) {
            *c->error_flag |= 1;
            return;
        }
        for (int q = Q; q < Q + nf; q += ORC_G)
            flush_block(c, b, q);
        Q += nf;
    }
    int slot = n % ORC_R;
    uint16_t *khat = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)hkv * ORC_D);
    uint16_t *norm = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)hkv);
    /* the new token sits at position n */
    orc_rotate_scale_key_pos(k_tok, dtype, 1, hkv, c->norm_scope, c->rope, n, khat, norm);
    for (int h = 0; h < hkv; h++) {
        memcpy(ring_k(c, b, h, slot), khat + h * ORC_D, ORC_D * sizeof(uint16_t));
        for (int ch = 0; ch < ORC_D; ch++)
            ring_v_ch(c, b, h, ch)[slot] =
                orc_f32_to_f16_sat(orc_in_to_f32(v_tok[h * ORC_D + ch], dtype));
        *ring_norm(c, b, h, slot) = c->norm_scope == ORC_NORM_TOKEN ? norm[0] : norm[h];
    }
    free(norm);
    free(khat);
    st[0] = n + 1;
    st[1] = Q;
}

/* One decode-step append: k_new, v_new are [B][Hkv][128]. */
void orc_append(orc_cache *c, const uint16_t *k_new, const uint16_t *v_new,
                int dtype)
{
    const size_t w = (size_t)c->num_kv_heads * ORC_D;
    for (int b = 0; b < c->batch; b++)
        orc_append_one(c, b, k_new + b * w, v_new + b * w, dtype);
}

/* Prefill is defined as n_tokens appends to an empty sequence ([RN]
 * End-to-End Flow: in prefill, Keys pass FHT, per-token scaling and INT2
 * per-channel quantization before entering the cache).  Returns -1 if the
 * sequence is not empty. */
int orc_prefill(orc_cache *c, int b, const uint16_t *k, const uint16_t *v,
                int n_tokens, int dtype)
{
    if (c->seq_state[2 * b] != 0)
        return -1;
    const size_t w = (size_t)c->num_kv_heads * ORC_D;
    for (int t = 0; t < n_tokens; t++)
        orc_append_one(c, b, k + (size_t)t * w, v + (size_t)t * w, dtype);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantization and decode attention                                       */
/* ------------------------------------------------------------------------ */

/* Key row of token t, head h, in fp64: dequantize then undo the scaling,
 * k = n * (z + delta * code) for quantized tokens, k = n * k_hat for the
 * residual window ([SUM] 方法步骤详情: inverse token scaling before
 * attention; [RN] End-to-End Flow: dequantization + inverse scaling).
 * The row stays in the rotated basis. */
void orc_key_row(const orc_cache *c, int b, int h, int t, double *out)
{
    int Q = c->seq_state[2 * b + 1];
    if (t < Q) {
        int p = c->block_table[(size_t)b * c->max_blocks_per_seq + t / ORC_G];
        const uint8_t *rec = pool_rec(c, p, h);
        int tt = t % ORC_G;
        double nrm = orc_f16_to_f32(*pool_norm(c, p, h, tt));
        for (int ch = 0; ch < ORC_D; ch++) {
            double d = orc_f16_to_f32(get_u16(rec + ORC_REC_KDELTA + 2 * ch));
            double z = orc_f16_to_f32(get_u16(rec + ORC_REC_KZERO + 2 * ch));
            out[ch] = nrm * (z + d * orc_kcode_get(rec, tt, ch));
        }
    } else {
        int slot = t % ORC_R;
        double nrm = orc_f16_to_f32(*ring_norm(c, b, h, slot));
        const uint16_t *kr = ring_k(c, b, h, slot);
        for (int ch = 0; ch < ORC_D; ch++)
            out[ch] = nrm * orc_f16_to_f32(kr[ch]);
    }
}

/* Value row of token t, head h, in fp64 (rotated basis: the Value rotation
 * is absorbed offline into the weights, [SUM] 方法步骤详情 (3)). */
void orc_value_row(const orc_cache *c, int b, int h, int t, double *out)
{
    int Q = c->seq_state[2 * b + 1];
    if (t < Q) {
        int p = c->block_table[(size_t)b * c->max_blocks_per_seq + t / ORC_G];
        const uint8_t *rec = pool_rec(c, p, h);
        int tt = t % ORC_G;
        for (int ch = 0; ch < ORC_D; ch++) {
            const uint8_t *pp = rec + ORC_REC_VPARAM + 4 * (32 * (ch / ORC_VG) + tt);
            double d = orc_f16_to_f32(get_u16(pp));
            double z = orc_f16_to_f32(get_u16(pp + 2));
            out[ch] = z + d * orc_vcode_get(rec, tt, ch);
        }
    } else {
        int slot = t % ORC_R;
        for (int ch = 0; ch < ORC_D; ch++)
            out[ch] = orc_f16_to_f32(ring_v_ch(c, b, h, ch)[slot]);
    }
}

/* softmax(q' K^T / sqrt(128)) V for query head i of sequence b over all n
 * cached tokens, the step's own new token included.  Query head i reads KV
 * head i / (Hq / Hkv) (contiguous GQA grouping, a reading).  q' is the
 * rotated query; since the same orthonormal H multiplies q and every k, the
 * scores equal those of the unrotated vectors ([POP] Q2; [RN] §II).
 * Accumulation in fp64; out fp32, lse = max score + ln(sum of exp). */
void orc_decode_attn_one(const orc_cache *c, const float *qrot, int b, int i,
                         float *out, float *lse)
{
    const int hq = c->num_q_heads, hkv = c->num_kv_heads;
    const int h = i / (hq / hkv);
    const int n = c->seq_state[2 * b];
    const float *q = qrot + ((size_t)b * hq + i) * ORC_D;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double row[ORC_D], acc[ORC_D];
    double m = -INFINITY;
    for (int t = 0; t < n; t++) {
        orc_key_row(c, b, h, t, row);
        double dot = 0.0;
        for (int ch = 0; ch < ORC_D; ch++)
            dot += (double)q[ch] * row[ch];
        s[t] = dot / sqrt((double)ORC_D);
        if (s[t] > m)
            m = s[t];
    }
    double l = 0.0;
    for (int ch = 0; ch < ORC_D; ch++)
        acc[ch] = 0.0;
    for (int t = 0; t < n; t++) {
        double p = exp(s[t] - m);
        l += p;
        orc_value_row(c, b, h, t, row);
        for (int ch = 0; ch < ORC_D; ch++)
            acc[ch] += p * row[ch];
    }
    for (int ch = 0; ch < ORC_D; ch++)
        out[ch] = n > 0 ? (float)(acc[ch] / l) : 0.0f;
    if (lse)
        *lse = n > 0 ? (float)(m + log(l)) : -INFINITY;
    free(s);
}

/* Split-K building blocks (FlashDecoding, the substrate named in [SUM]
 * 技术新颖性).  A partial over the tokens [t0, t1) of sequence b, query head
 * i, in fp64 and natural-log units:
 *   m = max_t s_t,  l = sum_t e^(s_t - m),  o[c] = sum_t e^(s_t - m) v_t[c]
 * (not normalised); an empty range gives m = -inf, l = 0, o = 0.  The scores
 * and rows are those of orc_decode_attn_one. */
void orc_decode_attn_partial(const orc_cache *c, const float *qrot, int b, int i,
                             int t0, int t1, double *m_out, double *l_out,
                             double *o_out)
{
    const int hq = c->num_q_heads, hkv = c->num_kv_heads;
    const int h = i / (hq / hkv);
    const float *q = qrot + ((size_t)b * hq + i) * ORC_D;
    const int n = t1 > t0 ? t1 - t0 : 0;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double row[ORC_D];
    double m = -INFINITY, l = 0.0;
    for (int ch = 0; ch < ORC_D; ch++)
        o_out[ch] = 0.0;
    for (int t = 0; t < n; t++) {
        orc_key_row(c, b, h, t0 + t, row);
        double dot = 0.0;
        for (int ch = 0; ch < ORC_D; ch++)
            dot += (double)q[ch] * row[ch];
        s[t] = dot / sqrt((double)ORC_D);
        if (s[t] > m)
            m = s[t];
    }
    for (int t = 0; t < n; t++) {
        double p = exp(s[t] - m);
        l += p;
        orc_value_row(c, b, h, t0 + t, row);
        for (int ch = 0; ch < ORC_D; ch++)
            o_out[ch] += p * row[ch];
    }
    *m_out = m;
    *l_out = l;
    free(s);
}

/* Cross-split log-sum-exp merge of n_parts partials (m[s], l[s], o[s][128])
 * of one query head:  M = max_s m_s,  L = sum_s l_s e^(m_s - M),
 * out = sum_s o_s e^(m_s - M) / L,  lse = M + ln L.  Partials with m = -inf
 * carry no tokens and weigh 0; all empty gives out = 0, lse = -inf. */
void orc_lse_merge(int n_parts, const double *m, const double *l,
                   const double *o, float *out, float *lse)
{
    double M = -INFINITY;
    for (int s = 0; s < n_parts; s++)
        if (m[s] > M)
            M = m[s];
    double L = 0.0, acc[ORC_D];
    for (int ch = 0; ch < ORC_D; ch++)
        acc[ch] = 0.0;
    if (M != -INFINITY) {
        for (int s = 0; s < n_parts; s++) {
            if (m[s] == -INFINITY)
                continue;
            double w = exp(m[s] - M);
            L += w * l[s];
            for (int ch = 0; ch < ORC_D; ch++)
                acc[ch] += w * o[(size_t)s * ORC_D + ch];
        }
    }
    for (int ch = 0; ch < ORC_D; ch++)
        out[ch] = M != -INFINITY ? (float)(acc[ch] / L) : 0.0f;
    if (lse)
        *lse = M != -INFINITY ? (float)(M + log(L)) : -INFINITY;
}

/* All sequences and query heads: qrot, out [B][Hq][128]; lse [B][Hq] or NULL. */
void orc_decode_attn(const orc_cache *c, const float *qrot, float *out,
                     float *lse)
{
    for (int b = 0; b < c->batch; b++)
        for (int i = 0; i < c->num_q_heads; i++)
            orc_decode_attn_one(c, qrot, b, i,
                                out + ((size_t)b * c->num_q_heads + i) * ORC_D,
                                lse ? lse + (size_t)b * c->num_q_heads + i : NULL);
}

/* ------------------------------------------------------------------------ */
/* Unquantized decode attention (the BF16 baseline)                          */
/* ------------------------------------------------------------------------ */

/* Plain decode attention over an unquantized cache: the BF16
 * FlashDecoding-v2 baseline against which the summary's efficiency results
 * (实验结果; 论文图表) and the popular-science article (四) measure the INT2
 * kernel.  No rotation, no scaling, no quantization: for query head i and
 * KV head h = i / (Hq/Hkv),
 *     s_t = (q_i . k_t) / sqrt(128),  out = sum_t e^(s_t - max) v_t / sum_t e^(s_t - max),
 *     lse = max + ln(sum_t e^(s_t - max)),
 * everything in fp64.  q [Hq][128]; k, v [n][Hkv][128] (fp32 values, e.g.
 * bf16 inputs converted exactly); out [Hq][128]; lse [Hq] or NULL.  n = 0
 * gives zeros and lse = -inf. */
void orc_dense_attn(const float *q, const float *k, const float *v, int n,
                    int hq, int hkv, float *out, float *lse)
{
    const int grp = hq / hkv;
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < hq; i++) {
        const int h = i / grp;
        const float *qi = q + (size_t)i * ORC_D;
        double m = -INFINITY;
        for (int t = 0; t < n; t++) {
            const float *kt = k + ((size_t)t * hkv + h) * ORC_D;
            double dot = 0.0;
            for (int ch = 0; ch < ORC_D; ch++)
                dot += (double)qi[ch] * (double)kt[ch];
            s[t] = dot / sqrt((double)ORC_D);
            if (s[t] > m)
                m = s[t];
        }
        double acc[ORC_D], l = 0.0;
        for (int ch = 0; ch < ORC_D; ch++)
            acc[ch] = 0.0;
        for (int t = 0; t < n; t++) {
            const float *vt = v + ((size_t)t * hkv + h) * ORC_D;
            const double p = exp(s[t] - m);
            l += p;
            for (int ch = 0; ch < ORC_D; ch++)
                acc[ch] += p * (double)vt[ch];
        }
        for (int ch = 0; ch < ORC_D; ch++)
            out[(size_t)i * ORC_D + ch] = n > 0 ? (float)(acc[ch] / l) : 0.0f;
        if (lse)
            lse[i] = n > 0 ? (float)(m + log(l)) : -INFINITY;
    }
    free(s);
}
