/*
 * qmv_oracle.c -- plain, slow, single-threaded CPU oracle for the
 * dequantize-fused GGUF matvec.  TEST INFRASTRUCTURE ONLY: the GPU library
 * never links, calls or includes anything here, and nothing here is shared
 * with it.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * load this file's shared object.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared (no FMA
 * contraction, so every f32 step below rounds exactly as written).
 *
 * What is computed, and where it is stated:
 *  - Block formats Q8_0, Q4_K, Q6_K.  BebeLM page ("BebeLM：纯Rust实现的端侧大模型
 *    推理引擎"), section "量化格式支持": Q4_K packs 256 weights in a 144-byte
 *    super-block, Q6_K holds the sensitive tensors, and dequantisation happens at
 *    run time with f32 activations.  Wick page, section "量化支持": Q4_K_M and
 *    Q8_0.  The pages give sizes only; the field order and the bit order inside
 *    the fields follow the standard GGUF conventions the pages say the engines
 *    load ("标准GGUF" row of the FlareLLM page's comparison table).  That is a
 *    reading, spelled out as index math at each decoder below.
 *  - More block formats from the pages' lists: FlareLLM page, section
 *    "量化技术的全面支持" names the standard 4- to 8-bit quantisations (Q4_0
 *    through Q8_1) and the K-quants; the BebeLM page, section "局限与未来",
 *    wants Q5_K_M; the K-quants include Q2_K and Q3_K.  Their layouts again
 *    follow the standard GGUF reading,
 *    written out at each decoder below.
 *  - The matvec itself is the plain definition y = dequant(W) x, each product
 *    formed exactly in f64 and summed in order k = 0..K-1.
 *  - MoE routing: BebeLM page, section "核心算子" (MoE FFN: sigmoid router,
 *    top-k = 4 of 32 experts, expert bias used only for selection, selected
 *    weights renormalised), with the router and bias kept in f32 (section
 *    "量化格式支持").
 *  - Greedy fused argmax: FlareLLM page, section "推理层面的深度优化" (at
 *    temperature 0 the most probable token is found without a logits buffer).
 *  - Small-batch verify: FlareLLM page, same section (n-gram speculative
 *    decoding verifies several drafted tokens against the same weights).
 *
 *  - Prefill-size product: BebeLM page, section "性能表现" (prompts go
 *    through as batches); the same definition as the small batch, so
 *    oracle_gemm_n serves both.
 *
 * Every function returns 0 on success and -1 on a bad argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define T_Q4_0 2
#define T_Q4_1 3
#define T_Q5_0 6
#define T_Q5_1 7
#define T_Q8_0 8
#define T_Q8_1 9
#define T_Q2_K 10
#define T_Q3_K 11
#define T_Q4_K 12
#define T_Q5_K 13
#define T_Q6_K 14

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary32, written from the format's definition.     */
/* ------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormals are frac * 2^-24; normals are (1024 + frac) * 2^(exp - 25).
 * Every binary16 value is exactly representable in binary32. */
float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

/* Nearest binary16 to f, ties to even; overflow goes to infinity. */
uint16_t oracle_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    int e2, E;
    double q;
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    if (a == 0.0)
        return sign;
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00u);
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    E = e2 - 1;             /* a = 1.xxx * 2^E */
    if (E < -14)
        E = -14;            /* below the normal range the spacing stays 2^-24 */
    /* significand in units of the spacing 2^(E-10), rounded to nearest even */
    q = nearbyint(ldexp(a, 10 - E));
    if (q >= 2048.0) {      /* rounded up into the next binade */
        q = q / 2.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7C00u);
    if (q < 1024.0)         /* subnormal (E == -14) */
        return (uint16_t)(sign | (uint16_t)q);
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024)));
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 255); p[1] = (uint8_t)(v >> 8); }

/* ------------------------------------------------------------------------- */
/* Block geometry                                                            */
/* ------------------------------------------------------------------------- */

int oracle_block_weights(int type)
{
    switch (type) {
    case T_Q4_0: case T_Q4_1: case T_Q5_0: case T_Q5_1: case T_Q8_0: case T_Q8_1: return 32;
    case T_Q2_K: case T_Q3_K: case T_Q4_K: case T_Q5_K: case T_Q6_K: return 256;
    default: return 0;
    }
}

int oracle_block_bytes(int type)
{
    switch (type) {
    case T_Q4_0: return 18;   /* fp16 d + 16 B nibbles */
    case T_Q4_1: return 20;   /* fp16 d, fp16 m + 16 B nibbles */
    case T_Q5_0: return 22;   /* fp16 d, 4 B high bits, 16 B nibbles */
    case T_Q5_1: return 24;   /* fp16 d, fp16 m, 4 B high bits, 16 B nibbles */
    case T_Q8_0: return 34;   /* fp16 d + 32 int8 */
    case T_Q8_1: return 36;   /* fp16 d, fp16 s + 32 int8 */
    case T_Q2_K: return 84;   /* 16 B 4-bit scale/min pairs, 64 B 2-bit codes, fp16 d, fp16 dmin */
    case T_Q3_K: return 110;  /* 32 B high bits, 64 B 2-bit codes, 12 B 6-bit scales, fp16 d */
    case T_Q4_K: return 144;  /* fp16 d, fp16 dmin, 12 B scales, 128 B nibbles */
    case T_Q5_K: return 176;  /* fp16 d, fp16 dmin, 12 B scales, 32 B high bits, 128 B nibbles */
    case T_Q6_K: return 210;  /* 128 B low nibbles, 64 B high pairs, 16 int8 scales, fp16 d */
    default: return 0;
    }
}

static int shape_ok(int type, int64_t M, int64_t K)
{
    int bw = oracle_block_weights(type);
    return bw > 0 && M >= 1 && K >= 1 && K % bw == 0;
}

static size_t row_bytes(int type, int64_t K)
{
    return (size_t)(K / oracle_block_weights(type)) * (size_t)oracle_block_bytes(type);
}

/* ------------------------------------------------------------------------- */
/* Decoders: one block -> its weights in f32 (bit-exact target).             */
/* ------------------------------------------------------------------------- */

/* Q8_0: d (fp16) at bytes [0,2), then 32 signed bytes q; weight i = d * q[i]. */
static void decode_q8_0(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    for (int i = 0; i < 32; i++)
        w[i] = d * (float)(int8_t)b[2 + i];
}

/* Q4_K 6-bit scale / min of sub-block j from the 12 packed bytes S.
 * Sub-blocks 0..3 keep their scale in the low 6 bits of S[j] and their min in
 * the low 6 bits of S[j+4]; sub-blocks 4..7 keep the low 4 bits of scale and
 * min in the two nibbles of S[j+4] and their top 2 bits in the top bits of
 * S[j-4] (scale) and S[j] (min). */
static void q4k_scale_min(const uint8_t *S, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = S[j] & 63;
        *m = S[j + 4] & 63;
    } else {
        *sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        *m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

/* Q4_K: d at [0,2), dmin at [2,4), packed scales S at [4,16), nibbles Q at
 * [16,144).  Weight i lies in 64-weight chunk c = i/64; its byte is
 * Q[32c + i%32]; the first 32 weights of a chunk use the low nibble and the
 * next 32 the high nibble, so sub-block j = i/32.  Weight value
 * (d*sc_j)*q - (dmin*m_j): both products are exact in f32 and the one
 * subtraction is the only rounding. */
static void decode_q4_k(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    float dmin = oracle_half_to_float(rd16(b + 2));
    const uint8_t *S = b + 4;
    const uint8_t *Q = b + 16;
    for (int i = 0; i < 256; i++) {
        int c = i / 64, hi = (i % 64) / 32, l = i % 32;
        int j = i / 32;
        int sc, m;
        uint8_t byte = Q[32 * c + l];
        int q = hi ? (byte >> 4) : (byte & 15);
        q4k_scale_min(S, j, &sc, &m);
        float s = d * (float)sc;
        float o = dmin * (float)m;
        w[i] = s * (float)q - o;
    }
}

/* Q6_K: QL (low 4 bits) at [0,128), QH (high 2 bits) at [128,192), 16 signed
 * sub-block scales at [192,208), d (fp16) at [208,210).  Weight i: half
 * n = i/128, r = i%128, quarter g = r/32, l = r%32.  Low bits come from
 * QL[64n + l + 32*(g%2)], low nibble for g < 2 and high nibble for g >= 2;
 * high bits are bits 2g..2g+1 of QH[32n + l]; q = (low | high<<4) - 32.
 * Sub-block j = i/16 (16 weights each).  Weight value (d*sc_j)*q, exact. */
static void decode_q6_k(const uint8_t *b, float *w)
{
    const uint8_t *QL = b, *QH = b + 128;
    const int8_t *SC = (const int8_t *)(b + 192);
    float d = oracle_half_to_float(rd16(b + 208));
    for (int i = 0; i < 256; i++) {
        int n = i / 128, r = i % 128, g = r / 32, l = r % 32;
        int lo = (QL[64 * n + l + 32 * (g % 2)] >> (4 * (g / 2))) & 15;
        int hi = (QH[32 * n + l] >> (2 * g)) & 3;
        int q = (lo | (hi << 4)) - 32;
        int j = i / 16;
        float s = d * (float)SC[j];
        w[i] = s * (float)q;
    }
}

/* The 32-weight formats share one nibble order: byte l (0..15) of the code
 * bytes holds weight l in its low nibble and weight l + 16 in its high
 * nibble.  The 5-bit formats add bit i of a little-endian 32-bit word as bit
 * 4 of weight i's code. */
static int nibble32(const uint8_t *Q, int i) { return (Q[i % 16] >> (4 * (i / 16))) & 15; }
static uint32_t rd32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* Q4_0: d at [0,2), codes at [2,18); weight i = d * (q_i - 8), exact. */
static void decode_q4_0(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    for (int i = 0; i < 32; i++)
        w[i] = d * (float)(nibble32(b + 2, i) - 8);
}

/* Q4_1: d at [0,2), m at [2,4), codes at [4,20); weight i = d * q_i + m
 * (the product is exact, the sum is the one rounding). */
static void decode_q4_1(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b)), m = oracle_half_to_float(rd16(b + 2));
    for (int i = 0; i < 32; i++)
        w[i] = d * (float)nibble32(b + 4, i) + m;
}

/* Q5_0: d at [0,2), high bits H at [2,6), codes at [6,22);
 * q_i = nibble | bit_i(H) << 4, weight i = d * (q_i - 16), exact. */
static void decode_q5_0(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    uint32_t H = rd32(b + 2);
    for (int i = 0; i < 32; i++) {
        int q = nibble32(b + 6, i) | (int)(((H >> i) & 1u) << 4);
        w[i] = d * (float)(q - 16);
    }
}

/* Q5_1: d at [0,2), m at [2,4), high bits H at [4,8), codes at [8,24);
 * weight i = d * q_i + m. */
static void decode_q5_1(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b)), m = oracle_half_to_float(rd16(b + 2));
    uint32_t H = rd32(b + 4);
    for (int i = 0; i < 32; i++) {
        int q = nibble32(b + 8, i) | (int)(((H >> i) & 1u) << 4);
        w[i] = d * (float)q + m;
    }
}

/* Q8_1: d at [0,2), s at [2,4) (d times the code sum, kept for activation
 * use; not part of the weight value), 32 signed codes at [4,36);
 * weight i = d * q_i, exact. */
static void decode_q8_1(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    for (int i = 0; i < 32; i++)
        w[i] = d * (float)(int8_t)b[4 + i];
}

/* Q5_K: d at [0,2), dmin at [2,4), packed scales S at [4,16) (the Q4_K
 * packing), high bits QH at [16,48), nibbles Q at [48,176).  Weight i lies
 * in 64-weight chunk c = i/64 with h = (i%64)/32 and l = i%32: its nibble is
 * the low (h = 0) or high (h = 1) nibble of Q[32c + l], its fifth bit is bit
 * 2c + h of QH[l], and sub-block j = i/32.  Weight value
 * (d*sc_j)*q - (dmin*m_j), q in 0..31. */
static void decode_q5_k(const uint8_t *b, float *w)
{
    float d = oracle_half_to_float(rd16(b));
    float dmin = oracle_half_to_float(rd16(b + 2));
    const uint8_t *S = b + 4, *QH = b + 16, *Q = b + 48;
    for (int i = 0; i < 256; i++) {
        int c = i / 64, h = (i % 64) / 32, l = i % 32;
        int j = i / 32;
        int sc, m;
        int q = ((Q[32 * c + l] >> (4 * h)) & 15) | (((QH[l] >> (2 * c + h)) & 1) << 4);
        q4k_scale_min(S, j, &sc, &m);
        float s = d * (float)sc;
        float o = dmin * (float)m;
        w[i] = s * (float)q - o;
    }
}

/* Q2_K: scale/min bytes S at [0,16) (sub-block j of 16 weights: scale =
 * low nibble of S[j], min = high nibble), 2-bit codes Q at [16,80), d at
 * [80,82), dmin at [82,84).  Weight i: half n = i/128, r = i%128, plane
 * p = r/32, l = r%32; q = bits 2p..2p+1 of Q[32n + l]; sub-block
 * j = 8n + 2p + l/16 (= i/16).  Weight value (d*sc_j)*q - (dmin*m_j). */
static void decode_q2_k(const uint8_t *b, float *w)
{
    const uint8_t *S = b, *Q = b + 16;
    float d = oracle_half_to_float(rd16(b + 80));
    float dmin = oracle_half_to_float(rd16(b + 82));
    for (int i = 0; i < 256; i++) {
        int n = i / 128, r = i % 128, p = r / 32, l = r % 32;
        int q = (Q[32 * n + l] >> (2 * p)) & 3;
        int j = i / 16;
        float s = d * (float)(S[j] & 15);
        float o = dmin * (float)(S[j] >> 4);
        w[i] = s * (float)q - o;
    }
}

/* Q3_K 6-bit scale of sub-block j (0..15) from the 12 packed bytes S: low
 * four bits from the low (j < 8) or high (j >= 8) nibble of S[j % 8], top
 * two bits from bits 2*(j/4)..+1 of S[8 + j%4]; the value is that minus 32. */
static int q3k_scale(const uint8_t *S, int j)
{
    int lo = j < 8 ? (S[j] & 15) : (S[j - 8] >> 4);
    int hi = (S[8 + j % 4] >> (2 * (j / 4))) & 3;
    return (lo | (hi << 4)) - 32;
}

/* Q3_K: high bits H at [0,32), 2-bit codes Q at [32,96), packed scales S at
 * [96,108), d at [108,110).  Weight i: half n = i/128, r = i%128, plane
 * p = r/32, l = r%32; low = bits 2p..2p+1 of Q[32n + l]; the code is
 * low - 4 when bit 4n + p of H[l] is clear, low when it is set (so -4..3);
 * sub-block j = i/16.  Weight value (d*sc_j)*q, exact. */
static void decode_q3_k(const uint8_t *b, float *w)
{
    const uint8_t *H = b, *Q = b + 32, *S = b + 96;
    float d = oracle_half_to_float(rd16(b + 108));
    for (int i = 0; i < 256; i++) {
        int n = i / 128, r = i % 128, p = r / 32, l = r % 32;
        int low = (Q[32 * n + l] >> (2 * p)) & 3;
        int q = low - (((H[l] >> (4 * n + p)) & 1) ? 0 : 4);
        float s = d * (float)q3k_scale(S, i / 16);
        w[i] = s * (float)q;
    }
}

static void decode_block(int type, const uint8_t *b, float *w)
{
    switch (type) {
    case T_Q2_K: decode_q2_k(b, w); break;
    case T_Q3_K: decode_q3_k(b, w); break;
    case T_Q4_0: decode_q4_0(b, w); break;
    case T_Q4_1: decode_q4_1(b, w); break;
    case T_Q5_0: decode_q5_0(b, w); break;
    case T_Q5_1: decode_q5_1(b, w); break;
    case T_Q8_0: decode_q8_0(b, w); break;
    case T_Q8_1: decode_q8_1(b, w); break;
    case T_Q4_K: decode_q4_k(b, w); break;
    case T_Q5_K: decode_q5_k(b, w); break;
    default: decode_q6_k(b, w); break;
    }
}

static void decode_row(int type, const uint8_t *row, int64_t K, float *w)
{
    int bw = oracle_block_weights(type), bb = oracle_block_bytes(type);
    for (int64_t kb = 0; kb < K / bw; kb++)
        decode_block(type, row + kb * bb, w + kb * bw);
}

/* Dequantise an M x K matrix (rows of consecutive blocks) to f32. */
int oracle_dequant(int type, const uint8_t *blocks, int64_t M, int64_t K, float *w_out)
{
    if (!shape_ok(type, M, K) || !blocks || !w_out) return -1;
    size_t rb = row_bytes(type, K);
    for (int64_t r = 0; r < M; r++)
        decode_row(type, blocks + (size_t)r * rb, K, w_out + (size_t)r * (size_t)K);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Quantisers: test-data generators only (the GPU path never quantises       */
/* inside the matvec).  The pages give no quantiser; these are plain         */
/* min/max rules in f32 with round-half-away-from-zero.                      */
/* ------------------------------------------------------------------------- */

/* Q8_0: d = max|w| / 127 (f32), stored as fp16; q = round(w * (1/d)). */
static void encode_q8_0(const float *w, uint8_t *b)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++)
        if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
    float d = amax / 127.0f;
    float id = d != 0.0f ? 1.0f / d : 0.0f;
    wr16(b, oracle_float_to_half(d));
    for (int i = 0; i < 32; i++) {
        float v = roundf(w[i] * id);
        if (v > 127.0f) v = 127.0f;
        if (v < -128.0f) v = -128.0f;
        b[2 + i] = (uint8_t)(int8_t)v;
    }
}

/* Q4_K and Q5_K, per 32-weight sub-block j with lo_j = min(0, min w) and
 * hi_j = max w, for codes 0..top (top = 15 or 31):
 *   dmin = max_j(-lo_j)/62 -> fp16;  m_j = min(63, ceil(-lo_j/dmin16));
 *   L_j = -dmin16*m_j;  s_j = (hi_j - L_j)/top;  d = max_j s_j / 62 -> fp16;
 *   sc_j = min(63, ceil(s_j/d16));  q = clamp(round((w - L_j)/(d16*sc_j)), 0, top).
 * The mins are fixed first so that each scale covers the offset that the
 * rounded min really produces.  Writes d, dmin and the packed scales (bytes
 * 0..15, the layout both formats share) and returns the codes. */
static void encode_kq_minmax(const float *w, int top, uint8_t *b, int *codes)
{
    float lo[8], hi[8], L[8], s[8];
    int sc[8], m[8];
    float maxneg = 0.0f, maxs = 0.0f;
    for (int j = 0; j < 8; j++) {
        float mn = 0.0f, mx = -INFINITY;
        for (int t = 0; t < 32; t++) {
            float v = w[32 * j + t];
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        lo[j] = mn;
        hi[j] = mx;
        if (-mn > maxneg) maxneg = -mn;
    }
    uint16_t dmin_h = oracle_float_to_half(maxneg / 62.0f);
    float dmin16 = oracle_half_to_float(dmin_h);
    for (int j = 0; j < 8; j++) {
        int mj = 0;
        if (dmin16 > 0.0f) {
            float t = ceilf(-lo[j] / dmin16);
            mj = t > 63.0f ? 63 : (int)t;
        }
        m[j] = mj;
        L[j] = -(dmin16 * (float)mj);
        s[j] = (hi[j] - L[j]) / (float)top;
        if (s[j] > maxs) maxs = s[j];
    }
    uint16_t d_h = oracle_float_to_half(maxs / 62.0f);
    float d16 = oracle_half_to_float(d_h);
    for (int j = 0; j < 8; j++) {
        int sj = 0;
        if (d16 > 0.0f) {
            float t = ceilf(s[j] / d16);
            sj = t > 63.0f ? 63 : (int)t;
        }
        sc[j] = sj;
    }
    wr16(b, d_h);
    wr16(b + 2, dmin_h);
    uint8_t *S = b + 4;
    for (int j = 0; j < 4; j++) {
        S[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        S[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        S[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    for (int i = 0; i < 256; i++) {
        int jj = i / 32;
        int q = 0;
        if (sc[jj] > 0) {
            float step = d16 * (float)sc[jj];
            float t = roundf((w[i] - L[jj]) / step);
            if (t < 0.0f) t = 0.0f;
            if (t > (float)top) t = (float)top;
            q = (int)t;
        }
        codes[i] = q;
    }
}

static void encode_q4_k(const float *w, uint8_t *b)
{
    int codes[256];
    encode_kq_minmax(w, 15, b, codes);
    uint8_t *Q = b + 16;
    memset(Q, 0, 128);
    for (int i = 0; i < 256; i++) {
        int c = i / 64, h = (i % 64) / 32, l = i % 32;
        Q[32 * c + l] |= (uint8_t)(h ? (codes[i] << 4) : codes[i]);
    }
}

static void encode_q5_k(const float *w, uint8_t *b)
{
    int codes[256];
    encode_kq_minmax(w, 31, b, codes);
    uint8_t *QH = b + 16, *Q = b + 48;
    memset(QH, 0, 160);
    for (int i = 0; i < 256; i++) {
        int c = i / 64, h = (i % 64) / 32, l = i % 32;
        Q[32 * c + l] |= (uint8_t)((codes[i] & 15) << (4 * h));
        QH[l] |= (uint8_t)((codes[i] >> 4) << (2 * c + h));
    }
}

/* Q2_K, per 16-weight sub-block j with lo_j = min(0, min w), hi_j = max w:
 *   dmin = max_j(-lo_j)/15 -> fp16; m_j = min(15, ceil(-lo_j/dmin16));
 *   L_j = -dmin16*m_j; s_j = (hi_j - L_j)/3; d = max_j s_j / 15 -> fp16;
 *   sc_j = min(15, ceil(s_j/d16)); q = clamp(round((w - L_j)/(d16*sc_j)), 0, 3). */
static void encode_q2_k(const float *w, uint8_t *b)
{
    float lo[16], hi[16], L[16], s[16];
    int sc[16], m[16];
    float maxneg = 0.0f, maxs = 0.0f;
    for (int j = 0; j < 16; j++) {
        float mn = 0.0f, mx = -INFINITY;
        for (int t = 0; t < 16; t++) {
            float v = w[16 * j + t];
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        lo[j] = mn;
        hi[j] = mx;
        if (-mn > maxneg) maxneg = -mn;
    }
    uint16_t dmin_h = oracle_float_to_half(maxneg / 15.0f);
    float dmin16 = oracle_half_to_float(dmin_h);
    for (int j = 0; j < 16; j++) {
        int mj = 0;
        if (dmin16 > 0.0f) {
            float t = ceilf(-lo[j] / dmin16);
            mj = t > 15.0f ? 15 : (int)t;
        }
        m[j] = mj;
        L[j] = -(dmin16 * (float)mj);
        s[j] = (hi[j] - L[j]) / 3.0f;
        if (s[j] > maxs) maxs = s[j];
    }
    uint16_t d_h = oracle_float_to_half(maxs / 15.0f);
    float d16 = oracle_half_to_float(d_h);
    for (int j = 0; j < 16; j++) {
        int sj = 0;
        if (d16 > 0.0f) {
            float t = ceilf(s[j] / d16);
            sj = t > 15.0f ? 15 : (int)t;
        }
        sc[j] = sj;
        b[j] = (uint8_t)(sj | (m[j] << 4));
    }
    memset(b + 16, 0, 64);
    for (int i = 0; i < 256; i++) {
        int j = i / 16, q = 0;
        if (sc[j] > 0) {
            float t = roundf((w[i] - L[j]) / (d16 * (float)sc[j]));
            if (t < 0.0f) t = 0.0f;
            if (t > 3.0f) t = 3.0f;
            q = (int)t;
        }
        int n = i / 128, r = i % 128, p = r / 32, l = r % 32;
        b[16 + 32 * n + l] |= (uint8_t)(q << (2 * p));
    }
    wr16(b + 80, d_h);
    wr16(b + 82, dmin_h);
}

/* Q3_K, per 16-weight sub-block j: v_j = the weight of largest magnitude
 * (first one on ties), s_j = -v_j/4 so that v_j sits on code -4 (the end
 * of -4..3 that reaches furthest); d = max_j |s_j| / 31 -> fp16;
 * sc_j = sign(s_j) * min(31, ceil(|s_j|/d16)) (stored + 32);
 * q = clamp(round(w/(d16*sc_j)), -4, 3). */
static void encode_q3_k(const float *w, uint8_t *b)
{
    float s[16], maxs = 0.0f;
    int sc[16];
    for (int j = 0; j < 16; j++) {
        float v = 0.0f;
        for (int t = 0; t < 16; t++)
            if (fabsf(w[16 * j + t]) > fabsf(v)) v = w[16 * j + t];
        s[j] = -v / 4.0f;
        if (fabsf(s[j]) > maxs) maxs = fabsf(s[j]);
    }
    uint16_t d_h = oracle_float_to_half(maxs / 31.0f);
    float d16 = oracle_half_to_float(d_h);
    memset(b, 0, 110);
    uint8_t *H = b, *Q = b + 32, *S = b + 96;
    for (int j = 0; j < 16; j++) {
        int sj = 0;
        if (d16 > 0.0f) {
            float t = ceilf(fabsf(s[j]) / d16);
            sj = t > 31.0f ? 31 : (int)t;
            if (s[j] < 0.0f) sj = -sj;
        }
        sc[j] = sj;
        int u = sj + 32;  /* 6-bit stored value, 1..63 */
        if (j < 8) S[j] |= (uint8_t)(u & 15);
        else S[j - 8] |= (uint8_t)((u & 15) << 4);
        S[8 + j % 4] |= (uint8_t)((u >> 4) << (2 * (j / 4)));
    }
    for (int i = 0; i < 256; i++) {
        int j = i / 16, q = 0;
        if (sc[j] != 0) {
            float t = roundf(w[i] / (d16 * (float)sc[j]));
            if (t < -4.0f) t = -4.0f;
            if (t > 3.0f) t = 3.0f;
            q = (int)t;
        }
        int n = i / 128, r = i % 128, p = r / 32, l = r % 32;
        int code = q + 4;  /* 0..7: bit 2 set means the code is not lowered by 4 */
        Q[32 * n + l] |= (uint8_t)((code & 3) << (2 * p));
        H[l] |= (uint8_t)((code >> 2) << (4 * n + p));
    }
    wr16(b + 108, d_h);
}

/* 32-weight formats.  Symmetric ones (Q4_0, Q5_0, Q8_1): d = max|w| / half
 * (half = 7, 15, 127) -> fp16, code = clamp(round(w/d16), -half-1, half)
 * stored with its offset (8, 16, or as a signed byte).  Asymmetric ones
 * (Q4_1, Q5_1): m = min w -> fp16, d = (max w - m16)/top -> fp16,
 * q = clamp(round((w - m16)/d16), 0, top). */
static void put_codes32(uint8_t *Q, uint8_t *H, const int *q)
{
    memset(Q, 0, 16);
    uint32_t hb = 0;
    for (int i = 0; i < 32; i++) {
        Q[i % 16] |= (uint8_t)((q[i] & 15) << (4 * (i / 16)));
        hb |= (uint32_t)((q[i] >> 4) & 1) << i;
    }
    if (H) {
        H[0] = (uint8_t)hb;
        H[1] = (uint8_t)(hb >> 8);
        H[2] = (uint8_t)(hb >> 16);
        H[3] = (uint8_t)(hb >> 24);
    }
}

static void encode_sym32(const float *w, int half, uint16_t *d_h, int *q)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++)
        if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
    *d_h = oracle_float_to_half(amax / (float)half);
    float d16 = oracle_half_to_float(*d_h);
    for (int i = 0; i < 32; i++) {
        float t = d16 > 0.0f ? roundf(w[i] / d16) : 0.0f;
        if (t < (float)(-half - 1)) t = (float)(-half - 1);
        if (t > (float)half) t = (float)half;
        q[i] = (int)t;
    }
}

static void encode_asym32(const float *w, int top, uint16_t *d_h, uint16_t *m_h, int *q)
{
    float mn = w[0], mx = w[0];
    for (int i = 1; i < 32; i++) {
        if (w[i] < mn) mn = w[i];
        if (w[i] > mx) mx = w[i];
    }
    *m_h = oracle_float_to_half(mn);
    float m16 = oracle_half_to_float(*m_h);
    *d_h = oracle_float_to_half((mx - m16) / (float)top);
    float d16 = oracle_half_to_float(*d_h);
    for (int i = 0; i < 32; i++) {
        float t = d16 > 0.0f ? roundf((w[i] - m16) / d16) : 0.0f;
        if (t < 0.0f) t = 0.0f;
        if (t > (float)top) t = (float)top;
        q[i] = (int)t;
    }
}

static void encode_q4_0(const float *w, uint8_t *b)
{
    int q[32];
    uint16_t d;
    encode_sym32(w, 7, &d, q);
    for (int i = 0; i < 32; i++) q[i] += 8;
    wr16(b, d);
    put_codes32(b + 2, NULL, q);
}

static void encode_q5_0(const float *w, uint8_t *b)
{
    int q[32];
    uint16_t d;
    encode_sym32(w, 15, &d, q);
    for (int i = 0; i < 32; i++) q[i] += 16;
    wr16(b, d);
    put_codes32(b + 6, b + 2, q);
}

static void encode_q4_1(const float *w, uint8_t *b)
{
    int q[32];
    uint16_t d, m;
    encode_asym32(w, 15, &d, &m, q);
    wr16(b, d);
    wr16(b + 2, m);
    put_codes32(b + 4, NULL, q);
}

static void encode_q5_1(const float *w, uint8_t *b)
{
    int q[32];
    uint16_t d, m;
    encode_asym32(w, 31, &d, &m, q);
    wr16(b, d);
    wr16(b + 2, m);
    put_codes32(b + 8, b + 4, q);
}

/* Q8_1: as Q8_0 with d16 for the codes, plus s = d16 * sum(q) -> fp16. */
static void encode_q8_1(const float *w, uint8_t *b)
{
    int q[32];
    uint16_t d;
    encode_sym32(w, 127, &d, q);
    float d16 = oracle_half_to_float(d);
    int sum = 0;
    for (int i = 0; i < 32; i++) {
        b[4 + i] = (uint8_t)(int8_t)q[i];
        sum += q[i];
    }
    wr16(b, d);
    wr16(b + 2, oracle_float_to_half(d16 * (float)sum));
}

/* Q6_K, per 16-weight sub-block j: s_j = max|w|/31; d = max_j s_j / 126 -> fp16;
 * sc_j = min(127, ceil(s_j/d16)); q = clamp(round(w/(d16*sc_j)), -32, 31) + 32. */
static void encode_q6_k(const float *w, uint8_t *b)
{
    float s[16], maxs = 0.0f;
    int sc[16];
    for (int j = 0; j < 16; j++) {
        float amax = 0.0f;
        for (int t = 0; t < 16; t++)
            if (fabsf(w[16 * j + t]) > amax) amax = fabsf(w[16 * j + t]);
        s[j] = amax / 31.0f;
        if (s[j] > maxs) maxs = s[j];
    }
    uint16_t d_h = oracle_float_to_half(maxs / 126.0f);
    float d16 = oracle_half_to_float(d_h);
    for (int j = 0; j < 16; j++) {
        int sj = 0;
        if (d16 > 0.0f) {
            float t = ceilf(s[j] / d16);
            sj = t > 127.0f ? 127 : (int)t;
        }
        sc[j] = sj;
    }
    uint8_t *QL = b, *QH = b + 128;
    memset(b, 0, 192);
    for (int j = 0; j < 16; j++)
        b[192 + j] = (uint8_t)(int8_t)sc[j];
    wr16(b + 208, d_h);
    for (int i = 0; i < 256; i++) {
        int j = i / 16;
        int q = 0;
        if (sc[j] > 0) {
            float step = d16 * (float)sc[j];
            float t = roundf(w[i] / step);
            if (t < -32.0f) t = -32.0f;
            if (t > 31.0f) t = 31.0f;
            q = (int)t;
        }
        int u = q + 32;
        int n = i / 128, r = i % 128, g = r / 32, l = r % 32;
        QL[64 * n + l + 32 * (g % 2)] |= (uint8_t)((u & 15) << (4 * (g / 2)));
        QH[32 * n + l] |= (uint8_t)((u >> 4) << (2 * g));
    }
}

int oracle_quantize(int type, const float *w, int64_t M, int64_t K, uint8_t *blocks_out)
{
    if (!shape_ok(type, M, K) || !w || !blocks_out) return -1;
    int bw = oracle_block_weights(type), bb = oracle_block_bytes(type);
    int64_t nblk = M * (K / bw);
    for (int64_t t = 0; t < nblk; t++) {
        const float *src = w + t * bw;
        uint8_t *dst = blocks_out + t * bb;
        switch (type) {
        case T_Q2_K: encode_q2_k(src, dst); break;
        case T_Q3_K: encode_q3_k(src, dst); break;
        case T_Q4_0: encode_q4_0(src, dst); break;
        case T_Q4_1: encode_q4_1(src, dst); break;
        case T_Q5_0: encode_q5_0(src, dst); break;
        case T_Q5_1: encode_q5_1(src, dst); break;
        case T_Q8_0: encode_q8_0(src, dst); break;
        case T_Q8_1: encode_q8_1(src, dst); break;
        case T_Q4_K: encode_q4_k(src, dst); break;
        case T_Q5_K: encode_q5_k(src, dst); break;
        default: encode_q6_k(src, dst); break;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Single-token matvec: y[i] = sum_k w_ik x_k in f64 (exact products, summed  */
/* in order), plus a[i] = sum_k |w_ik x_k|, the scale of the error bound.    */
/* ------------------------------------------------------------------------- */

static void dot_row(int type, const uint8_t *row, int64_t K, const float *x, float *wbuf,
                    double *y, double *a)
{
    decode_row(type, row, K, wbuf);
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double p = (double)wbuf[k] * (double)x[k];
        s += p;
        t += fabs(p);
    }
    *y = s;
    *a = t;
}

/* Rows given by index; a may be NULL. */
int oracle_qmv_rows(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x,
                    int64_t nrows, const int64_t *rows, double *y, double *a)
{
    if (!shape_ok(type, M, K) || !blocks || !x || !y || (nrows > 0 && !rows)) return -1;
    float *wbuf = (float *)malloc((size_t)K * sizeof(float));
    if (!wbuf) return -1;
    size_t rb = row_bytes(type, K);
    for (int64_t t = 0; t < nrows; t++) {
        if (rows[t] < 0 || rows[t] >= M) { free(wbuf); return -1; }
        double at;
        dot_row(type, blocks + (size_t)rows[t] * rb, K, x, wbuf, &y[t], &at);
        if (a) a[t] = at;
    }
    free(wbuf);
    return 0;
}

int oracle_qmv(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x,
               double *y, double *a)
{
    if (!shape_ok(type, M, K) || !blocks || !x || !y) return -1;
    float *wbuf = (float *)malloc((size_t)K * sizeof(float));
    if (!wbuf) return -1;
    size_t rb = row_bytes(type, K);
    for (int64_t r = 0; r < M; r++) {
        double at;
        dot_row(type, blocks + (size_t)r * rb, K, x, wbuf, &y[r], &at);
        if (a) a[r] = at;
    }
    free(wbuf);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gated FFN input (BebeLM page, section "核心算子": h = silu(g) * u with the  */
/* gate and up projections; FlareLLM page, section "推理层面的深度优化": gate  */
/* and up stacked as one matrix): the stack has 2I rows, rows 0..I-1 gate and */
/* I..2I-1 up; g_j = row j . x, u_j = row I+j . x (f64 as in the matvec),     */
/* h_j = g_j / (1 + e^-g_j) * u_j.  g, u, a_g, a_u may be NULL.               */
/* ------------------------------------------------------------------------- */

int oracle_gate_up_silu(int type, const uint8_t *blocks, int64_t I, int64_t K, const float *x,
                        double *h, double *g, double *u, double *a_g, double *a_u)
{
    if (I < 1 || !shape_ok(type, 2 * I, K) || !blocks || !x || !h) return -1;
    float *wbuf = (float *)malloc((size_t)K * sizeof(float));
    if (!wbuf) return -1;
    size_t rb = row_bytes(type, K);
    for (int64_t j = 0; j < I; j++) {
        double gv, uv, ag, au;
        dot_row(type, blocks + (size_t)j * rb, K, x, wbuf, &gv, &ag);
        dot_row(type, blocks + (size_t)(I + j) * rb, K, x, wbuf, &uv, &au);
        h[j] = gv / (1.0 + exp(-gv)) * uv;
        if (g) g[j] = gv;
        if (u) u[j] = uv;
        if (a_g) a_g[j] = ag;
        if (a_u) a_u[j] = au;
    }
    free(wbuf);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Gated short convolution for one token (BebeLM page, section "门控短卷积"   */
/* and "核心算子": B, C, x = split(in_proj(h), 3); Bx = B * x; a causal        */
/* depthwise convolution of kernel size 3 over the Bx sequence, its state the */
/* last 2 positions; y = C * conv_out; out = out_proj(y)).                    */
/* in_proj: 3D rows x H columns (rows 0..D-1 B, D..2D-1 C, 2D..3D-1 x);       */
/* out_proj: H rows x D columns.  w_conv[c][k], k = 0..2: tap k multiplies    */
/* the input k - 2 positions back, so conv_out_c = w[c][0] s[c][0] +           */
/* w[c][1] s[c][1] + w[c][2] Bx_c with s[c][0] the older and s[c][1] the       */
/* newer cached Bx (causal: only the current and past inputs).  The state    */
/* after the token is (s[c][1], Bx_c).  All in f64; state_in is read as       */
/* given.  Outputs (NULL to skip): y[D], bx[D], out[H], a_out[H] =            */
/* sum_j |W_out[i,j] y_j|, and A[3D] = the in_proj rows' sum |w h|.            */
/* ------------------------------------------------------------------------- */

int oracle_short_conv(int in_type, const uint8_t *in_proj, int64_t D, int64_t H, const float *h,
                      const float *w_conv, const float *state_in, int out_type,
                      const uint8_t *out_proj, double *state_out, double *y, double *bx_out,
                      double *out, double *a_out, double *A)
{
    if (D < 1 || !shape_ok(in_type, 3 * D, H) || !in_proj || !h || !w_conv || !state_in)
        return -1;
    if (out && (!out_proj || !shape_ok(out_type, H, D))) return -1;
    float *wbuf = (float *)malloc((size_t)(H > D ? H : D) * sizeof(float));
    double *yy = (double *)malloc((size_t)D * sizeof(double));
    if (!wbuf || !yy) { free(wbuf); free(yy); return -1; }
    size_t rb = row_bytes(in_type, H);
    for (int64_t c = 0; c < D; c++) {
        double b, cc, xv, ab, ac, ax;
        dot_row(in_type, in_proj + (size_t)c * rb, H, h, wbuf, &b, &ab);
        dot_row(in_type, in_proj + (size_t)(D + c) * rb, H, h, wbuf, &cc, &ac);
        dot_row(in_type, in_proj + (size_t)(2 * D + c) * rb, H, h, wbuf, &xv, &ax);
        double bx = b * xv;
        double s0 = state_in[2 * c], s1 = state_in[2 * c + 1];
        double conv = (double)w_conv[3 * c] * s0 + (double)w_conv[3 * c + 1] * s1 +
                      (double)w_conv[3 * c + 2] * bx;
        yy[c] = cc * conv;
        if (y) y[c] = yy[c];
        if (bx_out) bx_out[c] = bx;
        if (state_out) {
            state_out[2 * c] = s1;
            state_out[2 * c + 1] = bx;
        }
        if (A) {
            A[c] = ab;
            A[D + c] = ac;
            A[2 * D + c] = ax;
        }
    }
    if (out) {
        size_t orb = row_bytes(out_type, D);
        for (int64_t i = 0; i < H; i++) {
            decode_row(out_type, out_proj + (size_t)i * orb, D, wbuf);
            double acc = 0.0, at = 0.0;
            for (int64_t j = 0; j < D; j++) {
                double p = (double)wbuf[j] * yy[j];
                acc += p;
                at += fabs(p);
            }
            out[i] = acc;
            if (a_out) a_out[i] = at;
        }
    }
    free(wbuf);
    free(yy);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Greedy argmax of dequant(W) x: the lowest index among the maximal exact   */
/* (f64) row results.  Also returns that row's value and its sum |w x|.      */
/* ------------------------------------------------------------------------- */

int oracle_argmax(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x,
                  int64_t *idx, double *vmax, double *a_at)
{
    if (!shape_ok(type, M, K) || !blocks || !x || !idx || !vmax) return -1;
    float *wbuf = (float *)malloc((size_t)K * sizeof(float));
    if (!wbuf) return -1;
    size_t rb = row_bytes(type, K);
    int64_t best = -1;
    double bv = 0.0, ba = 0.0;
    for (int64_t r = 0; r < M; r++) {
        double y, a;
        dot_row(type, blocks + (size_t)r * rb, K, x, wbuf, &y, &a);
        if (best < 0 || y > bv) { best = r; bv = y; ba = a; }
    }
    free(wbuf);
    *idx = best;
    *vmax = bv;
    if (a_at) *a_at = ba;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Small batch: Y[j][i] = sum_k w_ik X[j][k] for j < n (X row-major n x K,    */
/* Y row-major n x M), the same f64 sums as the matvec, one column at a time. */
/* ------------------------------------------------------------------------- */

int oracle_gemm_n(int type, const uint8_t *blocks, int64_t M, int64_t K, int32_t n,
                  const float *X, double *Y, double *A)
{
    if (!shape_ok(type, M, K) || !blocks || !X || !Y || n < 1) return -1;
    float *wbuf = (float *)malloc((size_t)K * sizeof(float));
    if (!wbuf) return -1;
    size_t rb = row_bytes(type, K);
    for (int64_t r = 0; r < M; r++) {
        decode_row(type, blocks + (size_t)r * rb, K, wbuf);
        for (int32_t j = 0; j < n; j++) {
            const float *xj = X + (size_t)j * (size_t)K;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)wbuf[k] * (double)xj[k];
                s += p;
                t += fabs(p);
            }
            Y[(size_t)j * (size_t)M + (size_t)r] = s;
            if (A) A[(size_t)j * (size_t)M + (size_t)r] = t;
        }
    }
    free(wbuf);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* MoE FFN for one token (BebeLM page, section "核心算子", MoE FFN):          */
/*  1. router logits r_e = R[e,:] . x (R is E x H f32, row per expert)       */
/*  2. scores s_e = sigmoid(r_e) (sigmoid, not softmax)                      */
/*  3. pick the k experts with the largest s_e + b_e; the bias only ranks,   */
/*     ties go to the lower expert index; slots are in descending rank       */
/*  4. weights w = s_sel / sum(s_sel) (renormalised over the selected,      */
/*     unbiased scores)                                                      */
/*  5. per selected expert: g = G_e x, u = U_e x (gate rows 0..I-1 and up    */
/*     rows I..2I-1 of the expert's 2I x H block matrix), h = silu(g) * u,   */
/*     y_e = D_e h (D_e is H x I)                                            */
/*  6. y = sum over slots of w * y_e                                         */
/* All in f64.  Expert e's gate/up matrix starts e * 2I rows into gate_up;   */
/* its down matrix starts e * H rows into down.  Optional outputs (NULL to   */
/* skip): logits[E], scores[E], g/u/h[k][I] per slot, a_y[H] = sum over      */
/* slots of w * sum_j |D_e[i,j] h_j|.                                        */
/* ------------------------------------------------------------------------- */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_moe(const float *x, int64_t H, const float *router, const float *bias,
               int32_t E, int32_t k, int gu_type, const uint8_t *gate_up,
               int dn_type, const uint8_t *down, int64_t I,
               double *y, int32_t *sel, double *wsel,
               double *logits, double *scores, double *g_out, double *u_out, double *h_out,
               double *a_y)
{
    if (!x || !router || !bias || !gate_up || !down || !y || !sel || !wsel) return -1;
    if (E < 1 || k < 1 || k > E || H < 1 || I < 1) return -1;
    if (!shape_ok(gu_type, 2 * I, H) || !shape_ok(dn_type, H, I)) return -1;
    double *r = (double *)malloc((size_t)E * sizeof(double));
    double *s = (double *)malloc((size_t)E * sizeof(double));
    char *taken = (char *)calloc((size_t)E, 1);
    float *wrow = (float *)malloc((size_t)(H > I ? H : I) * sizeof(float));
    double *h = (double *)malloc((size_t)I * sizeof(double));
    if (!r || !s || !taken || !wrow || !h) {
        free(r); free(s); free(taken); free(wrow); free(h);
        return -1;
    }
    for (int32_t e = 0; e < E; e++) {
        double acc = 0.0;
        for (int64_t c = 0; c < H; c++)
            acc += (double)router[(size_t)e * (size_t)H + (size_t)c] * (double)x[c];
        r[e] = acc;
        s[e] = sigmoid(acc);
        if (logits) logits[e] = acc;
        if (scores) scores[e] = s[e];
    }
    double ssum = 0.0;
    for (int32_t t = 0; t < k; t++) {
        int32_t best = -1;
        double bv = 0.0;
        for (int32_t e = 0; e < E; e++) {
            if (taken[e]) continue;
            double v = s[e] + (double)bias[e];
            if (best < 0 || v > bv) { best = e; bv = v; }
        }
        taken[best] = 1;
        sel[t] = best;
        ssum += s[best];
    }
    for (int32_t t = 0; t < k; t++)
        wsel[t] = s[sel[t]] / ssum;
    for (int64_t i = 0; i < H; i++) {
        y[i] = 0.0;
        if (a_y) a_y[i] = 0.0;
    }
    size_t gu_rb = row_bytes(gu_type, H), dn_rb = row_bytes(dn_type, I);
    for (int32_t t = 0; t < k; t++) {
        int32_t e = sel[t];
        const uint8_t *gu = gate_up + (size_t)e * (size_t)(2 * I) * gu_rb;
        const uint8_t *dn = down + (size_t)e * (size_t)H * dn_rb;
        for (int64_t i = 0; i < I; i++) {
            double gv, uv, at;
            dot_row(gu_type, gu + (size_t)i * gu_rb, H, x, wrow, &gv, &at);
            dot_row(gu_type, gu + (size_t)(I + i) * gu_rb, H, x, wrow, &uv, &at);
            h[i] = gv / (1.0 + exp(-gv)) * uv;
            if (g_out) g_out[(size_t)t * (size_t)I + (size_t)i] = gv;
            if (u_out) u_out[(size_t)t * (size_t)I + (size_t)i] = uv;
            if (h_out) h_out[(size_t)t * (size_t)I + (size_t)i] = h[i];
        }
        for (int64_t i = 0; i < H; i++) {
            decode_row(dn_type, dn + (size_t)i * dn_rb, I, wrow);
            double acc = 0.0, at = 0.0;
            for (int64_t j = 0; j < I; j++) {
                double p = (double)wrow[j] * h[j];
                acc += p;
                at += fabs(p);
            }
            y[i] += wsel[t] * acc;
            if (a_y) a_y[i] += wsel[t] * at;
        }
    }
    free(r); free(s); free(taken); free(wrow); free(h);
    return 0;
}
