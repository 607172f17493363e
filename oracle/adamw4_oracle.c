/*
 * adamw4_oracle.c -- plain, slow CPU oracle of the fused 4-bit AdamW step (ZIP-SR / ZE-EDEN).
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the benchmark's
 * CPU-baseline leg are the only callers.  The HIP library never links, loads or calls this file
 * and the two share no code, header, table or generator.
 *
 * Sources (web pages about "Rounding in Preconditioner Space: Redesigning 4-bit AdamW
 * Optimizer-State Quantization", arXiv 2610.12444):
 *   [daiwk-CE]  daiwk.github.io notes "ZIP-SR / ZE-EDEN: 4-bit AdamW state quantization",
 *               section "Core equation": h(v), the ZIP-SR lower-level probability, the ZE-EDEN
 *               block rescale, and that weights are updated before the moments are requantized.
 *   [daiwk-PM]  same page, "Paper method and evidence" flowchart: decode -> update moments ->
 *               update weights -> ZIP-SR or ZE-EDEN -> pack.
 *   [daiwk-LR]  same page, "Local reproduction": uint8 nibble packing, FP32 block scales,
 *               FP32 fallback for tensors under 4096 elements.
 *   [lav-ST]    learnaivisually.com explainer "ZIP-SR 4-bit AdamW", storage paragraph: 4-bit m
 *               and v, one FP32 scale per 128-value block, normalization-layer states in FP32.
 *   [lav-RO]    same page, rounding-odds paragraph: state-space SR makes the mean stored value
 *               exact; ZIP-SR makes the mean multiplier 1/(sqrt(v)+eps) exact at storage time.
 *   [lav-ZE]    same page, ZE-EDEN / LM-head paragraph: NF4 for m; stochastic rounding of the
 *               LM head's m over the last 10% of training; TorchAO's positive floor for v.
 *   [kc-TC]     kongchang.com explainer, "Two Complementary Technical Approaches": ZIP-SR keeps
 *               zero in the v codebook, ZE-EDEN excludes it and rescales blocks.
 *   [kc-WHY]    same page, "Why 4-bit ... Second Look": AdamW keeps two exponential moving
 *               averages per parameter; decoupled weight decay.
 *
 * Arithmetic.  Everything that feeds a stored value or a quantization decision is IEEE binary32,
 * one rounding per operation, no FMA contraction (build with -ffp-contract=off), denormals kept.
 * The precision is the storage format's: FP32 master weights, FP32 fallback states, FP32 block
 * scales ([lav-ST], [daiwk-LR]).  Per-step scalars are formed in binary64 and rounded once.
 *
 * Readings of points the pages leave open (all listed in the design notes):
 *   - NF4 words: the QLoRA normal-quantile construction evaluated in binary64, rounded to FP32.
 *   - zero-inclusive v codebook V0[k] = k/15; zero-excluding V1[k] = (k+1)/16.
 *   - block scale = absmax; quantization works on y = x * fl(1/max(s, FLT_MIN)).
 *   - RTN: count of codebook midpoints strictly below y (ties go to the lower code).
 *   - ZIP-SR probability written in block-normalised coordinates (same value as the printed
 *     ratio of h differences, no underflow for tiny blocks); see orc_zip_p.
 *   - ZE-EDEN: RTN on V1, then gamma = sum(y^2) / max(sum(y * V1[code]), 1e-12), both sums by
 *     a recursive pairwise tree over the 128 zero-padded slots; stored scale gamma * s.
 *   - the controlled study's other v rules ([lav-RO]) on the zero-inclusive codebook:
 *     state-space RTN (nearest level), state-space SR (lower level with probability
 *     (b-y)/(b-a)), preconditioner-space RTN (the level with the nearest h; a tie goes low).
 *   - the baseline the pages measure against: RTN on the zero-free V1, absmax scale, no rescale
 *     (ZE-EDEN without its gamma).
 *   - RNG: Philox4x32-10 (Salmon et al., SC'11) keyed by the seed, counter
 *     (j lo, j hi | stream<<31, tensor position, t) with j = i >> 2; u = (word >> 8) * 2^-24;
 *     the lower level is chosen iff u < p.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>
#include <omp.h>

#define ORC_BLOCK 128
#define ORC_MIN_QUANT 4096

/* v encoders: the two methods, the controlled study's other rules on the zero-inclusive
 * codebook ([lav-RO]: state-space round-to-nearest and stochastic rounding, preconditioner-space
 * round-to-nearest), and the baseline the pages compare against ([lav-ZE], [lav-ST]: the
 * zero-free codebook with its positive floor, round to nearest, plain absmax scale) */
enum { ORC_ZIP_SR = 0, ORC_ZE_EDEN = 1, ORC_V_RTN = 2, ORC_V_SSR = 3, ORC_V_PRTN = 4,
       ORC_V_ZE_RTN = 5 };

/* codebook that a v encoded under `mode` decodes with: the zero-free one for ZE-EDEN and for
 * the baseline rule (round to nearest on the zero-free codebook, absmax scale, no rescale) */
static int uses_v1(int mode) { return mode == ORC_ZE_EDEN || mode == ORC_V_ZE_RTN; }
enum { ORC_CB_NF4 = 0, ORC_CB_V0 = 1, ORC_CB_V1 = 2 };

typedef struct {
    int64_t step;
    float lr, beta1, beta2, eps, weight_decay;
    int32_t mode;      /* v encoder used this step */
    int32_t prev_mode; /* codebook that encoded the incoming v (-1: same as mode) */
    int32_t sr_head;   /* 1: HEAD tensors' m uses stochastic rounding this step */
    uint64_t seed;
} orc_hparams;

/* IEEE behaviour on every thread: clear flush-to-zero and denormals-are-zero. */
static void ieee_mode(void) { _mm_setcsr(_mm_getcsr() & ~(0x8000u | 0x0040u)); }

/* ------------------------------------------------------------------------------------------ */
/* Codebooks                                                                                  */
/* ------------------------------------------------------------------------------------------ */

/* Standard normal CDF and its inverse by bisection: slow and plainly correct. */
static double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static double std_normal_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 400; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (std_normal_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* NF4 (QLoRA, Dettmers et al. 2023): 8 positive levels are the normal quantiles of 8 evenly
 * spaced probabilities from delta towards 1/2 (9 points, 1/2 dropped), 7 negative levels the
 * mirrored quantiles of 7 evenly spaced probabilities (8 points, 1/2 dropped), plus exact zero;
 * all divided by the largest, so the endpoints are -1 and +1.  delta is the mean of 1 - 1/30
 * and 1 - 1/32.  The pages name NF4 for m without printing its words ([lav-ZE], [kc-TC]). */
static void nf4_table(float out[16]) {
    const double delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
    const double top = std_normal_quantile(delta);
    double lv[16];
    int n = 0;
    for (int i = 0; i <= 6; ++i) { /* negatives, ascending */
        double p = delta + (0.5 - delta) * (double)i / 7.0;
        lv[n++] = -std_normal_quantile(p) / top;
    }
    lv[n++] = 0.0;
    for (int i = 7; i >= 0; --i) { /* positives, ascending */
        double p = delta + (0.5 - delta) * (double)i / 8.0;
        lv[n++] = std_normal_quantile(p) / top;
    }
    for (int k = 0; k < 16; ++k) out[k] = (float)lv[k];
}

/* Zero-inclusive 16-level v codebook for ZIP-SR: k/15 ([kc-TC]: zero is kept). */
static void v0_table(float out[16]) {
    for (int k = 0; k < 16; ++k) out[k] = (float)((double)k / 15.0);
}

/* Zero-excluding v codebook for ZE-EDEN: (k+1)/16, lowest level 1/16 ([lav-ST]: the
 * zero-free codebook's lowest level is positive; [lav-ZE]: TorchAO's positive floor is kept). */
static void v1_table(float out[16]) {
    for (int k = 0; k < 16; ++k) out[k] = (float)(k + 1) / 16.0f;
}

void orc_codebook(int which, float out[16]) {
    if (which == ORC_CB_NF4) nf4_table(out);
    else if (which == ORC_CB_V0) v0_table(out);
    else v1_table(out);
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of two 32x32->64 products     */
/* whose halves are xored with the other counter words and the round key; the key is bumped   */
/* by the Weyl constants between rounds.                                                      */
/* ------------------------------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform u in [0,1) with 24 bits for element i of a tensor: stream 0 = v, 1 = LM-head m. */
float orc_uniform(uint64_t seed, int64_t t, uint32_t pos, int stream, int64_t i) {
    uint64_t j = (uint64_t)i >> 2;
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32) | ((uint32_t)stream << 31), pos, (uint32_t)t};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return (float)(w[i & 3] >> 8) * 0x1p-24f;
}

/* ------------------------------------------------------------------------------------------ */
/* Per-step scalars: bias corrections 1-beta^t in binary64, each scalar rounded once.          */
/* ([daiwk-CE]: h carries the bias-corrected v; AdamW's step carries 1/(1-beta1^t).)          */
/* ------------------------------------------------------------------------------------------ */

typedef struct { float step_size, rs2, decay, omb1, omb2; } orc_scalars_t;

static orc_scalars_t scalars_of(const orc_hparams* hp) {
    orc_scalars_t s;
    double b1 = hp->beta1, b2 = hp->beta2, t = (double)hp->step;
    double bc1 = 1.0 - pow(b1, t), bc2 = 1.0 - pow(b2, t);
    s.step_size = (float)((double)hp->lr / bc1);
    s.rs2 = (float)(1.0 / sqrt(bc2));
    s.decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    s.omb1 = (float)(1.0 - b1);
    s.omb2 = (float)(1.0 - b2);
    return s;
}

void orc_step_scalars(const orc_hparams* hp, float out[5]) {
    orc_scalars_t s = scalars_of(hp);
    out[0] = s.step_size; out[1] = s.rs2; out[2] = s.decay; out[3] = s.omb1; out[4] = s.omb2;
}

/* ------------------------------------------------------------------------------------------ */
/* Element-level AdamW (decoupled weight decay, bias correction) in FP32.                     */
/* ------------------------------------------------------------------------------------------ */

static float widen_grad(const void* g, int g_bf16, int64_t i) {
    if (!g_bf16) return ((const float*)g)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)g)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

typedef struct { float w, m, v; } orc_elem;

/* m' = beta1 m + (1-beta1) g;  v' = beta2 v + (1-beta2) g^2;
 * w' = (1 - lr wd) w - (lr/bc1) * m' / (sqrt(v') / sqrt(bc2) + eps)
 * The weight uses the unquantized working moments ([daiwk-CE], [daiwk-PM]). */
static orc_elem adamw_elem(float w, float g, float m, float v, const orc_hparams* hp,
                           const orc_scalars_t* s) {
    orc_elem r;
    float m1 = hp->beta1 * m;
    float m2 = s->omb1 * g;
    r.m = m1 + m2;
    float gg = g * g;
    float v1 = hp->beta2 * v;
    float v2 = s->omb2 * gg;
    r.v = v1 + v2;
    float root = sqrtf(r.v);
    float den = root * s->rs2;
    den = den + hp->eps;
    float q = r.m / den;
    float upd = s->step_size * q;
    float dw = s->decay * w;
    r.w = dw - upd;
    return r;
}

/* ------------------------------------------------------------------------------------------ */
/* Block quantizers.  A block is 128 slots; slots past the end of the tensor hold 0.          */
/* ------------------------------------------------------------------------------------------ */

/* Recursive pairwise sum S[lo, lo+len) = S[lo, lo+len/2) + S[lo+len/2, lo+len). */
static float pairwise_sum(const float* x, int lo, int len) {
    if (len == 1) return x[lo];
    int h = len / 2;
    float a = pairwise_sum(x, lo, h);
    float b = pairwise_sum(x, lo + h, h);
    return a + b;
}

static float inv_scale(float s) { return 1.0f / fmaxf(s, FLT_MIN); }

/* number of codebook midpoints 0.5*(C[k]+C[k+1]) strictly below y: round to nearest level,
 * a tie goes to the lower code */
static int rtn_code(const float C[16], float y) {
    int code = 0;
    for (int k = 0; k < 15; ++k) {
        float mid = 0.5f * (C[k] + C[k + 1]);
        if (y > mid) ++code;
    }
    return code;
}

/* the cell [C[k], C[k+1]) holding y: largest k <= 14 with C[k] <= y (0 if none) */
static int cell_of(const float C[16], float y) {
    int k = 0;
    for (int j = 1; j < 15; ++j)
        if (C[j] <= y) k = j;
    return k;
}

/* ZIP-SR probability of the lower level alpha = V0[k] for a value y in block-normalised units.
 * The pages give p = [h(v) - h(b)] / [h(a) - h(b)] with h(x) = 1/(sqrt(x/bc2) + eps)
 * ([daiwk-CE]).  With x = y*s, a = alpha*s, b = beta*s and c = sqrt(s)*rs2 this is
 *   p = (sqrt(beta) - sqrt(y)) (sqrt(alpha) c + eps) / ((sqrt(beta) - sqrt(alpha)) (sqrt(y) c + eps))
 * and sqrt(beta) - sqrt(q) = (beta - q)/(sqrt(beta) + sqrt(q)) removes the cancellation:
 *   p = ((beta-y)(sqrt(beta)+sqrt(alpha)))(sqrt(alpha) c + eps) / (((beta-alpha)(sqrt(beta)+sqrt(y)))(sqrt(y) c + eps)).
 * Evaluated in FP32 in exactly this order. */
float orc_zip_p(float y, float alpha, float beta, float c, float eps) {
    float sa = sqrtf(alpha), sb = sqrtf(beta), sy = sqrtf(y);
    float n1 = beta - y;
    float n2 = sb + sa;
    float n3 = sa * c;
    n3 = n3 + eps;
    float num = n1 * n2;
    num = num * n3;
    float d1 = beta - alpha;
    float d2 = sb + sy;
    float d3 = sy * c;
    d3 = d3 + eps;
    float den = d1 * d2;
    den = den * d3;
    return num / den;
}

/* The printed formula, literally, in binary64 (for checking orc_zip_p). */
double orc_zip_p64(double v, double a, double b, double bc2, double eps) {
    double hv = 1.0 / (sqrt(v / bc2) + eps);
    double ha = 1.0 / (sqrt(a / bc2) + eps);
    double hb = 1.0 / (sqrt(b / bc2) + eps);
    return (hv - hb) / (ha - hb);
}

/* Debug record per element (optional): u and p of the v choice and of the m choice; p = -1
 * where no random choice was made. */
typedef struct { float u_v, p_v, u_m, p_m; } orc_dbg;

/* m block: absmax scale, NF4 RTN, or state-space SR between adjacent NF4 levels when sr != 0
 * (LM-head tensor in the last 10% of steps, [lav-ZE]).  SR picks the lower level with
 * probability (beta - y)/(beta - alpha), which keeps the mean stored value exact ([lav-RO]). */
static void encode_m_block(const float* x, int nvalid, int sr, const float NF4[16],
                           uint64_t seed, int64_t t, uint32_t pos, int64_t i0,
                           uint8_t* codes, float* scale, orc_dbg* dbg) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, fabsf(x[j]));
    *scale = s;
    for (int j = 0; j < ORC_BLOCK; ++j) {
        if (dbg && j < nvalid) { dbg[j].u_m = -1.0f; dbg[j].p_m = -1.0f; }
        if (s == 0.0f) { codes[j] = 7; continue; }
        float inv = inv_scale(s);
        float y = x[j] * inv;
        if (!sr) { codes[j] = (uint8_t)rtn_code(NF4, y); continue; }
        int k = cell_of(NF4, y);
        float lo = NF4[k], hi = NF4[k + 1];
        if (y <= lo) { codes[j] = (uint8_t)k; continue; }
        if (y >= hi) { codes[j] = (uint8_t)(k + 1); continue; }
        float p = (hi - y) / (hi - lo);
        float u = orc_uniform(seed, t, pos, 1, i0 + j);
        if (dbg && j < nvalid) { dbg[j].u_m = u; dbg[j].p_m = p; }
        codes[j] = (uint8_t)(u < p ? k : k + 1);
    }
}

/* v block under ZIP-SR ([daiwk-CE], [lav-RO]): absmax scale; pick the cell [V0[k], V0[k+1]) of
 * the normalised value and choose the lower level with the preconditioner-space probability. */
static void encode_v_zip_block(const float* x, int nvalid, const float V0[16], float rs2, float eps,
                               uint64_t seed, int64_t t, uint32_t pos, int64_t i0,
                               uint8_t* codes, float* scale, orc_dbg* dbg) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);
    *scale = s;
    float c = sqrtf(s) * rs2;
    for (int j = 0; j < ORC_BLOCK; ++j) {
        if (dbg && j < nvalid) { dbg[j].u_v = -1.0f; dbg[j].p_v = -1.0f; }
        if (s == 0.0f) { codes[j] = 0; continue; }
        float inv = inv_scale(s);
        float y = x[j] * inv;
        int k = cell_of(V0, y);
        float lo = V0[k], hi = V0[k + 1];
        if (y <= lo) { codes[j] = (uint8_t)k; continue; }
        if (y >= hi) { codes[j] = (uint8_t)(k + 1); continue; }
        float p = orc_zip_p(y, lo, hi, c, eps);
        float u = orc_uniform(seed, t, pos, 0, i0 + j);
        if (dbg && j < nvalid) { dbg[j].u_v = u; dbg[j].p_v = p; }
        codes[j] = (uint8_t)(u < p ? k : k + 1);
    }
}

/* v block under ZE-EDEN ([daiwk-CE], [kc-TC]): RTN on the zero-excluding codebook, then the
 * EDEN rescale gamma = |x|^2 / max(<x, Q(x)>, 1e-12 s^2), computed on normalised values (divide
 * numerator and denominator by s^2); the stored scale is gamma * s. */
static void encode_v_eden_block(const float* x, const float V1[16], uint8_t* codes, float* scale) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);
    if (s == 0.0f) {
        for (int j = 0; j < ORC_BLOCK; ++j) codes[j] = 0;
        *scale = 0.0f;
        return;
    }
    float inv = inv_scale(s);
    float sq[ORC_BLOCK], xq[ORC_BLOCK];
    for (int j = 0; j < ORC_BLOCK; ++j) {
        float y = x[j] * inv;
        int code = rtn_code(V1, y);
        codes[j] = (uint8_t)code;
        sq[j] = y * y;
        xq[j] = y * V1[code]; /* padding slots hold y = 0 and add nothing */
    }
    float nrm = pairwise_sum(sq, 0, ORC_BLOCK);
    float dot = pairwise_sum(xq, 0, ORC_BLOCK);
    float gamma = nrm / fmaxf(dot, 1e-12f);
    *scale = gamma * s;
}

/* deterministic encoder for initial states: RTN on the given codebook (no RNG; t is not
 * defined before the first step).  ZE-EDEN adds its rescale. */
static void encode_v_rtn_block(const float* x, const float V0[16], uint8_t* codes, float* scale) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);
    *scale = s;
    for (int j = 0; j < ORC_BLOCK; ++j) {
        if (s == 0.0f) { codes[j] = 0; continue; }
        codes[j] = (uint8_t)rtn_code(V0, x[j] * inv_scale(s));
    }
}

/* v block, state-space stochastic rounding on the zero-inclusive codebook (the controlled
 * study's state-space SR, [lav-RO]; the worked example's 75% chance of storing zero): the lower
 * level of the cell is kept with probability (beta - y)/(beta - alpha), so the mean stored v is
 * exact.  Same RNG stream and counter as ZIP-SR. */
static void encode_v_ssr_block(const float* x, int nvalid, const float V0[16], uint64_t seed,
                               int64_t t, uint32_t pos, int64_t i0, uint8_t* codes, float* scale,
                               orc_dbg* dbg) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);
    *scale = s;
    for (int j = 0; j < ORC_BLOCK; ++j) {
        if (dbg && j < nvalid) { dbg[j].u_v = -1.0f; dbg[j].p_v = -1.0f; }
        if (s == 0.0f) { codes[j] = 0; continue; }
        float y = x[j] * inv_scale(s);
        int k = cell_of(V0, y);
        float lo = V0[k], hi = V0[k + 1];
        if (y <= lo) { codes[j] = (uint8_t)k; continue; }
        if (y >= hi) { codes[j] = (uint8_t)(k + 1); continue; }
        float p = (hi - y) / (hi - lo);
        float u = orc_uniform(seed, t, pos, 0, i0 + j);
        if (dbg && j < nvalid) { dbg[j].u_v = u; dbg[j].p_v = p; }
        codes[j] = (uint8_t)(u < p ? k : k + 1);
    }
}

/* v block, preconditioner-space round to nearest on the zero-inclusive codebook (the controlled
 * study's deterministic preconditioner-space rule, [lav-RO]): the level whose multiplier h is
 * nearest to h(v).  h is decreasing, so it is one of the two levels of the cell, and with p the
 * ZIP-SR lower-level probability h(alpha) - h(v) = (1-p)(h(alpha) - h(beta)) and
 * h(v) - h(beta) = p (h(alpha) - h(beta)): the lower level is nearer iff p > 1/2; a tie goes to
 * the lower code.  The debug record carries u = 1/2 as the threshold p is compared with. */
static void encode_v_prtn_block(const float* x, int nvalid, const float V0[16], float rs2,
                                float eps, uint8_t* codes, float* scale, orc_dbg* dbg) {
    float s = 0.0f;
    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);
    *scale = s;
    float c = sqrtf(s) * rs2;
    for (int j = 0; j < ORC_BLOCK; ++j) {
        if (dbg && j < nvalid) { dbg[j].u_v = -1.0f; dbg[j].p_v = -1.0f; }
        if (s == 0.0f) { codes[j] = 0; continue; }
        float y = x[j] * inv_scale(s);
        int k = cell_of(V0, y);
        float lo = V0[k], hi = V0[k + 1];
        if (y <= lo) { codes[j] = (uint8_t)k; continue; }
        if (y >= hi) { codes[j] = (uint8_t)(k + 1); continue; }
        float p = orc_zip_p(y, lo, hi, c, eps);
        if (dbg && j < nvalid) { dbg[j].u_v = 0.5f; dbg[j].p_v = p; }
        codes[j] = (uint8_t)(p >= 0.5f ? k : k + 1);
    }
}

/* nibble packing: element 2q in the low nibble of byte q, element 2q+1 in the high nibble;
 * nibbles past the end of the tensor are 0 ([daiwk-LR]: uint8 nibble packing). */
static void pack_block(const uint8_t* codes, int nvalid, uint8_t* bytes) {
    for (int q = 0; q < ORC_BLOCK / 2; ++q) {
        if (2 * q >= nvalid) break;
        uint8_t lo = codes[2 * q], hi = (2 * q + 1 < nvalid) ? codes[2 * q + 1] : 0;
        bytes[q] = (uint8_t)(lo | (hi << 4));
    }
}

static int unpack(const uint8_t* bytes, int j) {
    uint8_t b = bytes[j >> 1];
    return (j & 1) ? (b >> 4) : (b & 15);
}

/* ------------------------------------------------------------------------------------------ */
/* Public oracle entry points                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* FP32 fallback tensor (numel < 4096 or a normalization layer, [lav-ST], [daiwk-LR]):
 * plain FP32 AdamW on cnt elements. */
void orc_step_fp32(float* w, const void* g, int g_bf16, int64_t cnt, float* m, float* v,
                   const orc_hparams* hp) {
    ieee_mode();
    orc_scalars_t s = scalars_of(hp);
    for (int64_t i = 0; i < cnt; ++i) {
        orc_elem r = adamw_elem(w[i], widen_grad(g, g_bf16, i), m[i], v[i], hp, &s);
        w[i] = r.w; m[i] = r.m; v[i] = r.v;
    }
}

/* v of one block by the encoder of hp->mode (v decoded with the previous step's codebook). */
static void encode_v_by_mode(const float* vw, int nvalid, const orc_hparams* hp,
                             const orc_scalars_t* s, const float V0[16], const float V1[16],
                             uint32_t pos, int64_t i0, uint8_t* cv, float* vscale, orc_dbg* d) {
    switch (hp->mode) {
    case ORC_ZIP_SR:
        encode_v_zip_block(vw, nvalid, V0, s->rs2, hp->eps, hp->seed, hp->step, pos, i0, cv, vscale, d);
        break;
    case ORC_ZE_EDEN: encode_v_eden_block(vw, V1, cv, vscale); break;
    case ORC_V_RTN: encode_v_rtn_block(vw, V0, cv, vscale); break;
    case ORC_V_SSR: encode_v_ssr_block(vw, nvalid, V0, hp->seed, hp->step, pos, i0, cv, vscale, d); break;
    case ORC_V_ZE_RTN: encode_v_rtn_block(vw, V1, cv, vscale); break;
    default: encode_v_prtn_block(vw, nvalid, V0, s->rs2, hp->eps, cv, vscale, d); break;
    }
}

/* Quantized tensor of n elements; this call covers elements [e0, e0 + cnt), e0 a multiple of
 * 128.  Every array points at the data for element e0: w[0], g[0], codes byte e0/2, scale
 * e0/128.  pos is the tensor's position in the step's tensor list (RNG key), is_head marks the
 * LM-head tensor.  dbg (optional) receives 4 floats per element (u_v, p_v, u_m, p_m).
 * Returns 0, or -1 on a bad range. */
int orc_step_quant(float* w, const void* g, int g_bf16, int64_t n, int64_t e0, int64_t cnt,
                   uint8_t* mcodes, uint8_t* vcodes, float* mscale, float* vscale,
                   int is_head, uint32_t pos, const orc_hparams* hp, float* dbg_out) {
    if (e0 < 0 || cnt < 0 || (e0 % ORC_BLOCK) != 0 || e0 + cnt > n) return -1;
    if (hp->mode < ORC_ZIP_SR || hp->mode > ORC_V_ZE_RTN) return -1;
    if (cnt == 0) return 0;
    float NF4[16], V0[16], V1[16];
    nf4_table(NF4); v0_table(V0); v1_table(V1);
    /* ZE-EDEN's and the baseline's codebook excludes zero; the others use the zero-inclusive one */
    const float* Vin = uses_v1(hp->prev_mode < 0 ? hp->mode : hp->prev_mode) ? V1 : V0;
    orc_scalars_t s = scalars_of(hp);
    int sr_m = (is_head && hp->sr_head) ? 1 : 0;
    int64_t nblk = (cnt + ORC_BLOCK - 1) / ORC_BLOCK;
    orc_dbg* dbg = (orc_dbg*)dbg_out;

#pragma omp parallel
    {
        ieee_mode();
#pragma omp for schedule(static)
        for (int64_t b = 0; b < nblk; ++b) {
            int64_t lo = b * ORC_BLOCK;                    /* local index of the block's first slot */
            int nvalid = (int)((cnt - lo) < ORC_BLOCK ? (cnt - lo) : ORC_BLOCK);
            float mw[ORC_BLOCK], vw[ORC_BLOCK];
            uint8_t cm[ORC_BLOCK], cv[ORC_BLOCK];
            float sm_old = mscale[b], sv_old = vscale[b];
            for (int j = 0; j < ORC_BLOCK; ++j) {
                if (j >= nvalid) { mw[j] = 0.0f; vw[j] = 0.0f; continue; }
                int64_t i = lo + j;
                float m = NF4[unpack(mcodes + lo / 2, j)] * sm_old;
                float v = Vin[unpack(vcodes + lo / 2, j)] * sv_old;
                orc_elem r = adamw_elem(w[i], widen_grad(g, g_bf16, i), m, v, hp, &s);
                w[i] = r.w; mw[j] = r.m; vw[j] = r.v;
            }
            orc_dbg* d = dbg ? dbg + lo : NULL;
            encode_m_block(mw, nvalid, sr_m, NF4, hp->seed, hp->step, pos, e0 + lo, cm, &mscale[b], d);
            encode_v_by_mode(vw, nvalid, hp, &s, V0, V1, pos, e0 + lo, cv, &vscale[b], d);
            pack_block(cm, nvalid, mcodes + lo / 2);
            pack_block(cv, nvalid, vcodes + lo / 2);
        }
    }
    return 0;
}

/* A quantized tensor whose first moment stays in FP32 (the controlled study's configuration,
 * [lav-RO]: FP32 first moments, 4-bit v on the zero-inclusive codebook): m32 holds the cnt FP32
 * first moments for elements [e0, e0 + cnt) and is updated in place; v is decoded, updated and
 * encoded exactly as in orc_step_quant.  Returns 0, or -1 on a bad range or mode. */
int orc_step_fp32m(float* w, const void* g, int g_bf16, int64_t n, int64_t e0, int64_t cnt,
                   float* m32, uint8_t* vcodes, float* vscale, uint32_t pos,
                   const orc_hparams* hp, float* dbg_out) {
    if (e0 < 0 || cnt < 0 || (e0 % ORC_BLOCK) != 0 || e0 + cnt > n) return -1;
    if (hp->mode < ORC_ZIP_SR || hp->mode > ORC_V_ZE_RTN) return -1;
    if (cnt == 0) return 0;
    float V0[16], V1[16];
    v0_table(V0); v1_table(V1);
    const float* Vprev = uses_v1(hp->prev_mode < 0 ? hp->mode : hp->prev_mode) ? V1 : V0;
    orc_scalars_t s = scalars_of(hp);
    int64_t nblk = (cnt + ORC_BLOCK - 1) / ORC_BLOCK;
    orc_dbg* dbg = (orc_dbg*)dbg_out;

#pragma omp parallel
    {
        ieee_mode();
#pragma omp for schedule(static)
        for (int64_t b = 0; b < nblk; ++b) {
            int64_t lo = b * ORC_BLOCK;
            int nvalid = (int)((cnt - lo) < ORC_BLOCK ? (cnt - lo) : ORC_BLOCK);
            float vnew[ORC_BLOCK];
            uint8_t cv[ORC_BLOCK];
            float sv_old = vscale[b];
            for (int j = 0; j < ORC_BLOCK; ++j) {
                if (j >= nvalid) { vnew[j] = 0.0f; continue; }
                int64_t i = lo + j;
                float v_old = Vprev[unpack(vcodes + lo / 2, j)] * sv_old;
                orc_elem e = adamw_elem(w[i], widen_grad(g, g_bf16, i), m32[i], v_old, hp, &s);
                w[i] = e.w;
                m32[i] = e.m;
                vnew[j] = e.v;
            }
            if (dbg)
                for (int j = 0; j < nvalid; ++j) { dbg[lo + j].u_m = -1.0f; dbg[lo + j].p_m = -1.0f; }
            encode_v_by_mode(vnew, nvalid, hp, &s, V0, V1, pos, e0 + lo, cv, &vscale[b],
                             dbg ? dbg + lo : NULL);
            pack_block(cv, nvalid, vcodes + lo / 2);
        }
    }
    return 0;
}

/* Encode given FP32 moments (NULL: zeros) into packed state, deterministically (RTN; ZE-EDEN
 * adds its rescale).  cnt elements starting at element e0 (multiple of 128). */
int orc_encode_init(const float* m0, const float* v0, int64_t n, int64_t e0, int64_t cnt, int mode,
                    uint8_t* mcodes, uint8_t* vcodes, float* mscale, float* vscale) {
    if (e0 < 0 || cnt < 0 || (e0 % ORC_BLOCK) != 0 || e0 + cnt > n) return -1;
    float NF4[16], V0[16], V1[16];
    nf4_table(NF4); v0_table(V0); v1_table(V1);
    int64_t nblk = (cnt + ORC_BLOCK - 1) / ORC_BLOCK;
    ieee_mode();
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t lo = b * ORC_BLOCK;
        int nvalid = (int)((cnt - lo) < ORC_BLOCK ? (cnt - lo) : ORC_BLOCK);
        float mw[ORC_BLOCK], vw[ORC_BLOCK];
        uint8_t cm[ORC_BLOCK], cv[ORC_BLOCK];
        for (int j = 0; j < ORC_BLOCK; ++j) {
            mw[j] = (j < nvalid && m0) ? m0[lo + j] : 0.0f;
            vw[j] = (j < nvalid && v0) ? v0[lo + j] : 0.0f;
        }
        encode_m_block(mw, nvalid, 0, NF4, 0, 0, 0, 0, cm, &mscale[b], NULL);
        if (mode == ORC_ZE_EDEN) encode_v_eden_block(vw, V1, cv, &vscale[b]);
        else encode_v_rtn_block(vw, uses_v1(mode) ? V1 : V0, cv, &vscale[b]);
        pack_block(cm, nvalid, mcodes + lo / 2);
        pack_block(cv, nvalid, vcodes + lo / 2);
    }
    return 0;
}

/* Decode cnt elements of packed state (codes byte 0 = element e0, e0 a multiple of 128):
 * m = NF4[code] * s_m, v = V[code] * s_v with V the codebook of `mode` ([daiwk-PM] decode). */
void orc_decode(const uint8_t* mcodes, const uint8_t* vcodes, const float* mscale,
                const float* vscale, int64_t cnt, int mode, float* m_out, float* v_out) {
    float NF4[16], V0[16], V1[16];
    nf4_table(NF4); v0_table(V0); v1_table(V1);
    const float* V = uses_v1(mode) ? V1 : V0;
    ieee_mode();
    for (int64_t i = 0; i < cnt; ++i) {
        int64_t b = i / ORC_BLOCK;
        int mc = (mcodes[i >> 1] >> ((i & 1) * 4)) & 15;
        int vc = (vcodes[i >> 1] >> ((i & 1) * 4)) & 15;
        if (m_out) m_out[i] = NF4[mc] * mscale[b];
        if (v_out) v_out[i] = V[vc] * vscale[b];
    }
}

/* Block encoders exposed for the pin tests: one 128-slot block (x padded with zeros by the
 * caller), codes unpacked, rule 0 = m RTN, 1 = m SR, 2 = v ZIP-SR, 3 = v ZE-EDEN, 4 = v RTN on
 * V0 (also init), 5 = v state-space SR, 6 = v preconditioner-space RTN, 7 = v RTN on V1 (the
 * baseline).  i0 is the global element index of slot 0 (RNG counter). */
void orc_encode_block(const float* x, int nvalid, int rule, float rs2, float eps, uint64_t seed,
                      int64_t t, uint32_t pos, int64_t i0, uint8_t* codes, float* scale,
                      float* dbg_out) {
    float NF4[16], V0[16], V1[16];
    nf4_table(NF4); v0_table(V0); v1_table(V1);
    ieee_mode();
    orc_dbg* d = (orc_dbg*)dbg_out;
    switch (rule) {
    case 0: encode_m_block(x, nvalid, 0, NF4, seed, t, pos, i0, codes, scale, d); break;
    case 1: encode_m_block(x, nvalid, 1, NF4, seed, t, pos, i0, codes, scale, d); break;
    case 2: encode_v_zip_block(x, nvalid, V0, rs2, eps, seed, t, pos, i0, codes, scale, d); break;
    case 3: encode_v_eden_block(x, V1, codes, scale); break;
    case 5: encode_v_ssr_block(x, nvalid, V0, seed, t, pos, i0, codes, scale, d); break;
    case 6: encode_v_prtn_block(x, nvalid, V0, rs2, eps, codes, scale, d); break;
    case 7: encode_v_rtn_block(x, V1, codes, scale); break;
    default: encode_v_rtn_block(x, V0, codes, scale); break;
    }
}

/* BF16 copy of FP32 weights (the model-side weights refreshed from the FP32 masters): the
 * upper half of the binary32 pattern rounded to nearest, ties to even, i.e. adding 0x7FFF plus
 * the kept half's lowest bit before truncating.  Finite inputs; a value past the largest BF16
 * rounds to infinity as IEEE rounding does. */
void orc_bf16_rne(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], sizeof u);
        uint32_t keep_lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + keep_lsb) >> 16);
    }
}

/* Threads the block loops use (OpenMP), and a way to set them: bookkeeping for timing runs. */
int orc_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
