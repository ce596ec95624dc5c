/*
 * bitlinear_oracle.c -- plain CPU oracle of the W1.58A8 BitLinear forward.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline call this file. The product library never links, loads or calls it, and
 * it shares no code, header, table or helper with the HIP path.
 *
 * Plain C99, single thread, no intrinsics. Build with -O2 -ffp-contract=off and
 * without -ffast-math: every fp32 operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even, every fp64 operation one binary64 operation.
 *
 * Sources (page title, section):
 *   [P1] "微软AI大模型炸场：0.4GB，CPU就能跑，中国团队打造！"  section 1 "极致量化"
 *        (absmean ternary weights; per-token absmax 8-bit activations; subln) and
 *        section 3 "软硬协同" (several trits packed into one byte in HBM).
 *   [P3] "微软以小搏大 … 发布首个开源 2B 参数范围 '原生 1bit' LLM"  section
 *        "权重映射为三元值 {-1, 0, +1}" (absmean, per-token absmax, subln).
 *   [P4] "20亿参数仅0.4GB … 「原生1.58bit」大模型"  section 2 "核心创新 / BitLinear层".
 *   [P5] "BitNet b1.58 深度解析：微软如何用1.58位量化颠覆大模型推理范式"
 *        section 2.1 (2-bit codes, one of four states unused), section 2.2
 *        (w_t = sign(w) * round(|w|/alpha); 127/max(|x|, 1e-8), round, clamp to
 *        [-128, 127]), section 2.3 (y = (W_q x_q) * scale).
 *
 * Readings where the pages are silent (each is listed with its reason in the design
 * notes): one gamma per matrix; gamma's fp64 sum taken as a pairwise tree over the
 * row-major array zero-padded to a power of two; ties rounded to even; 1e-8 floors on
 * both max|x| and gamma; code = t + 1 in field i at bits 2i of byte k/4; the per-token
 * subln RMSNorm factor cancels inside absmax and is kept only in the stored scale.
 *
 * Parity status of each function: pinned by tests/test_oracle_pins.py (closed forms,
 * hand-built examples under tests/golden/, brute force and library routines).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORA_FLOOR 1e-8f

/* ---------------------------------------------------------------------------------
 * O1  gamma = mean |W|  ("absmean": [P1] s.1, [P3], [P4] s.2; whole-tensor mean as in
 *     [P5] s.2.2 where the mean of |W| is taken over the full weight tensor).
 *
 * The sum of |W| is done in binary64 as the textbook pairwise recursion over the
 * row-major array, conceptually zero-extended to the next power of two P >= n:
 *     S(lo, len) = |W[lo]|                        if len == 1
 *                = S(lo, len/2) + S(lo+len/2, len/2)  otherwise
 * Ranges that start at or beyond n are zeros and contribute +0.0 (x + 0.0 == x).
 * ------------------------------------------------------------------------------- */
static double abs_sum_range(const float* w, int64_t n, int64_t lo, int64_t len)
{
    if (lo >= n)
        return 0.0;
    if (len == 1)
        return fabs((double)w[lo]);
    int64_t half = len / 2;
    return abs_sum_range(w, n, lo, half) + abs_sum_range(w, n, lo + half, half);
}

double ora_abs_sum(const float* w, int64_t n)
{
    int64_t p = 1;
    while (p < n)
        p *= 2;
    return abs_sum_range(w, n, 0, p);
}

float ora_weight_scale(const float* w, int64_t n)
{
    double s = ora_abs_sum(w, n);
    float gamma = (float)(s / (double)n);
    if (gamma < ORA_FLOOR)
        gamma = ORA_FLOOR;
    return gamma;
}

/* ---------------------------------------------------------------------------------
 * O2  ternary code  q = clip(round(W / gamma), -1, 1)
 *     [P5] s.2.2 writes sign(w) * round(|w| / alpha); with round-half-even that is the
 *     same as round(w / alpha) because the rounding is symmetric. The quotient is one
 *     fp32 division; the rounding is round-half-to-even (rintf in the default mode).
 * ------------------------------------------------------------------------------- */
void ora_weight_codes(const float* w, int64_t n, float gamma, int8_t* q)
{
    for (int64_t i = 0; i < n; ++i) {
        float r = rintf(w[i] / gamma);
        if (r > 1.0f)
            r = 1.0f;
        if (r < -1.0f)
            r = -1.0f;
        q[i] = (int8_t)r;
    }
}

/* ---------------------------------------------------------------------------------
 * O3  packing, four codes per byte  ([P1] s.3: several trits in one 8-bit integer in
 *     HBM; [P5] s.2.1: a 2-bit field has four states, one unused).
 *     Row-major [N][K/4]; byte j of row n holds codes k = 4j .. 4j+3, code k = 4j+i in
 *     bits 2i..2i+1 as the unsigned field value q + 1 (0 -> -1, 1 -> 0, 2 -> +1; 3 unused).
 * ------------------------------------------------------------------------------- */
void ora_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed)
{
    int64_t kb = K / 4;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < kb; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                unsigned field = (unsigned)(q[n * K + 4 * j + i] + 1);
                byte |= field << (2 * i);
            }
            packed[n * kb + j] = (uint8_t)byte;
        }
    }
}

/* Inverse of ora_pack. Returns the number of fields equal to 3 (never produced by the
 * packer); such a field decodes to +2 so that a test can see it. */
int64_t ora_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q)
{
    int64_t kb = K / 4, bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < kb; ++j) {
            unsigned byte = packed[n * kb + j];
            for (int i = 0; i < 4; ++i) {
                unsigned field = (byte >> (2 * i)) & 3u;
                if (field == 3u)
                    ++bad;
                q[n * K + 4 * j + i] = (int8_t)((int)field - 1);
            }
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------------
 * O3b packing, five codes per byte (1.6 bits per weight): the denser alternative to
 *     the 2-bit fields ([P1] s.3: several trits in one 8-bit integer; [P5] s.2.1: a
 *     2-bit field wastes one of its four states, and more compact encodings exist).
 *     3^5 = 243 <= 256, so five base-3 digits fit in a byte.
 *     Byte j of row n holds codes k = 5j .. 5j+4 as the base-3 number
 *         sum_{i=0..4} (q[n][5j+i] + 1) * 3^i          (digit i = code 5j+i, plus one)
 *     with q = 0 for k >= K. Rows are 16 * ceil(K/80) bytes long (whole 16-byte
 *     chunks of 80 codes); bytes past the last group of the row encode five zero
 *     codes (value 121).
 * ------------------------------------------------------------------------------- */
int64_t ora_pack5_row_bytes(int64_t K)
{
    return 16 * ((K + 79) / 80);
}

void ora_pack5(const int8_t* q, int64_t N, int64_t K, uint8_t* packed)
{
    int64_t rb = ora_pack5_row_bytes(K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < rb; ++j) {
            unsigned value = 0, weight = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * j + i;
                int code = k < K ? q[n * K + k] : 0;
                value += (unsigned)(code + 1) * weight;
                weight *= 3u;
            }
            packed[n * rb + j] = (uint8_t)value;
        }
    }
}

/* Inverse of ora_pack5 on the first K codes of each row. Returns the number of bytes
 * above 242 (never produced by the packer) plus the number of digits past K that are
 * not the zero code; such bytes still decode digit by digit. */
int64_t ora_unpack5(const uint8_t* packed, int64_t N, int64_t K, int8_t* q)
{
    int64_t rb = ora_pack5_row_bytes(K), bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < rb; ++j) {
            unsigned value = packed[n * rb + j];
            if (value > 242u)
                ++bad;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * j + i;
                int code = (int)(value % 3u) - 1;
                value /= 3u;
                if (k < K)
                    q[n * K + k] = (int8_t)code;
                else if (code != 0)
                    ++bad;
            }
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------------
 * O4  per-token absmax int8 activation quantization
 *     ([P1] s.1, [P3], [P4] s.2: absmax taken per token; [P5] s.2.2: scale
 *     127 / max(|x|, 1e-8), round, clamp to [-128, 127]).
 *     For token t:  m = max_k |x_tk|,  s_t = 127 / max(m, 1e-8)  (fp32 division),
 *                   xq_tk = clip(round_half_even(x_tk * s_t), -128, 127).
 *     s_t (the multiplier) is what is stored; dequantization divides by it.
 * ------------------------------------------------------------------------------- */
static int8_t quant_code(float v, float s)
{
    float r = rintf(v * s);
    if (r > 127.0f)
        r = 127.0f;
    if (r < -128.0f)
        r = -128.0f;
    return (int8_t)r;
}

void ora_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* scale)
{
    for (int64_t t = 0; t < M; ++t) {
        const float* row = x + t * K;
        float m = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > m)
                m = a;
        }
        if (m < ORA_FLOOR)
            m = ORA_FLOOR;
        float s = 127.0f / m;
        scale[t] = s;
        for (int64_t k = 0; k < K; ++k)
            xq[t * K + k] = quant_code(row[k], s);
    }
}

/* ---------------------------------------------------------------------------------
 * O5  subln input: [activation] -> RMSNorm(gain, eps) -> per-token absmax int8
 *     (subln: [P1] s.1 "归一化方法", [P3], [P4] s.2, no formula printed; RMSNorm
 *     layers before attention and FFN: [P5] s.2.4; squared ReLU in the FFN: [P1] s.2
 *     "特殊设计"; a gate projection next to the up projection: [P5] s.2.4; no bias
 *     anywhere: [P1] s.2 "偏置移除").
 *
 *     act = 0:  v_k = u_k                                   (row of K values)
 *     act = 1:  v_k = fl(p * p),        p = max(u_k, 0)     (row of K values)
 *     act = 2:  v_k = fl(fl(p * p) * up_k), p = max(gate_k, 0)
 *               (row of 2K values: gate_0..gate_{K-1}, up_0..up_{K-1})
 *     w_k  = fl(v_k * g_k)
 *     RMSNorm output is r * w with r = 1 / sqrt(mean(v^2) + eps), one positive number
 *     per token. Absmax quantization is invariant to a positive per-token factor:
 *     (r w) * 127 / max|r w| == w * 127 / max|w| in real arithmetic. The codes are
 *     therefore taken from w in fp32 exactly as in O4,
 *         s'   = 127 / max(max_k |w_k|, 1e-8),   xq = clip(rint(w * s'), -128, 127),
 *     and r survives only in the stored scale of the normalized activation,
 *         s_t  = s' / r = s' * sqrt(mean_k v_k^2 + eps)      (binary64, then to fp32).
 *     With gain == NULL no normalization is applied (only the activation).
 * ------------------------------------------------------------------------------- */
void ora_quantize_act_norm(const float* u, int64_t M, int64_t K, const float* gain, float eps,
                           int act, int8_t* xq, float* scale, float* work /* K floats */)
{
    const int64_t stride = act == 2 ? 2 * K : K;
    for (int64_t t = 0; t < M; ++t) {
        const float* row = u + t * stride;
        double sumsq = 0.0;
        float m = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = row[k];
            if (act == 1 || act == 2) {
                float p = v > 0.0f ? v : 0.0f;
                v = p * p;
                if (act == 2)
                    v = v * row[K + k];
            }
            sumsq += (double)v * (double)v;
            float w = gain ? v * gain[k] : v;
            work[k] = w;
            float a = fabsf(w);
            if (a > m)
                m = a;
        }
        if (m < ORA_FLOOR)
            m = ORA_FLOOR;
        float sp = 127.0f / m;
        for (int64_t k = 0; k < K; ++k)
            xq[t * K + k] = quant_code(work[k], sp);
        if (gain) {
            double ms = sumsq / (double)K;
            scale[t] = (float)((double)sp * sqrt(ms + (double)eps));
        } else {
            scale[t] = sp;
        }
    }
}

/* ---------------------------------------------------------------------------------
 * O6 + O7  accumulate and rescale  ([P5] s.2.3: y = (W_q x_q) * scale; [P5] s.2.2:
 *     the layer is F.linear with weight [out_features][in_features], y = x W^T, no bias;
 *     [P1] s.1: a ternary product needs only additions).
 *     acc[t][n] = sum_k q[n][k] * xq[t][k]   (exact integer; stored as int32)
 *     c_t       = gamma / s_t                (fp32 division)
 *     y[t][n]   = fl(float(acc) * c_t)
 * Returns the number of accumulators that did not fit in int32 (0 for K <= 2^24).
 * ------------------------------------------------------------------------------- */
int64_t ora_forward(const int8_t* xq, const float* scale, int64_t M, int64_t K,
                    const int8_t* q, float gamma, int64_t N, int32_t* acc, float* y)
{
    int64_t overflow = 0;
    for (int64_t t = 0; t < M; ++t) {
        float c = gamma / scale[t];
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k)
                a += (int64_t)q[n * K + k] * (int64_t)xq[t * K + k];
            if (a > INT32_MAX || a < INT32_MIN)
                ++overflow;
            acc[t * N + n] = (int32_t)a;
            y[t * N + n] = (float)a * c;
        }
    }
    return overflow;
}
