/*
 * bitlinear.h -- C ABI of the W1.58A8 BitLinear forward for AMD Instinct MI355X (gfx950).
 *
 * The operation is the BitNet b1.58 linear layer, a drop-in for nn.Linear without
 * bias: y = x W^T with W of shape [out_features = N][in_features = K]
 * ("BitNet b1.58 深度解析", s.2.2; "微软AI大模型炸场", s.2 "架构基础与创新" and
 * "偏置移除"). Weights are absmean-quantized to ternary codes {-1, 0, +1} and stored
 * four per byte; activations are quantized per token to int8 with absmax scaling;
 * the product is accumulated exactly in int32 and rescaled to fp32.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a HIP device pointer to caller-owned, row-major,
 *     contiguous memory, unless stated otherwise. Float and int8 activation buffers
 *     must be 16-byte aligned; outputs must not overlap any input.
 *   - The library allocates no memory, keeps no pointer after it returns and has no
 *     mutable global state; calls from several host threads are safe.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream). Arguments
 *     are checked before any HIP call: on an error status nothing was enqueued.
 *     A launch failure returns BITLINEAR_ERR_HIP (from hipGetLastError right after
 *     the launch). A fault inside a kernel surfaces at the caller's next
 *     synchronization with the stream.
 *   - Sizes: 1 <= M, 1 <= N <= 2^31 - 1, 4 <= K <= BITLINEAR_MAX_K, K % 4 == 0,
 *     M*K and N*K below 2^40. Non-finite inputs give unspecified results.
 *   - Rounding: every fp32 quotient is an IEEE division and every code is rounded
 *     half to even, so a CPU implementation of the same definitions reproduces the
 *     quantized codes, packed bytes and int32 accumulators bit for bit.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_MAX_K (1 << 20)
#define BITLINEAR_MAX_CONTEXT (1 << 24)

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_NULL = 1,      /* a required pointer is NULL */
    BITLINEAR_ERR_SHAPE = 2,     /* a size is out of range or K % 4 != 0 */
    BITLINEAR_ERR_ALIGN = 3,     /* a pointer lacks the alignment stated here */
    BITLINEAR_ERR_WORKSPACE = 4, /* workspace smaller than bitlinear_pack_workspace_bytes */
    BITLINEAR_ERR_ALIAS = 5,     /* an output buffer overlaps an input buffer */
    BITLINEAR_ERR_HIP = 6        /* the HIP runtime rejected a launch */
} bitlinear_status;

/* Human-readable name of a status code; never NULL. */
const char* bitlinear_status_string(int status);

/*
 * Weight quantization and packing (offline, once per matrix).
 *
 * gamma = mean |W| over the whole matrix ("absmean": "微软AI大模型炸场" s.1,
 * "20亿参数仅0.4GB" s.2; one scale per tensor as in "BitNet b1.58 深度解析" s.2.2),
 * summed in binary64 as a pairwise tree over the row-major array zero-padded to a
 * power of two, divided by N*K in binary64, rounded to fp32 and floored at 1e-8.
 * Code q = clip(round_half_even(W / gamma), -1, 1) with an fp32 division
 * ("BitNet b1.58 深度解析" s.2.2: sign(w) round(|w|/alpha)).
 * Packing ("微软AI大模型炸场" s.3: several ternary values in one 8-bit integer in HBM;
 * "BitNet b1.58 深度解析" s.2.1: 2-bit codes, one of the four states unused):
 * W_packed is uint8 [N][K/4]; byte j of row n holds codes k = 4j..4j+3, code 4j+i in
 * bits 2i..2i+1 as the field value q + 1 (0 = -1, 1 = 0, 2 = +1; 3 never written).
 *
 *   W          fp32 [N][K], 16-byte aligned (read only)
 *   W_packed   uint8 [N][K/4] (written)
 *   gamma      fp32 [1] on the device (written; read by bitlinear_forward*)
 *   workspace  device scratch of at least bitlinear_pack_workspace_bytes(N, K) bytes,
 *              8-byte aligned; its contents are undefined afterwards. Two calls that
 *              run concurrently need distinct workspaces.
 */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);
int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* gamma,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-token absmax int8 activation quantization, with an optional fused subln input.
 *
 * Plain (gain == NULL, act == 0): for token t, m = max_k |x_tk|,
 * s_t = 127 / max(m, 1e-8) (fp32 division), xq_tk = clip(round_half_even(x_tk s_t),
 * -128, 127) ("BitNet b1.58 深度解析" s.2.2; per token: "微软AI大模型炸场" s.1,
 * "20亿参数仅0.4GB" s.2).
 *
 * Fused subln input (squared ReLU: "微软AI大模型炸场" s.2 "特殊设计"; subln RMSNorm:
 * same page s.1, RMSNorm layers in "BitNet b1.58 深度解析" s.2.4; gate and up
 * projections of the FFN: "BitNet b1.58 深度解析" s.2.4):
 *   act 0: v = u;   act 1: v = max(u,0)^2;   act 2: v = max(g,0)^2 * p   (all fp32),
 * where for act 2 each token row holds 2K values, the gate g = row[0..K) followed by
 * the up projection p = row[K..2K);   w = v * gain (fp32) when gain != NULL.
 * The RMSNorm output r*w, r = 1/sqrt(mean(v^2) + eps), differs from w by a positive
 * per-token factor, which absmax quantization divides out; the codes are therefore
 * those of w, with s' = 127 / max(max|w|, 1e-8), and the stored scale is that of the
 * normalized activation, s_t = s' * sqrt(mean(v^2) + eps) (binary64, rounded to fp32).
 * act != 0 with gain == NULL applies only the activation.
 *
 *   X        fp32 [M][K] (act 0, 1) or [M][2K] (act 2), 16-byte aligned
 *   act      0, 1 or 2; any other value is BITLINEAR_ERR_SHAPE
 *   gain     fp32 [K] or NULL (no RMSNorm); eps is used only when gain != NULL
 *   Xq       int8 [M][K] (written), 4-byte aligned
 *   x_scale  fp32 [M] (written): s_t, the multiplier; dequantization is xq / s_t
 */
int bitlinear_quantize_act(const float* X, int64_t M, int64_t K, const float* gain, float eps,
                           int act, int8_t* Xq, float* x_scale, hipStream_t stream);

/*
 * The W1.58A8 product ("20亿参数仅0.4GB" s.2 BitLinear; custom W1.58A8 matmul kernel in
 * "微软以小搏大 … 原生 1bit LLM", section "微软在 1 bit LLM 上的探索"; rescale
 * y = (W_q x_q) * scale in "BitNet b1.58 深度解析" s.2.3):
 *   acc[t][n] = sum_k q[n][k] * xq[t][k]           (exact, int32)
 *   y[t][n]   = fl32(fl32(acc[t][n]) * fl32(gamma / s_t))
 *
 *   Xq        int8 [M][K], 4-byte aligned;   x_scale  fp32 [M]
 *   W_packed  uint8 [N][K/4] as written by bitlinear_pack_weights, 16-byte aligned
 *   gamma     fp32 [1] on the device
 *   Y         fp32 [M][N] (written)
 *   acc       int32 [M][N] (written) or NULL
 * A packed field equal to 3 (never written by the packer) gives unspecified results.
 * Every token count gives the same bits: the kernel (vector dot products for a few
 * tokens, the int8 matrix cores for 2..24 tokens on the shapes where they are faster and
 * for 16 tokens and more) only changes the order of exact integer additions.
 */
int bitlinear_forward(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K,
                      const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int32_t* acc,
                      hipStream_t stream);

/*
 * Fused input quantization and product in one launch: bit for bit the result of
 * bitlinear_quantize_act(X, M, K, gain, eps, act, ...) followed by bitlinear_forward,
 * without the int8 round trip through memory. Arguments as in those two calls.
 */
int bitlinear_forward_f32(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                          const uint8_t* W_packed, const float* gamma, int64_t N, float* Y,
                          hipStream_t stream);

/*
 * Residual forms: the product is added to what Y holds,
 *   Y[t][n] = fl32(Y[t][n] + y[t][n]),   y[t][n] as computed by the call without the suffix,
 * so a sublayer's output goes into the residual stream of the Transformer block
 * ("BitNet b1.58 深度解析" s.2.4: a standard Transformer block with every nn.Linear
 * replaced by BitLinear) without a separate add pass. Y is read and written by the
 * same thread; it may not overlap any input. Other arguments, layouts and errors as in
 * bitlinear_forward (without acc) and bitlinear_forward_f32.
 */
int bitlinear_forward_residual(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K,
                               const uint8_t* W_packed, const float* gamma, int64_t N, float* Y,
                               hipStream_t stream);
int bitlinear_forward_f32_residual(const float* X, int64_t M, int64_t K, const float* gain, float eps,
                                   int act, const uint8_t* W_packed, const float* gamma, int64_t N,
                                   float* Y, hipStream_t stream);

/*
 * The fused call for any number of tokens, with a caller workspace (the same operation
 * and result as bitlinear_forward_f32, or its residual form when residual != 0).
 *
 * One launch converts the input inside the product only while the tokens fit a few
 * token tiles of the decode product; from 16 tokens on every tile would read all the
 * weights again, and from 3 tokens (2 for the largest matrices) the product is faster on
 * the matrix cores. For those sizes this entry quantizes into the workspace and runs the
 * matrix-core product: bit for bit bitlinear_quantize_act followed by
 * bitlinear_forward_ws (or its residual form), the same result the one-launch call gives.
 *
 *   workspace        device scratch of at least bitlinear_forward_f32_workspace_bytes(M, N, K)
 *                    bytes, 16-byte aligned, overlapping no argument; its contents after
 *                    the call are unspecified; calls that may run concurrently need
 *                    distinct workspaces. When that size is 0 (one token, the sizes
 *                    that stay on the one-launch product, or sizes out of range) the
 *                    workspace is not used and may be NULL.
 *   residual         0: Y = product; 1: Y = fl32(Y + product)
 * Other arguments, layouts and errors as in bitlinear_forward_f32; additionally
 * BITLINEAR_ERR_NULL for a NULL workspace and BITLINEAR_ERR_WORKSPACE for a short one
 * when one is needed. bitlinear_forward_f32_workspace_bytes returns 0 for sizes out of
 * range.
 */
size_t bitlinear_forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bitlinear_forward_f32_ws(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                             const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int residual,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The fused call with a caller workspace, for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments (except the workspace) and result as bitlinear_forward_f32_ws, with
 * the workspace taken from a fixed scratch array that the library holds in each device's
 * memory from the time it is loaded until the process ends. It calls no allocating
 * routine. Limit: the sizes may need at most BITLINEAR_NOALLOC_SCRATCH_BYTES of workspace
 * (bitlinear_forward_f32_workspace_bytes(M, N, K) <= 32 MiB: the M x K codes, the M scales
 * and any K-split partials; for example 2048 tokens with K = 8192 fit); larger sizes return
 * BITLINEAR_ERR_WORKSPACE before anything is enqueued. Sizes that need no workspace (one
 * token, and the sizes the one-launch product takes) do not touch the scratch. The first
 * call on each device looks up that device's copy of the array (hipGetSymbolAddress; make
 * that call outside graph capture); a failed lookup returns
 * BITLINEAR_ERR_HIP. Every call on one device shares that device's array, which keeps the
 * last call's contents: calls that may overlap on one device (several streams or host
 * threads) race on it and must be ordered by the caller.
 */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (32u << 20)
int bitlinear_forward_f32_noalloc(const float* X, int64_t M, int64_t K, const float* gain, float eps, int act,
                                  const uint8_t* W_packed, const float* gamma, int64_t N, float* Y, int residual,
                                  hipStream_t stream);

/*
 * The product with a caller workspace (the same operation and result as bitlinear_forward,
 * or bitlinear_forward_residual when residual != 0; "BitNet b1.58 深度解析" s.2.3).
 *
 * With few tokens (10 to 32, or 8 on matrices of >= 64M weights) and long rows
 * (K >= 16384) the matrix-core product has too
 * few output tiles to occupy the GPU and each tile walks all of K in sequence. With a
 * workspace the K range is cut into up to 8 slices computed by separate blocks, each
 * writing its exact int32 partial sum to the workspace; a second launch adds the slices
 * (integer addition: the same accumulator in any order) and applies the rescale of the
 * unsplit product, so the result is bit for bit that of bitlinear_forward. The partials
 * then stay within a quarter of the packed weight bytes; for other sizes the workspace
 * size is 0 and the call is bitlinear_forward's.
 *
 *   workspace   device scratch of at least bitlinear_forward_workspace_bytes(M, N, K)
 *               bytes (the slices' int32 partials), 16-byte aligned, overlapping no
 *               argument; contents unspecified after the call; concurrent calls need
 *               distinct workspaces. When that size is 0 (no split for these sizes) the
 *               workspace is not used and may be NULL.
 * Other arguments, layouts and errors as in bitlinear_forward; additionally
 * BITLINEAR_ERR_NULL / BITLINEAR_ERR_WORKSPACE for a missing or short workspace when one
 * is needed. bitlinear_forward_workspace_bytes returns 0 for sizes out of range.
 */
size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bitlinear_forward_ws(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed,
                         const float* gamma, int64_t N, float* Y, int32_t* acc, int residual, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Five ternary codes per byte (1.6 bits per weight) instead of four: "微软AI大模型炸场"
 * s.3 packs several trits into one 8-bit integer, and "BitNet b1.58 深度解析" s.2.1 notes
 * that a 2-bit field leaves one of its four states unused; 3^5 = 243 <= 256.
 *
 * Format: byte j of row n is the base-3 numeral sum_{i=0..4} (q[n][5j+i] + 1) * 3^i
 * (first code least significant; q = 0 past K). A row is
 * bitlinear_packed5_row_bytes(K) = 16 * ceil(K / 80) bytes; bytes past the row's codes
 * encode five zero codes (121). gamma is the one bitlinear_pack_weights computes.
 *
 * bitlinear_packed5_row_bytes returns 0 for an invalid K.
 *
 * bitlinear_repack5 converts bitlinear_pack_weights' 2-bit layout W_packed [N][K/4] into
 * this one, W_packed5 [N][row bytes] (4-byte aligned, written; must not overlap W_packed).
 *
 * bitlinear_forward5 is bitlinear_forward on W_packed5: the same exact int32 sums and
 * the same rescale, y[t][n] = fl32(fl32(acc[t][n]) * fl32(gamma / s_t)). K must be a
 * multiple of 16 and at most 131072 (a token's codes are staged in LDS), N below
 * 2^27; Xq and W_packed5 16-byte aligned. A byte above
 * 242 (never written by the packer) gives unspecified results.
 */
int64_t bitlinear_packed5_row_bytes(int64_t K);
int bitlinear_repack5(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W_packed5, hipStream_t stream);
int bitlinear_forward5(const int8_t* Xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* W_packed5,
                       const float* gamma, int64_t N, float* Y, int32_t* acc, hipStream_t stream);

/*
 * Decode attention at real context length: one new token per sequence attends over its
 * key/value cache. Scaled dot-product attention ("BitNet b1.58 深度解析" s.2.4 block
 * diagram, between the Q/K/V and output BitLinears) with rotary position embedding
 * ("微软AI大模型炸场" s.2, 特殊设计) and grouped-query heads: query head h reads KV head
 * h / (heads / kv_heads). The pages fix neither the rotary layout nor the cache format;
 * this library rotates dimension i with dimension i + head_dim/2 by the angle
 * pos * theta^(-2i/head_dim) and stores keys and values as bfloat16.
 *
 *   qkv       fp32 [M][(heads + 2 kv_heads) * head_dim]: the new token's query heads,
 *             then key heads, then value heads (the Q/K/V BitLinear's output); read only
 *   k_cache   bf16 bit patterns [M][kv_heads][capacity][head_dim]: rotated keys; slot
 *   v_cache   pos[t] of sequence t is written, slots 0 .. pos[t]-1 are read, the others
 *             are neither read nor written
 *   pos       int32 [M] on the device: the new token's position per sequence
 *   out       fp32 [M][heads * head_dim] (written)
 *   workspace device scratch of at least bitlinear_attention_workspace_bytes(M, heads,
 *             capacity) bytes, 16-byte aligned, contents undefined afterwards; concurrent
 *             calls need distinct workspaces
 *
 * For each sequence t with 0 <= p = pos[t] < capacity:
 *   k' = rotate(k, p) in binary32: cos and sin of the binary64 angle rounded once to
 *        binary32, then x1*c - x2*s and x2*c + x1*s with each product and sum rounded;
 *   k_cache[t][g][p] = bf16(k'_g), v_cache[t][g][p] = bf16(v_g) (nearest, ties to even);
 *   out[t][h] = sum_{j<=p} softmax_j(rotate(q_h, p) . K[j] / sqrt(head_dim)) V[j] over
 *        the cache rows of KV head g(h) (in fp32, weights as exp2 of base-2 scores).
 * A sequence whose pos lies outside [0, capacity) gets NaN outputs and its caches are left
 * untouched (pos is read on the device, so this is not an error status).
 *
 * Requirements: head_dim == 128; heads a multiple of kv_heads, heads <= 4096;
 * 1 <= M <= 65535; 1 <= capacity <= BITLINEAR_MAX_CONTEXT; theta > 0 and finite; every
 * pointer 16-byte aligned (pos 4-byte). No written buffer (caches, out, workspace) may
 * overlap any other argument buffer. Two kernels are enqueued on `stream` (rotate, append
 * and attend over 64-position chunks; merge the chunks).
 * bitlinear_attention_workspace_bytes returns 0 for out-of-range sizes.
 */
size_t bitlinear_attention_workspace_bytes(int64_t M, int64_t heads, int64_t capacity);
int bitlinear_attention_decode(const float* qkv, uint16_t* k_cache, uint16_t* v_cache, const int32_t* pos,
                               int64_t M, int64_t heads, int64_t kv_heads, int64_t head_dim, int64_t capacity,
                               double theta, float* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
