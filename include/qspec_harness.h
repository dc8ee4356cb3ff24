/*
 * qspec_harness.h -- decoder kernels of libqspec.so that surround the
 * dual-mode linear layers in the end-to-end self-speculative loop, plus the
 * device-side bookkeeping of one speculation round.
 *
 * The loop follows "QSpec: Speculative Decoding with Complementary
 * Quantization Schemes", Abstract (arXiv): drafting and verification run the
 * same model and reuse the same weights and the same KV cache; here the
 * verify forward overwrites the cache rows of every position it processes.
 * The draft/verify/rewrite cycle is the one the agihunt.info review of
 * SpecQuant describes in its method paragraph.  The pages name no model
 * architecture: these kernels implement the plain Llama-style reading
 * (pre-norm RMSNorm with weight 1, rotate-half RoPE, grouped-query causal
 * attention with head size 128 and scale 1/sqrt(128), SwiGLU with gate|up as
 * one matrix, gate rows first).
 *
 * Conventions are those of qspec.h (device pointers owned by the caller,
 * asynchronous on `stream`, host-side validation, nothing allocated), except
 * alignment: pointers need only the alignment of their element type, save
 * `emb`, which must be 16-byte aligned.  Every kernel computes each row
 * independently with a fixed operation order, so a row's result is the same
 * whatever other rows share the call.
 *
 * Rounding points: residual stream fp32; GEMM inputs bf16 (normalised
 * activations, attention output, silu * up); keys (after RoPE) and values
 * bf16 in the cache; queries after RoPE fp32.  Values headed for bf16 are
 * computed in fp64 and rounded once, to nearest even.
 *
 * KV cache of one layer: K and V each bf16 [B][n_kv][cap][128].
 */
#ifndef QSPEC_HARNESS_H_
#define QSPEC_HARNESS_H_

#include "qspec.h"

#ifdef __cplusplus
extern "C" {
#endif

#define QSPEC_HEAD_DIM 128
#define QSPEC_MAX_CAP 3968  /* positions per sequence in a KV cache */
#define QSPEC_MAX_D 4096    /* model width handled by qspec_add_rmsnorm */

/* x[m][:] = float(emb[tok[m]][:]).  emb bf16 bits [V][d] (d % 8 == 0, 16-byte
 * aligned), tok int32 [M] (ids outside [0, V) are clamped), x fp32 [M][d]. */
qspec_status qspec_embed(const uint16_t* emb, int64_t V, int64_t d, const int32_t* tok,
                         int64_t M, float* x, qspec_stream stream);

/* Residual add and RMSNorm: x[m] += add[m] (skipped when add is NULL; the sum
 * is rounded to fp32 and stored back into x), then
 * y[m] = bf16(x[m] / sqrt(mean(x[m]^2) + eps)).  x and add are fp32 rows of
 * strides x_stride, add_stride >= d elements (add may be NULL), y bf16 bits
 * [M][d] (dense); 1 <= d <= 4096.  A row's result does not depend on the
 * other rows of the call; it is computed by one of two kernels whose fp64
 * sums of squares associate differently -- the 16-byte one when d % 4 == 0,
 * x, add (and their strides) are 16-byte aligned and y 8-byte aligned, a
 * scalar one otherwise -- so the same row given in the two layouts may
 * round y one bf16 unit apart. */
qspec_status qspec_add_rmsnorm(float* x, int64_t x_stride, const float* add, int64_t add_stride,
                               int64_t M, int64_t d, double eps, uint16_t* y,
                               qspec_stream stream);

/* RoPE and KV write.  qkv fp32 [M][(n_heads + 2 n_kv) * 128] = [q | k | v];
 * row m belongs to sequence seq[m] at position pos[m].  q_out fp32
 * [M][n_heads * 128] = q after RoPE; the cache rows [seq][g][pos][:] of
 * kcache / vcache receive bf16(k after RoPE) / bf16(v).  RoPE: the pair
 * (i, i + 64) of each head turns by pos * base^(-i/64).  Rows with seq
 * outside [0, B) or pos outside [0, cap) write nothing. */
qspec_status qspec_rope_kv(const float* qkv, int64_t M, int n_heads, int n_kv,
                           const int32_t* seq, const int32_t* pos, double rope_base,
                           float* q_out, uint16_t* kcache, uint16_t* vcache, int64_t B,
                           int64_t cap, qspec_stream stream);

/* Causal grouped-query attention: query head h of row m (q fp32
 * [M][n_heads * 128]) attends to cache positions 0..pos[m] of sequence
 * seq[m], key/value head h / (n_heads / n_kv); softmax(K q / sqrt(128))
 * weights the values; out bf16 [M][n_heads * 128].  n_heads % n_kv == 0;
 * cap <= QSPEC_MAX_CAP.  Rows outside the cache produce zeros. */
qspec_status qspec_attention(const float* q, const uint16_t* kcache, const uint16_t* vcache,
                             int64_t M, int n_heads, int n_kv, const int32_t* seq,
                             const int32_t* pos, int64_t B, int64_t cap, uint16_t* out,
                             qspec_stream stream);

/* qspec_rope_kv followed by qspec_attention, in one launch, for launches
 * whose M rows belong to M different sequences (decode and draft forwards:
 * one row per sequence).  Same arguments, results (bit for bit) and errors as
 * the two calls; out bf16 [M][n_heads * 128].  Precondition, not checked:
 * no two rows share a sequence (rows of one sequence would race on its
 * cache rows; results are then undefined, every access stays in bounds). */
qspec_status qspec_rope_attention(const float* qkv, int64_t M, int n_heads, int n_kv,
                                  const int32_t* seq, const int32_t* pos, double rope_base,
                                  float* q_out, uint16_t* kcache, uint16_t* vcache, int64_t B,
                                  int64_t cap, uint16_t* out, qspec_stream stream);

/* qspec_add_rmsnorm with the drafter's input in the same pass: besides y,
 * yq [M][d/2] and ys [M] receive exactly what qspec_quant_act gives for the
 * bf16 rows y (per-token absmax / 7, codes rne(y / s) clamped, nibble
 * packed), one launch instead of two in every draft forward.  d is a
 * multiple of 128 (<= 4096); yq, ys 16-byte aligned; other arguments and
 * errors as for qspec_add_rmsnorm. */
qspec_status qspec_add_rmsnorm_quant(float* x, int64_t x_stride, const float* add,
                                     int64_t add_stride, int64_t M, int64_t d, double eps,
                                     uint16_t* y, uint8_t* yq, float* ys, qspec_stream stream);

/* qspec_add_rmsnorm with the W4A8 drafter's input in the same pass: besides
 * y, yq int8 [M][d] and ys [M] receive exactly what qspec_quant_act8 gives
 * for the bf16 rows y (per-token absmax / 127, codes rne(y / s) clamped to
 * [-128, 127]; the 8-bit middle tier on the shared INT4 weights, a reading
 * of the 8-bit variant in "SpecQuant: Speculative Decoding with
 * Multi-Parent Quantization for Adaptive LLM Inference", Abstract), one
 * launch instead of two in every W4A8 draft forward.  d is a multiple of
 * 128 (<= 4096); yq, ys 16-byte aligned; other arguments and errors as for
 * qspec_add_rmsnorm. */
qspec_status qspec_add_rmsnorm_quant8(float* x, int64_t x_stride, const float* add,
                                      int64_t add_stride, int64_t M, int64_t d, double eps,
                                      uint16_t* y, int8_t* yq, float* ys, qspec_stream stream);

/* SwiGLU: a[m][j] = bf16(silu(g) * u), g = gu[m][j], u = gu[m][ffn + j],
 * silu(g) = g / (1 + exp(-g)).  gu fp32 [M][2 ffn], a bf16 bits [M][ffn]. */
qspec_status qspec_silu_mul(const float* gu, int64_t M, int64_t ffn, uint16_t* a,
                            qspec_stream stream);

/* SwiGLU over gate|up outputs in pair order (the row order of
 * qspec_gemm_w4a16_swiglu's buffer): gu fp32 [M][2 ffn], in each 16-column
 * block b columns 16b .. 16b+7 gate and 16b+8 .. 16b+15 the matching up
 * values; a[m][8b + i] = bf16(silu(gu[m][16b+i]) * gu[m][16b+8+i]) as in
 * qspec_silu_mul.  ffn % 8 == 0. */
qspec_status qspec_silu_mul_pairs(const float* gu, int64_t M, int64_t ffn, uint16_t* a,
                                  qspec_stream stream);

/* out[m * out_stride] = the lowest index of the largest value of row m of
 * x fp32 [M][V]. */
qspec_status qspec_argmax(const float* x, int64_t M, int64_t V, int32_t* out,
                          int64_t out_stride, qspec_stream stream);

/* Row set-up of one forward of a speculation round, from the device state
 * len int32 [B] (tokens so far, prompt included) and vtok int32 [B][gamma+1]
 * (column 0: the last emitted token, columns 1.. the drafts so far).
 *   phase 0, draft step j (0 <= j <= gamma, gamma >= 0): B rows,
 *     seq = b, pos = len[b] - 1 + j, tok = vtok[b][j];
 *   phase 1, verify (gamma >= 1): B (gamma + 1) rows r = b (gamma+1) + i,
 *     seq = b, pos = len[b] - 1 + i, tok = vtok[b][i]; also
 *     drafts[b][i-1] = vtok[b][i] (drafts int32 [B][gamma]).
 * seq/pos/tok int32 arrays of the row count. */
qspec_status qspec_spec_prepare(int phase, int64_t B, int gamma, int j, const int32_t* len,
                                const int32_t* vtok, int32_t* drafts, int32_t* seq,
                                int32_t* pos, int32_t* tok, qspec_stream stream);

/* End of a round: for every sequence with n_gen[b] < max_gen, append
 * out_tok[b][0..n] to gen[b][n_gen[b]..] (n = n_accept[b], or 0 when
 * n_accept is NULL; entries past gen_cap are dropped), add n + 1 to n_gen[b]
 * and len[b], and set vtok[b * vtok_stride] = out_tok[b][n].  out_tok int32
 * [B][gamma+1] (gamma >= 0), gen int32 [B][gen_cap].  stats int64 [3]:
 * stats[0] += accepted drafts, stats[1] += sequences active this round,
 * stats[2] = sequences still short of max_gen afterwards.  B <= 65536. */
qspec_status qspec_spec_commit(int64_t B, int gamma, const int32_t* n_accept,
                               const int32_t* out_tok, int32_t* len, int32_t* vtok,
                               int64_t vtok_stride, int32_t* gen, int64_t gen_cap,
                               int32_t* n_gen, int max_gen, int64_t* stats,
                               qspec_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QSPEC_HARNESS_H_ */
