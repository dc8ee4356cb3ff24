/*
 * qspec.h -- C ABI of libqspec.so: the hot path of quantization-based
 * self-speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * One packed INT4 weight buffer is read by two modes of the same linear layer:
 * a W4A4 drafter (weights and activations at four bits) and a W4A16 verifier
 * (weights at four bits, bf16 activations); a verify step then accepts or
 * rewrites the drafted tokens.
 *   Pages: "QSpec: Speculative Decoding with Complementary Quantization
 *   Schemes", Abstract (arXiv) -- low-precision joint quantization drafts,
 *   high-precision weight-only quantization verifies, weights and KV cache are
 *   reused across the two stages; the tech-dashboard summary of QSpec,
 *   paragraphs 2-4 (W4A16 vs W4A4; draft-then-verify; one shared set of
 *   quantized weights); the agihunt.info review of SpecQuant, method paragraph
 *   (a full match is accepted, the first mismatch is rewritten by the parent).
 * The pages print no formula, layout or precision for these operations; the
 * readings used are stated at each call.
 *
 * Conventions for every call
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps a pointer after the call returns.
 *  - Arrays are dense and row-major; sizes are int64_t element counts; every
 *    array pointer must be 16-byte aligned (QSPEC_ERR_ALIGN otherwise).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  Buffers must stay alive until that work completes.
 *  - Outputs are fully overwritten, never accumulated into.  Inputs and
 *    outputs must not overlap.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and the status says why (qspec_last_error()
 *    gives a thread-local message).  A failed launch returns QSPEC_ERR_HIP.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Calls never abort or exit the process.  They are thread-safe.  Global
 *    state: a per-device cache of the device check and the per-device
 *    scratch array of qspec_verify_noalloc (read its note).
 *  - Non-finite inputs (NaN/Inf weights, activations or logits) are not
 *    supported: results are unspecified, but every kernel still terminates.
 */
#ifndef QSPEC_H_
#define QSPEC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int qspec_status;
typedef void* qspec_stream;

enum {
  QSPEC_OK = 0,
  QSPEC_ERR_NULL = -1,        /* a required pointer is NULL                  */
  QSPEC_ERR_SHAPE = -2,       /* a size is out of range or inconsistent      */
  QSPEC_ERR_UNSUPPORTED = -3, /* group != 128, unknown mode or variant       */
  QSPEC_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned            */
  QSPEC_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required     */
  QSPEC_ERR_DEVICE = -6,      /* current device is not gfx950                */
  QSPEC_ERR_HIP = -7          /* a HIP runtime call or launch failed         */
};

/* operation ids for qspec_workspace_bytes */
enum { QSPEC_OP_GEMM_W4A4 = 1, QSPEC_OP_GEMM_W4A16 = 2, QSPEC_OP_VERIFY = 3, QSPEC_OP_GEMM_W4A8 = 4 };

/* verify modes */
enum { QSPEC_VERIFY_GREEDY = 0, QSPEC_VERIFY_SAMPLE = 1 };

/* GEMM kernel families.  Within one family every output row is computed by
 * the same sequence of operations whatever M is, so row r of Y is bitwise
 * identical at any M; a caller that needs this (for example greedy
 * self-speculation that must reproduce plain verifier decoding token for
 * token) passes the same explicit family for every M.  AUTO picks by M, N
 * and K: STREAM for M <= 16 (W4A4) or M <= 8 (W4A16) when N < 16384 (where
 * SKINNY would have too few workgroups to fill the GPU), else SKINNY up to
 * M = 128 (W4A16) or
 * M = 256 (W4A4), TILED beyond -- except that TILED is taken from M = 64
 * (W4A16) or M = 96 (W4A4) when its grid has at least 256 tiles (32 x 256
 * for W4A16, 64 x 256 for W4A4), and that up to M = 512 SKINNY stays when K
 * has at least 64 groups and TILED would have fewer than 128 tiles.  The
 * W4A8 tier follows the same rule but runs SKINNY wherever it says TILED. */
enum {
  QSPEC_GEMM_AUTO = 0,
  QSPEC_GEMM_GEMV = 1,   /* W4A16 only: VALU GEMV with wavefront reduction   */
  QSPEC_GEMM_SKINNY = 2, /* MFMA, weights streamed once per up to 64 rows of
                            M, activations staged in LDS (decode, verify)   */
  QSPEC_GEMM_TILED = 3,  /* MFMA, weights straight into registers, the
                            activation slice through LDS (prefill shapes)   */
  QSPEC_GEMM_STREAM = 4  /* MFMA, M <= 16: one 16-row weight block per
                            workgroup, K split across its wavefronts and
                            reduced in LDS (decode shapes)                  */
};

#define QSPEC_GROUP 128
#define QSPEC_MAX_K (1 << 20) /* K: a multiple of 128 in [128, 2^20] */
#define QSPEC_MAX_GAMMA 16

const char* qspec_status_str(qspec_status s);
const char* qspec_last_error(void);
const char* qspec_version(void);

/* QSPEC_OK if the current HIP device is gfx950, QSPEC_ERR_DEVICE if not,
 * QSPEC_ERR_HIP if the runtime cannot be queried.  Every compute call below
 * performs this check first. */
qspec_status qspec_device_check(void);

/* Bytes of scratch `ws` that the call with these sizes needs (0 = none).
 *   QSPEC_OP_GEMM_W4A4 / _W4A16 / _W4A8:      (M, N, K)
 *   QSPEC_OP_VERIFY:                           (B, gamma, V)
 * The answer is the maximum over all variants and modes, so one workspace
 * sized by it serves every call of that op with sizes no larger.
 * A GEMM workspace must hold zeros the first time it is used (hipMemset it
 * once): the k-split's arrival counters live in its first half and count up
 * from zero; every family's partials go to its second half (the halves are
 * taken from ws_bytes, so pass one workspace with the same ws_bytes every
 * time).  Every GEMM call leaves its counters at zero again, so a workspace
 * is reused without clearing by any later GEMM call of any shape on the
 * same stream (calls that overlap in time must not share one; a call that
 * never finished, e.g. after a device fault, leaves the workspace to be
 * zeroed again).  A verify workspace needs no initialisation. */
size_t qspec_workspace_bytes(int op, int64_t a, int64_t b, int64_t c);

/* The GEMM family (QSPEC_GEMM_GEMV, _SKINNY, _TILED or _STREAM) that a call
 * of QSPEC_OP_GEMM_W4A4 / _W4A16 / _W4A8 with these M, N, K and `variant`
 * runs: AUTO resolved, which depends on M, N and K only.  Within one family
 * a row's result does not depend on M; the fused SwiGLU entries reproduce
 * their family's layer bit for bit.  Returns -1 (qspec_last_error() says
 * why) for sizes or a variant the GEMM call would reject; reads no device
 * state. */
int qspec_gemm_family(int op, int64_t M, int64_t N, int64_t K, int variant);

/* ---------------------------------------------------------------------------
 * qspec_pack_w4 -- quantize fp32 weights to the shared INT4 buffer.
 * One buffer serves both modes (QSpec Abstract: weights reused across the
 * stages; tech-dashboard summary, paragraph 4: both configurations share the
 * same quantized weights).  Reading of the unspecified format: per row n and
 * group j of 128 consecutive k,
 *     a = max|W[n,k]|;  s = fp16(a / 7.0f)  (IEEE fp32 divide, then RNE);
 *     q[n,k] = clamp(rne(W[n,k] / float(s)), -8, 7), all 0 when s == 0.
 *   W   [N][K] fp32 (in).   N >= 1, K % 128 == 0, 128 <= K <= QSPEC_MAX_K.
 *   Wq  [Np][K/2] u8 (out), Np = ceil(N/16)*16, so Np*K/2 bytes: the codes
 *       in the tiled storage order both GEMMs read.  Codes pack two per byte,
 *       code 2i of a row in bits 0-3 and code 2i+1 in bits 4-7 (two's
 *       complement); the row-major byte rows (padded with zero codes to Np
 *       rows) are stored as 1 KiB tiles, tile (b, g) for rows 16b..16b+15 and
 *       group g at byte (b*(K/128) + g)*1024; in a tile, 16-byte slot l holds
 *       row 16b + l%16, row bytes [64g + 16*(l/16), +16).  Each wavefront's
 *       weight load is then one contiguous 1 KiB.
 *   Ws  [Np][K/128] fp16 bits (out), so Np*(K/128) elements -- every one is
 *       written, padding rows with scale 0: the scale of row n and group g
 *       is element ((n/16)*(K/128) + g)*16 + n%16 (the same 16-row tiling).
 *   A caller that sizes Wq or Ws for N rather than Np rows when N % 16 != 0
 *   gets writes past its buffers.
 *   group must be 128.  Non-finite W, or a/7 beyond the fp16 range, is
 *   unsupported (results unspecified).
 * ------------------------------------------------------------------------- */
qspec_status qspec_pack_w4(const float* W, int64_t N, int64_t K, int group,
                           uint8_t* Wq, uint16_t* Ws, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_quant_act -- per-token INT4 quantization of bf16 activations (the
 * W4A4 drafter quantizes activations as well as weights: tech-dashboard
 * summary, paragraph 2; QSpec Abstract, "low-precision joint quantization").
 * Reading: per row m, a = max_k |x|, s = a / 7.0f kept in fp32, and
 * q = clamp(rne(x / s), -8, 7) with an IEEE fp32 divide (not a reciprocal
 * multiply), all codes 0 when a == 0; subnormals are kept.
 *   X   [M][K] bf16 bits (in).  M >= 1, K % 128 == 0, 128 <= K <= QSPEC_MAX_K.
 *   Xq  [M][K/2] u8 (out), same nibble layout as Wq.
 *   Xs  [M] fp32 (out).
 * ------------------------------------------------------------------------- */
qspec_status qspec_quant_act(const uint16_t* X, int64_t M, int64_t K,
                             uint8_t* Xq, float* Xs, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * Rotation ahead of the quantizers (QSpec page, Builds on: QuaRot, "Outlier-
 * Free 4-Bit Inference in Rotated LLMs" -- the pages give the title only).
 * Reading: per 128-group, the Sylvester Walsh-Hadamard matrix H (entries
 * +-1, H H^T = 128 I), activations x' = H x / 16 and weights w' = H w / 8,
 * so x' . w' = x . w and a layer on (x', w') is the layer on (x, w); the
 * group structure of the shared buffer is kept.  H is applied as the fast
 * transform: stages s = 0..6, the pair (i, i + 2^s) with bit s of i clear
 * becomes (a + b, a - b), one fp32 add or subtract each, then the exact
 * power-of-two scale -- every output bit is fixed.  With x20 outlier channels
 * this spreads each outlier over its group, so the per-token INT4 codes keep
 * the inlier channels (the W4A4 layer error drops about 3x).
 *
 * qspec_rotate_w: W [N][K] fp32 -> Wr = H W / 8 per group, fp32 (offline, then
 *   qspec_pack_w4(Wr)).  Wr may equal W.
 * qspec_rotate_x: X [M][K] bf16 bits -> Xr = bf16(H x / 16) (round to nearest
 *   even), the verifier's input to qspec_gemm_w4a16.  Xr may equal X.
 * qspec_quant_act_rot: X [M][K] bf16 bits -> the codes and scale of
 *   qspec_quant_act applied to the fp32 values H x / 16 (not rounded to
 *   bf16), the drafter's input to qspec_gemm_w4a4.  Xq [M][K/2], Xs [M].
 * K % 128 == 0 (QSPEC_ERR_SHAPE otherwise); 16-byte aligned pointers.
 * ------------------------------------------------------------------------- */
qspec_status qspec_rotate_w(const float* W, int64_t N, int64_t K, float* Wr,
                            qspec_stream stream);
qspec_status qspec_rotate_x(const uint16_t* X, int64_t M, int64_t K, uint16_t* Xr,
                            qspec_stream stream);
qspec_status qspec_quant_act_rot(const uint16_t* X, int64_t M, int64_t K,
                                 uint8_t* Xq, float* Xs, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_gemm_w4a4 -- the drafter's linear layer (QSpec Abstract: W4A4 joint
 * quantization drafts).  Reading:
 *     P[m,n,g] = sum_{k in group g} qa[m,k] * qw[n,k]     (exact int32)
 *     Y[m,n]   = Xs[m] * sum_g float(Ws[n,g]) * P[m,n,g]  (fp32 epilogue)
 * computed with int8 MFMA on the unpacked codes.  P is exact in every
 * family; the fp32 epilogue's rounding order is the family's (TILED keeps
 * a biased running sum, which adds at most about 1/85 of one unit of P per
 * group to the rounding).
 *   Xq [M][K/2], Xs [M]   from qspec_quant_act.
 *   Wq [Np][K/2], Ws [Np][K/128], Np = ceil(N/16)*16, tiled, from
 *   qspec_pack_w4.
 *   Y  [M][N] fp32 (out); exactly M*N elements are written.
 *   P  [M][N][K/128] int32 (out, optional: NULL skips it).  When given, the
 *   family that computes Y (the one `variant` or AUTO names) stores the
 *   integer group sums its own MFMA chain produced, so P checks that family.
 *   variant: QSPEC_GEMM_AUTO, _SKINNY, _TILED or _STREAM (M <= 16); GEMV is
 *   W4A16-only.
 *   ws/ws_bytes: scratch of qspec_workspace_bytes(QSPEC_OP_GEMM_W4A4,M,N,K)
 *   bytes (NULL allowed when that is 0), zero-filled before its first use
 *   (read qspec_workspace_bytes).
 * ------------------------------------------------------------------------- */
qspec_status qspec_gemm_w4a4(const uint8_t* Xq, const float* Xs,
                             const uint8_t* Wq, const uint16_t* Ws,
                             int64_t M, int64_t N, int64_t K, int group,
                             int variant, float* Y, int32_t* P,
                             void* ws, size_t ws_bytes, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_gemm_w4a4_bf16 -- the drafter's linear layer with a bf16 output, for
 * chaining into the next bf16 consumer without an fp32 round trip.  Same
 * arguments, validation, variants and workspace as qspec_gemm_w4a4 (no P);
 * Y [M][N] receives bf16 bits: the round-to-nearest-even bf16 of exactly the
 * fp32 value qspec_gemm_w4a4 stores for the same variant and inputs (finite
 * results; the conversion is the epilogue's last step, inside the kernel).
 * ------------------------------------------------------------------------- */
qspec_status qspec_gemm_w4a4_bf16(const uint8_t* Xq, const float* Xs,
                                  const uint8_t* Wq, const uint16_t* Ws,
                                  int64_t M, int64_t N, int64_t K, int group,
                                  int variant, uint16_t* Y,
                                  void* ws, size_t ws_bytes, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * A W4A8 middle tier on the same shared buffer.  SpecQuant (Abstract) derives
 * an 8-bit variant between INT4 and FP16 from one base model; QSpec's
 * Builds-on list names QServe (4-bit weights, 8-bit activations).  Reading:
 * the packed INT4 weights and fp16 group scales are read unchanged (no extra
 * copy); only the activations move to 8 bits.
 *
 * qspec_quant_act8 -- per token row: a = max|x|, s = a / 127 (fp32 IEEE
 *   divide) stored in Xs[m]; code = clamp(rne(x / s), -128, 127), one signed
 *   byte each; a == 0 gives s = 0 and zero codes.
 *   X [M][K] bf16 bits; Xq [M][K] int8 (out); Xs [M] fp32 (out).
 * qspec_gemm_w4a8 -- Y[m,n] = Xs[m] * sum_g float(Ws[n,g]) * P[m,n,g] with
 *   P the exact int32 group partial of the 8-bit codes and the 4-bit
 *   weights, computed with int8 MFMA; variant AUTO (STREAM where W4A4's AUTO
 *   takes it, else SKINNY), SKINNY or STREAM (M <= 16); GEMV and TILED give
 *   QSPEC_ERR_UNSUPPORTED.  Within one family a row's result does not depend
 *   on M.  Wq/Ws as for qspec_gemm_w4a4; Y [M][N] fp32 (out); P [M][N][K/128]
 *   int32 (out, optional: NULL skips it), the exact group partials of the
 *   family that computes Y; ws/ws_bytes: qspec_workspace_bytes(
 *   QSPEC_OP_GEMM_W4A8, M, N, K) bytes (the W4A4 size).  Validation and
 *   errors as for qspec_gemm_w4a4.
 * ------------------------------------------------------------------------- */
qspec_status qspec_quant_act8(const uint16_t* X, int64_t M, int64_t K,
                              int8_t* Xq, float* Xs, qspec_stream stream);
qspec_status qspec_gemm_w4a8(const int8_t* Xq, const float* Xs,
                             const uint8_t* Wq, const uint16_t* Ws,
                             int64_t M, int64_t N, int64_t K, int group,
                             int variant, float* Y, int32_t* P,
                             void* ws, size_t ws_bytes, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_gemm_w4a16 -- the verifier's linear layer (QSpec Abstract:
 * weight-only quantization verifies; tech-dashboard summary, paragraph 2:
 * W4A16 keeps activations at higher precision).  Reading:
 *     Y[m,n] = sum_g float(Ws[n,g]) * sum_{k in g} x[m,k] * q[n,k]
 * with the codes turned into bf16 in registers, bf16 MFMA (or VALU dot
 * products for the GEMV family) accumulating each group in fp32, and the
 * fp16 scale applied in fp32 per group.
 *   X  [M][K] bf16 bits (in);  Wq [Np][K/2], Ws [Np][K/128] (tiled, from
 *   qspec_pack_w4, Np = ceil(N/16)*16);  Y [M][N] fp32 (out).
 *   variant: QSPEC_GEMM_AUTO, _GEMV, _SKINNY, _TILED or _STREAM (M <= 16).
 *   ws/ws_bytes: scratch of qspec_workspace_bytes(QSPEC_OP_GEMM_W4A16,M,N,K),
 *   zero-filled before its first use (read qspec_workspace_bytes).
 * ------------------------------------------------------------------------- */
qspec_status qspec_gemm_w4a16(const uint16_t* X, const uint8_t* Wq,
                              const uint16_t* Ws, int64_t M, int64_t N,
                              int64_t K, int group, int variant, float* Y,
                              void* ws, size_t ws_bytes, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_gemm_w4a16_swiglu -- the verifier's gate|up layer with its SwiGLU
 * in the GEMM's epilogue (one launch instead of the layer and
 * qspec_silu_mul).  The N = 2F rows of the packed buffer are in pair order:
 * in 16-row block b, rows 16b .. 16b+7 are gate rows 8b .. 8b+7 and rows
 * 16b+8 .. 16b+15 the matching up rows.  With Y the SKINNY-family result of
 * qspec_gemm_w4a16 on the same buffer (the same k-split, a function of
 * N and K),
 *     A[m, 8b+i] = bf16(silu(Y[m,16b+i]) * Y[m,16b+8+i]),
 *     silu(g) = g / (1 + exp(-g)), fp64 with one rounding,
 * bitwise what qspec_silu_mul_pairs gives on that Y.
 *   X [M][K] bf16 bits (in); Wq, Ws tiled as for qspec_gemm_w4a16 (pair
 *   order, N % 16 == 0); A [M][N/2] bf16 bits (out, 16-byte aligned).
 *   ws/ws_bytes: as for qspec_gemm_w4a16 (QSPEC_OP_GEMM_W4A16, M, N, K).
 * ------------------------------------------------------------------------- */
qspec_status qspec_gemm_w4a16_swiglu(const uint16_t* X, const uint8_t* Wq,
                                     const uint16_t* Ws, int64_t M, int64_t N,
                                     int64_t K, int group, uint16_t* A,
                                     void* ws, size_t ws_bytes,
                                     qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_gemm_w4a4_swiglu, qspec_gemm_w4a8_swiglu -- the drafters' gate|up
 * layer (QSpec Abstract: W4A4 joint quantization drafts; the W4A8 tier
 * above) with its SwiGLU in the epilogue of the STREAM family (M <= 16).  Rows in pair order as for qspec_gemm_w4a16_swiglu;
 * with Y the STREAM-family result of qspec_gemm_w4a4 (qspec_gemm_w4a8) on the
 * same operands,
 *     A[m, 8b+i] = bf16(silu(Y[m,16b+i]) * Y[m,16b+8+i]),
 * bitwise what qspec_silu_mul_pairs gives on that Y.
 *   Xq, Xs as for qspec_gemm_w4a4 (qspec_gemm_w4a8); Wq, Ws tiled, pair
 *   order, N % 16 == 0; A [M][N/2] bf16 bits (out, 16-byte aligned).  No
 *   workspace.  M > 16 gives QSPEC_ERR_UNSUPPORTED; other validation as for
 *   qspec_gemm_w4a4.
 * ------------------------------------------------------------------------- */
qspec_status qspec_gemm_w4a4_swiglu(const uint8_t* Xq, const float* Xs,
                                    const uint8_t* Wq, const uint16_t* Ws,
                                    int64_t M, int64_t N, int64_t K, int group,
                                    uint16_t* A, qspec_stream stream);
qspec_status qspec_gemm_w4a8_swiglu(const int8_t* Xq, const float* Xs,
                                    const uint8_t* Wq, const uint16_t* Ws,
                                    int64_t M, int64_t N, int64_t K, int group,
                                    uint16_t* A, qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_verify -- accept or reject gamma drafted tokens per sequence.
 * Greedy (mode 0; SpecQuant review, method paragraph: a full match is
 * accepted and the first mismatch is rewritten by the parent):
 *     t_i = argmax_v target[b,i,v] (lowest index on ties), i = 0..gamma;
 *     n = first i < gamma with draft[b,i] != t_i, else gamma;
 *     out = draft[b,0..n-1], t_n, then -1.
 * Sampling at temperature 1 (mode 1; tech-dashboard summary, paragraph 3:
 * the output distribution equals the target's -- the rule of the
 * speculative-sampling papers QSpec builds on):
 *     p_i = softmax(target[b,i]), q_i = softmax(draft_logits[b,i]);
 *     accept draft d_i iff u_accept[b,i] <= p_i(d_i) / q_i(d_i)
 *     (q_i(d_i) == 0: accept iff p_i(d_i) > 0);
 *     first reject at n: r = max(0, p_n - q_n) (r = p_n if that sums to 0);
 *     all accepted: n = gamma, r = p_gamma;
 *     emitted = smallest j with cumsum(r)_j > u_sample[b] * sum(r)
 *     (if none: the last j with r_j > 0).
 *   draft_tok     [B][gamma] int32 in [0, V)   (in)
 *   draft_logits  [B][gamma][V] fp32   (in; NULL iff greedy)
 *   target_logits [B][gamma+1][V] fp32 (in)
 *   u_accept      [B][gamma] fp32 in [0,1) (in; NULL iff greedy)
 *   u_sample      [B] fp32 in [0,1)        (in; NULL iff greedy)
 *   n_accept      [B] int32 (out);  out_tok [B][gamma+1] int32 (out, -1 pad)
 *   1 <= gamma <= QSPEC_MAX_GAMMA, B >= 1, 1 <= V <= 2^23,
 *   B * (2 gamma + 1) <= 65535.  Out-of-range draft
 *   tokens are not supported (they are clamped into [0, V) on the device).
 *   ws/ws_bytes: scratch of qspec_workspace_bytes(QSPEC_OP_VERIFY,B,gamma,V).
 * Decisions are taken in fp32; they can differ from exact arithmetic only
 * where p/q or the sampling threshold sits within about 1e-6 (relative) of
 * the decision boundary.
 * ------------------------------------------------------------------------- */
qspec_status qspec_verify(int mode, int64_t B, int gamma, int64_t V,
                          const int32_t* draft_tok, const float* draft_logits,
                          const float* target_logits, const float* u_accept,
                          const float* u_sample, int32_t* n_accept,
                          int32_t* out_tok, void* ws, size_t ws_bytes,
                          qspec_stream stream);

/* ---------------------------------------------------------------------------
 * qspec_verify_noalloc -- qspec_verify without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * modes, validation and results as qspec_verify (bitwise); the scratch the
 * verify kernels need lives in a fixed array of QSPEC_VERIFY_NOALLOC_SCRATCH
 * bytes per device, part of the library's code object and held until the
 * process ends.  Sizes whose qspec_workspace_bytes(QSPEC_OP_VERIFY, B, gamma,
 * V) exceeds it are rejected with QSPEC_ERR_WORKSPACE before anything is
 * enqueued (B = 256, gamma = 8, V = 152064 needs about 2.5 MiB).  Nothing is
 * allocated: no hipMalloc, no hipFree.  Every call on one device shares that
 * device's array and leaves its contents behind (no call depends on them);
 * calls that overlap in time on one device -- on different streams, or from
 * different threads -- race on the array and must be serialised by the
 * caller.
 * ------------------------------------------------------------------------- */
#define QSPEC_VERIFY_NOALLOC_SCRATCH (8u << 20)
qspec_status qspec_verify_noalloc(int mode, int64_t B, int gamma, int64_t V,
                                  const int32_t* draft_tok, const float* draft_logits,
                                  const float* target_logits, const float* u_accept,
                                  const float* u_sample, int32_t* n_accept,
                                  int32_t* out_tok, qspec_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QSPEC_H_ */
