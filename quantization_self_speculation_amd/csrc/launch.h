// Internal launcher interface between the C-ABI layer (capi.cpp) and the HIP
// kernels.  Every launcher assumes its arguments were validated by the C-ABI
// layer and only enqueues work on `s`.
#pragma once

#include "common.h"

namespace qspec {

hipError_t launch_pack_w4(const float* W, int64_t N, int64_t K, uint8_t* Wq, uint16_t* Ws,
                          hipStream_t s);
hipError_t launch_quant_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                            hipStream_t s);

// per-group Walsh-Hadamard rotation: x' = H x * scale per 128-group of each
// of R rows (bf16 in and out, or fp32 in and out); the quantizer on the
// rotated row x' = H x / 16
hipError_t launch_rotate(bool bf16, const void* in, int64_t R, int64_t K, float scale, void* out,
                         hipStream_t s);
hipError_t launch_quant_act_rot(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                                hipStream_t s);

hipError_t launch_quant_act8(const uint16_t* X, int64_t M, int64_t K, int8_t* Xq, float* Xs,
                             hipStream_t s);

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                        int64_t N, int64_t K, int variant, float* Y, void* ws, size_t ws_bytes,
                        hipStream_t s);
// the W4A16 gate|up layer in the SKINNY family with its SwiGLU in the
// epilogue: rows of Wq/Ws in pair order, A bf16 [M][N/2]
hipError_t launch_w4a16_swiglu(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                               int64_t N, int64_t K, uint16_t* A, void* ws, size_t ws_bytes,
                               hipStream_t s);

// the drafters' gate|up layer (STREAM family, M <= 16) with its SwiGLU in
// the epilogue: rows in pair order, A bf16 [M][N/2]
hipError_t launch_w4a4_swiglu(const uint8_t* Xq, const float* Xs, const uint8_t* Wq,
                              const uint16_t* Ws, int64_t M, int64_t N, int64_t K, uint16_t* A,
                              hipStream_t s);
hipError_t launch_w4a8_swiglu(const int8_t* Xq, const float* Xs, const uint8_t* Wq,
                              const uint16_t* Ws, int64_t M, int64_t N, int64_t K, uint16_t* A,
                              hipStream_t s);

// the family a GEMM call runs (AUTO resolved; M, N, K only)
int w4a16_pick(int variant, int64_t M, int64_t N, int64_t K);
int w4a4_pick(int variant, int64_t M, int64_t N, int64_t K);
int w4a8_pick(int variant, int64_t M, int64_t N, int64_t K);

size_t w4a4_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a4(const uint8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, uint16_t* Yb,
                       int32_t* P, void* ws, size_t ws_bytes, hipStream_t s);

hipError_t launch_w4a8(const int8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, int32_t* P,
                       void* ws, size_t ws_bytes, hipStream_t s);

size_t verify_ws_bytes(int64_t B, int gamma, int64_t V);
// the fixed per-device scratch of the allocation-free verify entry point
constexpr size_t kVerifyScratchBytes = (size_t)QSPEC_VERIFY_NOALLOC_SCRATCH;
hipError_t launch_verify_noalloc(int mode, int64_t B, int gamma, int64_t V,
                                 const int32_t* draft_tok, const float* draft_logits,
                                 const float* target_logits, const float* u_accept,
                                 const float* u_sample, int32_t* n_accept, int32_t* out_tok,
                                 hipStream_t s);
hipError_t launch_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                         const float* draft_logits, const float* target_logits,
                         const float* u_accept, const float* u_sample, int32_t* n_accept,
                         int32_t* out_tok, void* ws, hipStream_t s);

// ceiling probes (probe.hip)
hipError_t launch_probe_read(const void* buf, int64_t bytes, int blocks, int unroll,
                             uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_probe_empty(hipStream_t s);

// decoder kernels of the end-to-end loop (harness.hip)
constexpr int kHarnessHeadDim = 128;
constexpr int64_t kHarnessMaxCap = 3968;  // positions per sequence in a KV cache (the API limit)
constexpr int64_t kHarnessMaxD = 4096;
hipError_t launch_embed(const uint16_t* emb, int64_t V, int64_t d, const int32_t* tok, int64_t M,
                        float* x, hipStream_t s);
hipError_t launch_add_rmsnorm(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                              int64_t d, double eps, uint16_t* y, hipStream_t s);
hipError_t launch_rope_kv(const float* qkv, int64_t M, int H, int Hkv, int hd, const int32_t* seq,
                          const int32_t* pos, double base, float* q, uint16_t* kc, uint16_t* vc,
                          int64_t B, int64_t cap, hipStream_t s);
hipError_t launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t M,
                            int H, int Hkv, const int32_t* seq, const int32_t* pos, int64_t B,
                            int64_t cap, uint16_t* out, hipStream_t s);
hipError_t launch_rope_attention(const float* qkv, int64_t M, int H, int Hkv, const int32_t* seq,
                                 const int32_t* pos, double base, float* q, uint16_t* kc,
                                 uint16_t* vc, int64_t B, int64_t cap, uint16_t* out,
                                 hipStream_t s);
hipError_t launch_silu_mul(const float* gu, int64_t M, int64_t F, uint16_t* a, hipStream_t s);
hipError_t launch_silu_mul_pairs(const float* gu, int64_t M, int64_t F, uint16_t* a,
                                 hipStream_t s);
hipError_t launch_add_rmsnorm_quant(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                                    int64_t d, double eps, uint16_t* y, uint8_t* yq, float* ys,
                                    hipStream_t s);
hipError_t launch_add_rmsnorm_quant8(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                                     int64_t d, double eps, uint16_t* y, int8_t* yq, float* ys,
                                     hipStream_t s);
hipError_t launch_argmax(const float* x, int64_t M, int64_t V, int32_t* out, int64_t stride,
                         hipStream_t s);
hipError_t launch_spec_prepare(int phase, int64_t B, int gamma, int j, const int32_t* len,
                               const int32_t* vtok, int32_t* drafts, int32_t* seq, int32_t* pos,
                               int32_t* tok, hipStream_t s);
hipError_t launch_spec_commit(int64_t B, int gamma, const int32_t* n_accept, const int32_t* out_tok,
                              int32_t* len, int32_t* vtok, int64_t vstride, int32_t* gen,
                              int64_t gen_cap, int32_t* n_gen, int max_gen, int64_t* stats,
                              hipStream_t s);

}  // namespace qspec
