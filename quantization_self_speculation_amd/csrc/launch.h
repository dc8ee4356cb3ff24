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

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                        int64_t N, int64_t K, int variant, float* Y, void* ws, hipStream_t s);

size_t w4a4_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a4(const uint8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, int32_t* P,
                       void* ws, hipStream_t s);

size_t verify_ws_bytes(int64_t B, int gamma, int64_t V);
hipError_t launch_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                         const float* draft_logits, const float* target_logits,
                         const float* u_accept, const float* u_sample, int32_t* n_accept,
                         int32_t* out_tok, void* ws, hipStream_t s);

}  // namespace qspec
