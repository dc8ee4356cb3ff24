// Weight packer and per-token activation quantizer.
//
// Both follow one reading of the pages ("QSpec: Speculative Decoding with
// Complementary Quantization Schemes", Abstract (arXiv); tech-dashboard QSpec
// summary, paragraphs 2 and 4), which print no formula: symmetric INT4 with
// scale = absmax / 7 (IEEE fp32 divide; rounded to fp16 for weights, kept in
// fp32 for activations), code = clamp(rne(v / scale), -8, 7) with an IEEE
// fp32 divide, two's-complement nibbles with element 2i in the low nibble.
// The library is compiled with correctly rounded fp32 division and IEEE
// denormals, so these kernels take every rounding decision exactly as stated.
#include "launch.h"

namespace qspec {
namespace {

__device__ __forceinline__ int quant_code(float v, float s) {
  // s > 0 here; IEEE divide, round half to even, clamp
  const float r = __builtin_rintf(v / s);
  return (int)fminf(fmaxf(r, -8.0f), 7.0f);
}

// One wavefront per (row n, group g) of the row-padded matrix: lane l owns
// k = 2l, 2l+1 of the group, i.e. byte l of the group's 64 row-major bytes,
// and writes it to its place in the tiled storage order: 1 KiB tile per
// (16-row block, group); inside it, 16-byte slot 16*(l/16) + n%16 holds row n's
// bytes [16*(l/16), +16) of the group.  The scale goes to element n%16 of the
// (block, group) 32-byte scale tile.  Padding rows (n >= N) get zero codes
// and zero scales.
__global__ __launch_bounds__(256) void pack_w4_kernel(const float* __restrict__ W, int64_t N,
                                                      int64_t Np, int64_t K,
                                                      uint8_t* __restrict__ Wq,
                                                      uint16_t* __restrict__ Ws) {
  const int64_t G = K / kGroup;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= Np * G) return;  // uniform per wavefront
  const int lane = threadIdx.x & 63;
  const int64_t n = item / G, g = item - (item / G) * G;
  uint8_t byte = 0;
  if (n < N) {  // uniform per wavefront
    const float2 w = *reinterpret_cast<const float2*>(W + n * K + g * kGroup + 2 * lane);
    const float a = wave_max(fmaxf(fabsf(w.x), fabsf(w.y)));
    const _Float16 sh = (_Float16)(a / 7.0f);
    const float s = (float)sh;
    int q0 = 0, q1 = 0;
    if (s != 0.0f) {
      q0 = quant_code(w.x, s);
      q1 = quant_code(w.y, s);
    }
    byte = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    if (lane == 0) Ws[((n >> 4) * G + g) * 16 + (n & 15)] = __builtin_bit_cast(uint16_t, sh);
  } else if (lane == 0) {
    Ws[((n >> 4) * G + g) * 16 + (n & 15)] = 0;  // padding row
  }
  const int64_t tile = (n >> 4) * G + g;
  const int slot = (lane >> 4) * 16 + (int)(n & 15);
  Wq[(tile * 64 + slot) * 16 + (lane & 15)] = byte;
}

__device__ __forceinline__ float absmax8(uint4 v) {
  // |bf16| via the sign bit; the max of exact values is exact
  const float a = fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                        fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  const float b = fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                        fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return fmaxf(a, b);
}

// The code of v at the activation scale s = absmax / 7 (s > 0), with r the
// IEEE reciprocal of s.  |v / s| <= 7 (about), so v * r is within 2^-20 of
// the exact quotient and within 2^-19 of the IEEE quotient v / s; wherever
// v * r lies farther than 2^-19 from a half-integer both round to the same
// integer.  Nearer (or NaN, or an infinite r) the IEEE quotient decides, so
// every code equals rne(v / s) clamped, as the divide would give it.
__device__ __forceinline__ int quant_code_act(float v, float s, float r) {
  const float qa = v * r;
  float k = __builtin_rintf(qa);
  if (!(fabsf(qa - k) < 0.5f - 0x1p-19f)) k = __builtin_rintf(v / s);
  return (int)fminf(fmaxf(k, -8.0f), 7.0f);
}

__device__ __forceinline__ uint32_t pack8(uint4 v, float s, float r) {
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)(quant_code_act(x[i], s, r) & 0xF) << (4 * i);
  return word;
}

// One NT-thread block per token row.  The row is read once into registers
// (NC 16-byte chunks per thread), reduced to its absmax, then coded.
template <int NT, int NC>
__global__ __launch_bounds__(NT) void quant_act_kernel(const uint16_t* __restrict__ X,
                                                       int64_t K, uint8_t* __restrict__ Xq,
                                                       float* __restrict__ Xs) {
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  const int64_t m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(X + m * K);
  const int nch = (int)(K / 8);
  uint4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + NT * i;
    v[i] = c < nch ? row[c] : make_uint4(0, 0, 0, 0);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) a = fmaxf(a, absmax8(v[i]));
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) a = fmaxf(a, red[w]);
  const float s = a / 7.0f;
  const float r = 1.0f / s;
  uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * (K / 2));
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + NT * i;
    if (c < nch) out[c] = s != 0.0f ? pack8(v[i], s, r) : 0u;
  }
  if (threadIdx.x == 0) Xs[m] = s;
}

// rows longer than 1024 * 8 * 8 = 65536 values: two passes (the second hits L2)
__global__ __launch_bounds__(256) void quant_act_long_kernel(const uint16_t* __restrict__ X,
                                                             int64_t K, uint8_t* __restrict__ Xq,
                                                             float* __restrict__ Xs) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(X + m * K);
  const int64_t nch = K / 8;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) a = fmaxf(a, absmax8(row[c]));
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = a / 7.0f;
  const float r = 1.0f / s;
  uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * (K / 2));
  for (int64_t c = threadIdx.x; c < nch; c += 256) out[c] = s != 0.0f ? pack8(row[c], s, r) : 0u;
  if (threadIdx.x == 0) Xs[m] = s;
}

}  // namespace

hipError_t launch_pack_w4(const float* W, int64_t N, int64_t K, uint8_t* Wq, uint16_t* Ws,
                          hipStream_t s) {
  const int64_t Np = cdiv(N, 16) * 16;
  const int64_t items = Np * (K / kGroup);
  hipLaunchKernelGGL(pack_w4_kernel, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, s, W, N, Np, K,
                     Wq, Ws);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                            hipStream_t s) {
  // one block per row, sized so each thread holds at most a few chunks: the
  // short latency chain (load, block max, code) is what a decode row costs
  const int64_t nch = K / 8;  // 16-byte chunks of a row
  const dim3 g((unsigned)M);
  if (nch <= 512) {
    hipLaunchKernelGGL((quant_act_kernel<256, 2>), g, dim3(256), 0, s, X, K, Xq, Xs);
  } else if (nch <= 2048) {
    hipLaunchKernelGGL((quant_act_kernel<1024, 2>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else if (nch <= 4096) {
    hipLaunchKernelGGL((quant_act_kernel<1024, 4>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else if (nch <= 8192) {
    hipLaunchKernelGGL((quant_act_kernel<1024, 8>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else {
    hipLaunchKernelGGL(quant_act_long_kernel, g, dim3(256), 0, s, X, K, Xq, Xs);
  }
  return hipGetLastError();
}

}  // namespace qspec
