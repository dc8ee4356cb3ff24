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

// eight fp32 values -> their eight codes, code i in bits 4i .. 4i + 3
__device__ __forceinline__ uint32_t pack8f(const float x[8], float s, float r) {
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)(quant_code_act(x[i], s, r) & 0xF) << (4 * i);
  return word;
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float x[8]) {
  x[0] = bf16_lo(v.x);
  x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y);
  x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z);
  x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w);
  x[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint32_t pack8(uint4 v, float s, float r) {
  float x[8];
  bf16x8_to_f32(v, x);
  return pack8f(x, s, r);
}

// The 8-bit code of v at s = absmax / 127 (s > 0), r = 1 / s: here

// eight bf16 values -> their eight 8-bit codes, code i in byte i
__device__ __forceinline__ uint2 pack8_i8(uint4 v, float s, float r) {
  float x[8];
  bf16x8_to_f32(v, x);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)(quant_code_act8(x[i], s, r) & 0xFF) << (8 * (i & 3));
  return make_uint2(w[0], w[1]);
}

// ------------------------------------------------------------------ rotation
// Walsh-Hadamard transform of one 128-value group (Sylvester order), held by
// 16 consecutive lanes with 8 consecutive values each: stages 0-2 inside the
// lane, stages 3-6 across the 16 lanes.  At stage s the pair of positions
// (i, i + 2^s) with bit s of i clear becomes (a + b, a - b), one fp32 add or
// subtract each, so every value is fixed whatever the launch shape.  All 16
// lanes of a group must execute it together.
__device__ __forceinline__ void fwht128_lane(float f[8], int l16) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!(e & h)) {
        const float a = f[e], b = f[e | h];
        f[e] = a + b;
        f[e | h] = a - b;
      }
  // partner lane = lane ^ m: ds_swizzle in bit-mask mode (and 0x1F, xor m)
#define QSPEC_FWHT_XSTAGE(m)                                                              \
  _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                         \
    const float u = __int_as_float(                                                       \
        __builtin_amdgcn_ds_swizzle(__float_as_int(f[e]), 0x1F | ((m) << 10)));           \
    f[e] = (l16 & (m)) ? u - f[e] : f[e] + u; /* bit set: a = partner, b = mine */       \
  }
  QSPEC_FWHT_XSTAGE(1)
  QSPEC_FWHT_XSTAGE(2)
  QSPEC_FWHT_XSTAGE(4)
  QSPEC_FWHT_XSTAGE(8)
#undef QSPEC_FWHT_XSTAGE
}

// x' = H x * scale per 128-group of each row (scale a power of two: exact).
// One 16-lane team per (row, group); BF16: bf16 in and out (rounded to
// nearest even), else fp32.  A team reads its group before it writes it, so
// out may equal in.
template <bool BF16>
__global__ __launch_bounds__(256) void rotate_kernel(const void* in, void* out, int64_t R,
                                                     int64_t K, float scale) {
  const int64_t G = K / kGroup;
  const int64_t team = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  const bool ok = team < R * G;  // uniform over the team
  const int64_t off = ok ? (team / G) * K + (team % G) * kGroup + l16 * 8 : 0;
  float f[8];
  if (BF16) {
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + off)
                       : make_uint4(0, 0, 0, 0);
    bf16x8_to_f32(v, f);
  } else {
    const float* p = static_cast<const float*>(in) + off;
    const float4 a = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 b = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  fwht128_lane(f, l16);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] *= scale;
  if (!ok) return;
  if (BF16) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)f32_to_bf16_rne(f[2 * j]) | ((uint32_t)f32_to_bf16_rne(f[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float* p = static_cast<float*>(out) + off;
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
}

// The quantizer on the rotated row x' = H x / 16 (fp32, not rounded to bf16):
// one NT-thread block per row, NC chunks of 8 values per thread (chunk c =
// tid + NT i, so the 16 chunks of a group sit in 16 consecutive lanes), every
// thread looping the same number of times.
template <int NT, int NC>
__global__ __launch_bounds__(NT) void quant_act_rot_kernel(const uint16_t* __restrict__ X,
                                                           int64_t K, uint8_t* __restrict__ Xq,
                                                           float* __restrict__ Xs) {
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  const int64_t m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(X + m * K);
  const int nch = (int)(K / 8);
  const int l16 = threadIdx.x & 15;
  float f[NC][8];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + NT * i;
    bf16x8_to_f32(c < nch ? row[c] : make_uint4(0, 0, 0, 0), f[i]);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    fwht128_lane(f[i], l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[i][e] *= 0.0625f;
      a = fmaxf(a, fabsf(f[i][e]));
    }
  }
  a = wave_max_dpp(a);
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
    if (c < nch) out[c] = s != 0.0f ? pack8f(f[i], s, r) : 0u;
  }
  if (threadIdx.x == 0) Xs[m] = s;
}

// rows longer than 1024 * 8 * 8 values: two passes, the second recomputes
// the rotation (same operations, same values) from L2
__global__ __launch_bounds__(256) void quant_act_rot_long_kernel(const uint16_t* __restrict__ X,
                                                                 int64_t K, uint8_t* __restrict__ Xq,
                                                                 float* __restrict__ Xs) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(X + m * K);
  const int64_t nch = K / 8;
  const int l16 = threadIdx.x & 15;
  float a = 0.0f;
  for (int64_t c0 = 0; c0 < nch; c0 += 256) {  // uniform trip count
    const int64_t c = c0 + threadIdx.x;
    float f[8];
    bf16x8_to_f32(c < nch ? row[c] : make_uint4(0, 0, 0, 0), f);
    fwht128_lane(f, l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e] * 0.0625f));
  }
  a = wave_max_dpp(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = a / 7.0f;
  const float r = 1.0f / s;
  uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * (K / 2));
  for (int64_t c0 = 0; c0 < nch; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    float f[8];
    bf16x8_to_f32(c < nch ? row[c] : make_uint4(0, 0, 0, 0), f);
    fwht128_lane(f, l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= 0.0625f;
    if (c < nch) out[c] = s != 0.0f ? pack8f(f, s, r) : 0u;
  }
  if (threadIdx.x == 0) Xs[m] = s;
}

// One NT-thread block per token row.  The row is read once into registers
// (NC 16-byte chunks per thread), reduced to its absmax, then coded.
template <int NT, int NC, int BITS>
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
  // the row max over DPP lane moves (a maximum is the same in any order)
  a = wave_max_dpp(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) a = fmaxf(a, red[w]);
  const float s = a / (BITS == 4 ? 7.0f : 127.0f);
  const float r = 1.0f / s;
  if (BITS == 4) {
    uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * (K / 2));
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < nch) out[c] = s != 0.0f ? pack8(v[i], s, r) : 0u;
    }
  } else {
    uint2* out = reinterpret_cast<uint2*>(Xq + m * K);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < nch) out[c] = s != 0.0f ? pack8_i8(v[i], s, r) : make_uint2(0u, 0u);
    }
  }
  if (threadIdx.x == 0) Xs[m] = s;
}

// rows longer than 1024 * 8 * 8 = 65536 values: two passes (the second hits L2)
template <int BITS>
__global__ __launch_bounds__(256) void quant_act_long_kernel(const uint16_t* __restrict__ X,
                                                             int64_t K, uint8_t* __restrict__ Xq,
                                                             float* __restrict__ Xs) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(X + m * K);
  const int64_t nch = K / 8;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) a = fmaxf(a, absmax8(row[c]));
  a = wave_max_dpp(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = a / (BITS == 4 ? 7.0f : 127.0f);
  const float r = 1.0f / s;
  if (BITS == 4) {
    uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * (K / 2));
    for (int64_t c = threadIdx.x; c < nch; c += 256) out[c] = s != 0.0f ? pack8(row[c], s, r) : 0u;
  } else {
    uint2* out = reinterpret_cast<uint2*>(Xq + m * K);
    for (int64_t c = threadIdx.x; c < nch; c += 256)
      out[c] = s != 0.0f ? pack8_i8(row[c], s, r) : make_uint2(0u, 0u);
  }
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

// launch shape of the short-row band (threads x 16-byte chunks per thread,
// at least 512 chunks) and the threads of the <= 4096-chunk band
#ifndef QSPEC_QA_SNT
#define QSPEC_QA_SNT 256
#endif
#ifndef QSPEC_QA_SNC
#define QSPEC_QA_SNC 2
#endif
#ifndef QSPEC_QA_MNT
#define QSPEC_QA_MNT 1024
#endif
template <int BITS>
hipError_t launch_quant_act_bits(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                                 hipStream_t s) {
  // one block per row, sized so each thread holds at most a few chunks: the
  // short latency chain (load, block max, code) is what a decode row costs
  const int64_t nch = K / 8;  // 16-byte chunks of a row
  const dim3 g((unsigned)M);
  if (nch <= QSPEC_QA_SNT * QSPEC_QA_SNC) {
    hipLaunchKernelGGL((quant_act_kernel<QSPEC_QA_SNT, QSPEC_QA_SNC, BITS>), g, dim3(QSPEC_QA_SNT), 0,
                       s, X, K, Xq, Xs);
  } else if (nch <= 2048) {
    hipLaunchKernelGGL((quant_act_kernel<1024, 2, BITS>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else if (nch <= 4096) {
    hipLaunchKernelGGL((quant_act_kernel<QSPEC_QA_MNT, 4096 / QSPEC_QA_MNT, BITS>), g,
                       dim3(QSPEC_QA_MNT), 0, s, X, K, Xq, Xs);
  } else if (nch <= 8192) {
    hipLaunchKernelGGL((quant_act_kernel<1024, 8, BITS>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else {
    hipLaunchKernelGGL(quant_act_long_kernel<BITS>, g, dim3(256), 0, s, X, K, Xq, Xs);
  }
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                            hipStream_t s) {
  return launch_quant_act_bits<4>(X, M, K, Xq, Xs, s);
}

hipError_t launch_quant_act8(const uint16_t* X, int64_t M, int64_t K, int8_t* Xq, float* Xs,
                             hipStream_t s) {
  return launch_quant_act_bits<8>(X, M, K, reinterpret_cast<uint8_t*>(Xq), Xs, s);
}

hipError_t launch_rotate(bool bf16, const void* in, int64_t R, int64_t K, float scale, void* out,
                         hipStream_t s) {
  const int64_t teams = R * (K / kGroup);
  const dim3 grid((unsigned)cdiv(teams, 16)), block(256);
  if (bf16)
    hipLaunchKernelGGL(rotate_kernel<true>, grid, block, 0, s, in, out, R, K, scale);
  else
    hipLaunchKernelGGL(rotate_kernel<false>, grid, block, 0, s, in, out, R, K, scale);
  return hipGetLastError();
}

hipError_t launch_quant_act_rot(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                                hipStream_t s) {
  const int64_t nch = K / 8;
  const dim3 g((unsigned)M);
  if (nch <= 512) {
    hipLaunchKernelGGL((quant_act_rot_kernel<256, 2>), g, dim3(256), 0, s, X, K, Xq, Xs);
  } else if (nch <= 2048) {
    hipLaunchKernelGGL((quant_act_rot_kernel<1024, 2>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else if (nch <= 4096) {
    hipLaunchKernelGGL((quant_act_rot_kernel<1024, 4>), g, dim3(1024), 0, s, X, K, Xq, Xs);
  } else {
    hipLaunchKernelGGL(quant_act_rot_long_kernel, g, dim3(256), 0, s, X, K, Xq, Xs);
  }
  return hipGetLastError();
}

}  // namespace qspec
