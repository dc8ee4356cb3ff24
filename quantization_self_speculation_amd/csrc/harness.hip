// Decoder kernels around the dual-mode linear layers, for the end-to-end
// self-speculative loop: embedding gather, residual add + RMSNorm to bf16,
// RoPE + KV-cache write, causal grouped-query attention, SiLU * up, row
// argmax, and the device-side bookkeeping of a speculation round.
//
// Every kernel computes each row on its own with a fixed operation order, so
// a row's result does not depend on how many rows share the launch -- the
// property that lets a verify pass over gamma+1 positions reproduce, bit for
// bit, what pure decoding computes one position at a time.
//
// Rounding points: residual fp32; normalised activations, attention output
// and silu * up are bf16 (GEMM inputs); keys after RoPE and values are bf16
// in the cache; queries after RoPE are fp32.  Values headed for bf16 are
// computed in fp64 and rounded once (round to odd into fp32, then to nearest
// even into bf16, which equals a single rounding from fp64).
#include "launch.h"

namespace qspec {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
__device__ __forceinline__ T block_sum_256(T v, T* red) {
  // 256 threads: wave sums, then one wave over the four partials
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  T s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// ------------------------------------------------------------------ embedding
// x[m][:] = float(emb[tok[m]][:]); d % 8 == 0; ids outside [0, V) are clamped
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* __restrict__ emb, int64_t V,
                                                    int64_t d, const int32_t* __restrict__ tok,
                                                    float* __restrict__ x) {
  const int64_t m = blockIdx.x;
  const int64_t id = min(max((int64_t)tok[m], (int64_t)0), V - 1);  // out-of-range ids clamp
  const uint16_t* src = emb + id * d;
  float* dst = x + m * d;
  for (int64_t j = (int64_t)threadIdx.x * 8; j < d; j += 256 * 8) {
    const uint4 p = *reinterpret_cast<const uint4*>(src + j);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[j + 2 * i] = __uint_as_float(w[i] << 16);
      dst[j + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

// ------------------------------------------------------------------ add + RMSNorm
// x[m] (row stride xs) += add[m] (row stride as; if add), stored back in fp32; then
// y[m] = bf16(x / sqrt(mean(x^2) + eps)) in fp64.  One 256-thread block per
// row; each thread keeps up to kNormPer elements.
constexpr int kNormPer = 16;  // d <= 4096

// The drafter's per-token 4-bit codes of a row that a block has just
// produced as bf16 (thread t holds elements t + 256 i): the row's absmax, the
// scale s = absmax / 7 and each code exactly as the stand-alone quantizer
// takes them, so the codes equal that quantizer's on the stored bf16 row.
// The even thread of each pair packs its element's code (low nibble) with
// its neighbour's (high nibble).
// BITS = 8: the W4A8 drafter's codes instead (absmax / 127, one byte per
// element, as the stand-alone 8-bit quantizer takes them).
template <int PER, int BITS>
__device__ __forceinline__ void quant_row_bf16(const uint16_t (&yb)[PER], int n, float* red,
                                               uint8_t* __restrict__ q, float* __restrict__ qs) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if ((int)threadIdx.x + 256 * i < n) a = fmaxf(a, fabsf(__uint_as_float((uint32_t)yb[i] << 16)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  __syncthreads();  // red may still be read by an earlier reduction
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = a / (BITS == 4 ? 7.0f : 127.0f);
  const float r = 1.0f / s;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x + 256 * i;
    const float v = __uint_as_float((uint32_t)yb[i] << 16);
    if (BITS == 8) {
      if (j < n) q[j] = (uint8_t)(s != 0.0f ? quant_code_act8(v, s, r) : 0);
      continue;
    }
    const int c = (j < n && s != 0.0f) ? quant_code_act(v, s, r) : 0;
    const int nb = __shfl_xor(c, 1, 64);
    if (!(threadIdx.x & 1) && j < n) q[j >> 1] = (uint8_t)((c & 0xF) | ((nb & 0xF) << 4));
  }
  if (threadIdx.x == 0) *qs = s;
}

template <int BITS>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float* __restrict__ x, int64_t xs,
                                                          const float* __restrict__ add, int64_t as,
                                                          int d, double eps,
                                                          uint16_t* __restrict__ y,
                                                          uint8_t* __restrict__ yq,
                                                          float* __restrict__ ys) {
  __shared__ double red[4];
  __shared__ float redf[4];
  const int64_t m = blockIdx.x;
  float* xr = x + m * xs;
  float v[kNormPer];
  double ss = 0.0;
  // all loads first (independent), then the residual update and the sum
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int j = threadIdx.x + 256 * i;
    v[i] = j < d ? xr[j] : 0.f;
  }
  if (add != nullptr) {
    float ad[kNormPer];
#pragma unroll
    for (int i = 0; i < kNormPer; ++i) {
      const int j = threadIdx.x + 256 * i;
      ad[i] = j < d ? add[m * as + j] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kNormPer; ++i) {
      const int j = threadIdx.x + 256 * i;
      v[i] = v[i] + ad[i];
      if (j < d) xr[j] = v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) ss += (double)v[i] * (double)v[i];
  ss = block_sum_256(ss, red);
  const double den = sqrt(ss / (double)d + eps);
  uint16_t* yr = y + m * d;
  uint16_t yb[kNormPer];
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int j = threadIdx.x + 256 * i;
    yb[i] = f64_to_bf16_rne((double)v[i] / den);
    if (j < d) yr[j] = yb[i];
  }
  if (yq != nullptr)  // uniform
    quant_row_bf16<kNormPer, BITS>(yb, d, redf, yq + m * (BITS == 4 ? d / 2 : d), ys + m);
}

// The same add + RMSNorm (+ codes) for 16-byte aligned rows with d % 4 == 0:
// thread t owns the four consecutive elements of each float4 t + NT i, so
// every access is one 16-byte (x, add), 8-byte (y) or 2-byte (codes) vector
// per group, and a group's two code bytes are packed in-thread.  The
// reductions run over DPP lane moves within each 16-lane row, the four row
// values of a wavefront read in a fixed order, then the wavefronts' values
// through LDS in wave order: one barrier per reduction, no LDS round trip
// inside a wavefront.  The sum of squares is fp64 in a fixed order (a
// different order from add_rmsnorm_kernel's: the two kernels may differ in
// the last bit of den, never a row from another launch of the same kernel);
// the absmax is order-free, so the codes are exactly the stand-alone
// quantizer's on the stored bf16 row.
#ifndef QSPEC_NORM_THREADS
#define QSPEC_NORM_THREADS 512
#endif
constexpr int kNormThreads = QSPEC_NORM_THREADS;
constexpr int kNormV4 = 4096 / (4 * kNormThreads);  // float4 groups per thread (d <= 4096)

template <int BITS>
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_v4_kernel(
    float* __restrict__ x, int64_t xs, const float* __restrict__ add, int64_t as, int d, double eps,
    uint16_t* __restrict__ y, uint8_t* __restrict__ yq, float* __restrict__ ys) {
  constexpr int NW = kNormThreads / 64;
  __shared__ double red[NW];
  __shared__ float redf[NW];
  const int64_t m = blockIdx.x;
  const int w = threadIdx.x >> 6;
  float4* xr = reinterpret_cast<float4*>(x + m * xs);
  const int ng = d / 4;
  float4 v[kNormV4];
#pragma unroll
  for (int i = 0; i < kNormV4; ++i) {
    const int gi = (int)threadIdx.x + kNormThreads * i;
    v[i] = gi < ng ? xr[gi] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (add != nullptr) {
    const float4* ar = reinterpret_cast<const float4*>(add + m * as);
    float4 ad[kNormV4];
#pragma unroll
    for (int i = 0; i < kNormV4; ++i) {
      const int gi = (int)threadIdx.x + kNormThreads * i;
      ad[i] = gi < ng ? ar[gi] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kNormV4; ++i) {
      const int gi = (int)threadIdx.x + kNormThreads * i;
      v[i].x += ad[i].x;
      v[i].y += ad[i].y;
      v[i].z += ad[i].z;
      v[i].w += ad[i].w;
      if (gi < ng) xr[gi] = v[i];
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kNormV4; ++i) {
    ss += (double)v[i].x * (double)v[i].x;
    ss += (double)v[i].y * (double)v[i].y;
    ss += (double)v[i].z * (double)v[i].z;
    ss += (double)v[i].w * (double)v[i].w;
  }
  ss = wave_sum_f64_dpp(ss);
  if ((threadIdx.x & 63) == 0) red[w] = ss;
  __syncthreads();
  ss = red[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) ss += red[k];
  const double den = sqrt(ss / (double)d + eps);
  uint2* yr = reinterpret_cast<uint2*>(y + m * d);
  uint16_t yb[kNormV4][4];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < kNormV4; ++i) {
    const int gi = (int)threadIdx.x + kNormThreads * i;
    yb[i][0] = f64_to_bf16_rne((double)v[i].x / den);
    yb[i][1] = f64_to_bf16_rne((double)v[i].y / den);
    yb[i][2] = f64_to_bf16_rne((double)v[i].z / den);
    yb[i][3] = f64_to_bf16_rne((double)v[i].w / den);
    if (gi < ng) {
      yr[gi] = make_uint2((uint32_t)yb[i][0] | ((uint32_t)yb[i][1] << 16),
                          (uint32_t)yb[i][2] | ((uint32_t)yb[i][3] << 16));
#pragma unroll
      for (int c = 0; c < 4; ++c) a = fmaxf(a, fabsf(bf16_to_f32(yb[i][c])));
    }
  }
  if (yq == nullptr) return;  // uniform
  a = wave_max_dpp(a);
  if ((threadIdx.x & 63) == 0) redf[w] = a;
  __syncthreads();
  a = redf[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) a = fmaxf(a, redf[k]);
  const float sc = a / (BITS == 4 ? 7.0f : 127.0f);
  const float r = 1.0f / sc;
  if (BITS == 8) {
    // one byte per element: a thread's four codes are one 4-byte store
    uint32_t* qr = reinterpret_cast<uint32_t*>(yq + m * d);
#pragma unroll
    for (int i = 0; i < kNormV4; ++i) {
      const int gi = (int)threadIdx.x + kNormThreads * i;
      if (gi < ng) {
        uint32_t wv = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wv |= (uint32_t)((sc != 0.0f ? quant_code_act8(bf16_to_f32(yb[i][k]), sc, r) : 0) & 0xFF) << (8 * k);
        qr[gi] = wv;
      }
    }
  } else {
    uint16_t* qr = reinterpret_cast<uint16_t*>(yq + m * (d / 2));
#pragma unroll
    for (int i = 0; i < kNormV4; ++i) {
      const int gi = (int)threadIdx.x + kNormThreads * i;
      if (gi < ng) {
        int c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = sc != 0.0f ? quant_code_act(bf16_to_f32(yb[i][k]), sc, r) : 0;
        qr[gi] = (uint16_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4) | ((c[2] & 0xF) << 8) | ((c[3] & 0xF) << 12));
      }
    }
  }
  if (threadIdx.x == 0) ys[m] = sc;
}

// ------------------------------------------------------------------ RoPE + KV write
// qkv[m] = [q (H*hd) | k (Hkv*hd) | v (Hkv*hd)] fp32.  q -> fp32 after RoPE,
// k -> bf16 after RoPE, v -> bf16, both written at [seq][g][pos][:] of the
// layer's caches.  The pair (i, i + hd/2) turns by pos * base^(-2i/hd); the
// angles, cosines, sines and products are fp64.
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* __restrict__ qkv, int H, int Hkv,
                                                      int hd, const int32_t* __restrict__ seq,
                                                      const int32_t* __restrict__ pos, double base,
                                                      float* __restrict__ q,
                                                      uint16_t* __restrict__ kc,
                                                      uint16_t* __restrict__ vc, int64_t B,
                                                      int64_t cap) {
  __shared__ double cs[2][128];
  const int64_t m = blockIdx.x;
  const int half = hd / 2;
  const int p = pos[m];
  const int64_t b = seq[m];
  if (b < 0 || b >= B || p < 0 || p >= cap) return;  // rows outside the cache write nothing
  if (threadIdx.x < half) {
    const double f = pow(base, -2.0 * (double)threadIdx.x / (double)hd);
    double s, c;
    sincos((double)p * f, &s, &c);
    cs[0][threadIdx.x] = c;
    cs[1][threadIdx.x] = s;
  }
  __syncthreads();
  const int rowlen = (H + 2 * Hkv) * hd;
  const float* r = qkv + m * rowlen;
  // rotated pairs of q and k heads
  const int npairs = (H + Hkv) * half;
  for (int t = threadIdx.x; t < npairs; t += blockDim.x) {
    const int h = t / half, i = t % half;
    const double a = r[h * hd + i], bb = r[h * hd + i + half];
    const double c = cs[0][i], s = cs[1][i];
    const double lo = a * c - bb * s, hi = bb * c + a * s;
    if (h < H) {
      q[m * (H * hd) + h * hd + i] = (float)lo;
      q[m * (H * hd) + h * hd + i + half] = (float)hi;
    } else {
      const int g = h - H;
      uint16_t* dst = kc + ((b * Hkv + g) * cap + p) * hd;
      dst[i] = f64_to_bf16_rne(lo);
      dst[i + half] = f64_to_bf16_rne(hi);
    }
  }
  for (int t = threadIdx.x; t < Hkv * hd; t += blockDim.x) {
    const int g = t / hd, i = t % hd;
    vc[((b * Hkv + g) * cap + p) * hd + i] = f32_to_bf16_rne(r[(H + Hkv) * hd + t]);
  }
}

// ------------------------------------------------------------------ attention
// One block of kAttnWaves wavefronts per (row, kv head, part): the part's
// HPB query heads of the kv head (HPB = 4, 2 or 1, chosen per launch) share
// every key and value load.  The T = pos + 1 keys are split into kAttnWaves
// contiguous ranges (a function of T only); a wavefront walks its range in
// chunks of up to kAttnChunk keys, issuing all of a chunk's key and value
// loads at once, and keeps a running softmax:
//   scores: 16 lanes share a key (lane l reads dims 8 (l % 16) .. + 7 of key
//     4 j + l / 16, one coalesced 16-byte load), each lane's 8 products are
//     summed in order and the 16 partials by fixed DPP lane moves, fp32; the
//     first lane of the 16 keeps the score;
//   per chunk: its max m', the running max m = max(m, m'), the old sums
//     scaled by exp(m_old - m), p = exp(s - m), sum of p in a fixed order,
//     and lane l accumulates p * v for dims 2l, 2l+1 over the chunk's keys
//     in increasing order;
//   the wavefronts' (m, sum, o) are merged in wave order.
// Every step of a head depends on T alone and on no other head, so a row's
// output is the same whatever other rows share the launch and however many
// heads a block serves.  Output bf16.
constexpr int kHeadDim = 128;
// Block shape (measured on MI355X; the key split is part of a row's result,
// so one shape serves every M: 8 wavefronts with 32-key chunks beat 64-key
// chunks at every decode, verify and prefill point -- 192 instead of 256
// registers -- and 4 or 16 wavefronts lose at one end or the other).
#ifndef QSPEC_ATTN_WAVES
#define QSPEC_ATTN_WAVES 8
#endif
#ifndef QSPEC_ATTN_CHUNK
#define QSPEC_ATTN_CHUNK 32
#endif
constexpr int kAttnWaves = QSPEC_ATTN_WAVES;

// Sum over the 16 lanes of a DPP row, by VALU lane moves (no LDS round trip):
// swap neighbours, swap pairs (now every lane holds its quad's sum), then add
// the quads 4 and 8 lanes around the row.  Every lane ends with the row's sum;
// the association differs between quads, so a caller keeps the value of one
// fixed lane (it is then a fixed function of the 16 inputs).
__device__ __forceinline__ float sum16_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row rotate 4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row rotate 8
  return v;
}
constexpr int kAttnChunk = QSPEC_ATTN_CHUNK;  // keys per wavefront chunk (all loads in flight)
constexpr int kAttnQuads = kAttnChunk / 4;

// The block's kv head and first query head (within the kv head's group):
// blockIdx.y = g * parts + part, parts = ceil(grp / HPB).
template <int HPB>
__device__ __forceinline__ void attn_block_heads(int H, int Hkv, int& g, int& h0, int& nh) {
  const int grp = H / Hkv, parts = (grp + HPB - 1) / HPB;
  g = blockIdx.y / parts;
  h0 = (blockIdx.y % parts) * HPB;
  nh = min(HPB, grp - h0);
}

template <int HPB>
__device__ __forceinline__ void attend(const float* __restrict__ q, const uint16_t* __restrict__ kc,
                                       const uint16_t* __restrict__ vc, int H, int Hkv,
                                       const int32_t* __restrict__ seq,
                                       const int32_t* __restrict__ pos, int64_t B, int64_t cap,
                                       uint16_t* __restrict__ out) {
  // LDS: per wavefront, the chunk's scores [HPB][kAttnChunk]; then the
  // wavefronts' results: o [kAttnWaves][HPB][128], m and sum
  // [kAttnWaves][HPB]
  __shared__ float sc[kAttnWaves][HPB][kAttnChunk];
  __shared__ float po[kAttnWaves][HPB][kHeadDim];
  __shared__ float pm[kAttnWaves][HPB], pl[kAttnWaves][HPB];
  const int64_t m = blockIdx.x;
  int g, h0, nh;
  attn_block_heads<HPB>(H, Hkv, g, h0, nh);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = H / Hkv;
  const int64_t b = seq[m];
  // rows outside the cache attend to nothing (output 0)
  const bool ok = b >= 0 && b < B && pos[m] >= 0 && pos[m] < cap;
  const int T = ok ? pos[m] + 1 : 0;
  const int64_t bb = ok ? b : 0;
  const uint16_t* K = kc + (bb * Hkv + g) * cap * kHeadDim;
  const uint32_t* Vw = reinterpret_cast<const uint32_t*>(vc + (bb * Hkv + g) * cap * kHeadDim) + lane;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  // this wave's keys [t0, t1): contiguous, whole quads except the last
  const int per = ((T + 3) / 4 + kAttnWaves - 1) / kAttnWaves;
  const int t0 = min(T, w * per * 4), t1 = min(T, t0 + per * 4);
  const int kk = lane >> 4, dc = (lane & 15) * 8;
  float* scw = &sc[w][0][0];
  auto wave_sync = [] {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  {
    float rm[HPB], rl[HPB], o0[HPB], o1[HPB];
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      rm[hh] = -INFINITY;
      rl[hh] = o0[hh] = o1[hh] = 0.f;
    }
    float qf[HPB][8];
    for (int c0 = t0; c0 < t1; c0 += kAttnChunk) {
      const int len = min(kAttnChunk, t1 - c0);
      // every key and value load of the chunk, then (first chunk) the queries
      uint4 kr[kAttnQuads];
      uint32_t vv[kAttnChunk];
#pragma unroll
      for (int j = 0; j < kAttnQuads; ++j)
        if (4 * j < len)  // uniform
          kr[j] = *reinterpret_cast<const uint4*>(K + (int64_t)min(c0 + 4 * j + kk, t1 - 1) * kHeadDim + dc);
#pragma unroll
      for (int i = 0; i < kAttnChunk; ++i)
        if (i < len) vv[i] = Vw[(int64_t)(c0 + i) * (kHeadDim / 2)];
      if (c0 == t0) {
#pragma unroll
        for (int hh = 0; hh < HPB; ++hh) {
          const float* qr = q + m * (H * kHeadDim) +
                            (int64_t)(g * grp + h0 + min(hh, nh - 1)) * kHeadDim + dc;
          const float4 x0 = *reinterpret_cast<const float4*>(qr);
          const float4 x1 = *reinterpret_cast<const float4*>(qr + 4);
          qf[hh][0] = x0.x; qf[hh][1] = x0.y; qf[hh][2] = x0.z; qf[hh][3] = x0.w;
          qf[hh][4] = x1.x; qf[hh][5] = x1.y; qf[hh][6] = x1.z; qf[hh][7] = x1.w;
        }
      }
      // scores and the chunk max
      float cm[HPB];
#pragma unroll
      for (int hh = 0; hh < HPB; ++hh) cm[hh] = -INFINITY;
#pragma unroll
      for (int j = 0; j < kAttnQuads; ++j) {
        if (4 * j >= len) break;     // uniform
        const int t = 4 * j + kk;    // within the chunk
        const uint32_t wv[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
        for (int hh = 0; hh < HPB; ++hh) {
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = fmaf(qf[hh][2 * i], __uint_as_float(wv[i] << 16), part);
            part = fmaf(qf[hh][2 * i + 1], __uint_as_float(wv[i] & 0xFFFF0000u), part);
          }
          part = sum16_dpp(part);
          const float sv = part * scale;
          if (t < len && (lane & 15) == 0) {  // lane 16 j of the row keeps the score
            cm[hh] = fmaxf(cm[hh], sv);
            scw[hh * kAttnChunk + t] = sv;
          }
        }
      }
      wave_sync();
      // running max, rescale, p = exp(s - m), chunk sums (lane t of the chunk)
#pragma unroll
      for (int hh = 0; hh < HPB; ++hh) {
        cm[hh] = wave_max_dpp(cm[hh]);  // exact: every lane gets the chunk's largest score
        const float mn = fmaxf(rm[hh], cm[hh]);
        const float f = rm[hh] == -INFINITY ? 0.f : __expf(rm[hh] - mn);
        rl[hh] *= f;
        o0[hh] *= f;
        o1[hh] *= f;
        rm[hh] = mn;
        float pv = 0.f;
        if (lane < len) {
          pv = __expf(scw[hh * kAttnChunk + lane] - mn);
          scw[hh * kAttnChunk + lane] = pv;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) pv += __shfl_xor(pv, o);
        rl[hh] += pv;
      }
      wave_sync();
      // values: dims 2 lane, 2 lane + 1 over the chunk's keys in order
#pragma unroll
      for (int i = 0; i < kAttnChunk; ++i) {
        if (i < len) {  // uniform
          const float va = __uint_as_float(vv[i] << 16), vb = __uint_as_float(vv[i] & 0xFFFF0000u);
#pragma unroll
          for (int hh = 0; hh < HPB; ++hh) {
            const float pt = scw[hh * kAttnChunk + i];
            o0[hh] = fmaf(pt, va, o0[hh]);
            o1[hh] = fmaf(pt, vb, o1[hh]);
          }
        }
      }
      wave_sync();  // the next chunk rewrites this wave's scores
    }
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      po[w][hh][2 * lane] = o0[hh];
      po[w][hh][2 * lane + 1] = o1[hh];
      if (lane == 0) {
        pm[w][hh] = rm[hh];
        pl[w][hh] = rl[hh];
      }
    }
    __syncthreads();
    // the wavefronts merged in wave order; one output element per thread
    for (int e = threadIdx.x; e < nh * kHeadDim; e += 64 * kAttnWaves) {
      const int hh = e / kHeadDim, d = e % kHeadDim;
      float M_ = pm[0][hh];
      for (int ww = 1; ww < kAttnWaves; ++ww) M_ = fmaxf(M_, pm[ww][hh]);
      float o = 0.f, l = 0.f;
      for (int ww = 0; ww < kAttnWaves; ++ww) {
        if (pm[ww][hh] == -INFINITY) continue;  // an empty range
        const float f = __expf(pm[ww][hh] - M_);
        o = fmaf(po[ww][hh][d], f, o);
        l = fmaf(pl[ww][hh], f, l);
      }
      const float inv = T > 0 ? 1.0f / l : 0.f;
      out[m * (H * kHeadDim) + (int64_t)(g * grp + h0 + hh) * kHeadDim + d] = f32_to_bf16_rne(o * inv);
    }
  }
}

template <int HPB>
__global__ __launch_bounds__(64 * kAttnWaves) void attention_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    int H, int Hkv, const int32_t* __restrict__ seq, const int32_t* __restrict__ pos, int64_t B,
    int64_t cap, uint16_t* __restrict__ out) {
  attend<HPB>(q, kc, vc, H, Hkv, seq, pos, B, cap, out);
}

// RoPE + KV write + attention in one launch, for launches whose rows belong
// to different sequences (one row per sequence: decode and draft forwards).
// Block (m, g, part) first does rope_kv's work for row m restricted to what
// it attends with -- its query heads rotated into q, key head g rotated and
// value head g written into the caches at the row's position, the same fp64
// arithmetic and roundings -- then attends exactly as attention_kernel does.
// Every part of kv head g writes the same key and value bytes (the same
// arithmetic on the same inputs), each before its own barrier, so each block
// reads the row's key and value as its own stores left them; no block of
// another row writes to this sequence's cache rows.
template <int HPB>
__global__ __launch_bounds__(64 * kAttnWaves) void rope_attention_kernel(
    const float* __restrict__ qkv, int H, int Hkv, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, double base, float* __restrict__ q, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, int64_t B, int64_t cap, uint16_t* __restrict__ out) {
  __shared__ double cs[2][kHeadDim / 2];
  const int64_t m = blockIdx.x;
  int g, h0, nh;
  attn_block_heads<HPB>(H, Hkv, g, h0, nh);
  const int hd = kHeadDim, half = hd / 2, grp = H / Hkv;
  const int p = pos[m];
  const int64_t b = seq[m];
  const bool ok = b >= 0 && b < B && p >= 0 && p < cap;
  if (ok) {  // uniform
    if (threadIdx.x < half) {
      const double f = pow(base, -2.0 * (double)threadIdx.x / (double)hd);
      double sn, c;
      sincos((double)p * f, &sn, &c);
      cs[0][threadIdx.x] = c;
      cs[1][threadIdx.x] = sn;
    }
    __syncthreads();
    const float* r = qkv + m * (int64_t)((H + 2 * Hkv) * hd);
    // this block's nh query heads, then key head g (index nh)
    for (int t = threadIdx.x; t < (nh + 1) * half; t += blockDim.x) {
      const int hh = t / half, i = t % half;
      const int h = hh < nh ? g * grp + h0 + hh : H + g;  // column block of qkv
      const double a = r[h * hd + i], bb = r[h * hd + i + half];
      const double c = cs[0][i], sn = cs[1][i];
      const double lo = a * c - bb * sn, hi = bb * c + a * sn;
      if (hh < nh) {
        q[m * (H * hd) + h * hd + i] = (float)lo;
        q[m * (H * hd) + h * hd + i + half] = (float)hi;
      } else {
        uint16_t* dst = kc + ((b * Hkv + g) * cap + p) * hd;
        dst[i] = f64_to_bf16_rne(lo);
        dst[i + half] = f64_to_bf16_rne(hi);
      }
    }
    for (int t = threadIdx.x; t < hd; t += blockDim.x)
      vc[((b * Hkv + g) * cap + p) * hd + t] = f32_to_bf16_rne(r[(H + Hkv + g) * hd + t]);
  }
  __syncthreads();  // the rotated queries and this row's key and value are in memory
  attend<HPB>(q, kc, vc, H, Hkv, seq, pos, B, cap, out);
}

// ------------------------------------------------------------------ SiLU * up
// a[m][j] = bf16(silu(g) * u), g = gu[m][j], u = gu[m][F + j], fp64 inside
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ gu, int64_t M,
                                                       int64_t F, uint16_t* __restrict__ a) {
  const int64_t n = M * F;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / F, j = t % F;
    a[t] = swiglu_bf16(gu[m * 2 * F + j], gu[m * 2 * F + F + j]);
  }
}

// The same over gate|up outputs in pair order (the row order the fused
// gate|up GEMM reads): in each 16-column block b of gu[m], columns 16b ..
// 16b + 7 are gate rows 8b .. 8b + 7 and columns 16b + 8 .. 16b + 15 the
// matching up rows, so a[m][8b + i] = bf16(silu(gu[m][16b + i]) *
// gu[m][16b + 8 + i]).  F % 8 == 0.
__global__ __launch_bounds__(256) void silu_mul_pairs_kernel(const float* __restrict__ gu,
                                                             int64_t M, int64_t F,
                                                             uint16_t* __restrict__ a) {
  const int64_t n = M * F;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / F, j = t % F;
    const int64_t c = m * 2 * F + (j >> 3) * 16 + (j & 7);
    a[t] = swiglu_bf16(gu[c], gu[c + 8]);
  }
}

// ------------------------------------------------------------------ argmax
// out[m * stride] = the first index of the largest value of row m.  One
// 1024-thread block per row; thread t takes 16-byte groups t, t + 1024, ...
// (or single values when the row is not 16-byte aligned), kArgmaxBatch loads
// in flight, each thread's values in index order; the lowest index wins among
// equal values, so the answer does not depend on the merge order.
constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxBatch = 8;

__device__ __forceinline__ void argmax_take(float& best, int& idx, float v, int i) {
  if (v > best || idx == 0x7FFFFFFF) {  // the first value counts even at -inf
    best = v;
    idx = i;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const float* __restrict__ x,
                                                                int64_t V,
                                                                int32_t* __restrict__ out,
                                                                int64_t stride) {
  __shared__ float bv[kArgmaxThreads / 64];
  __shared__ int bi[kArgmaxThreads / 64];
  const int64_t m = blockIdx.x;
  const float* r = x + m * V;
  float best = -INFINITY;
  int idx = 0x7FFFFFFF;
  const int t = threadIdx.x;
  if (VEC) {
    const float4* r4 = reinterpret_cast<const float4*>(r);
    const int64_t n4 = V / 4;
    int64_t g = t;
    for (; g + (kArgmaxBatch - 1) * kArgmaxThreads < n4; g += kArgmaxBatch * kArgmaxThreads) {
      float4 v[kArgmaxBatch];
#pragma unroll
      for (int i = 0; i < kArgmaxBatch; ++i) v[i] = r4[g + i * kArgmaxThreads];
#pragma unroll
      for (int i = 0; i < kArgmaxBatch; ++i) {
        const int e = (int)(4 * (g + i * kArgmaxThreads));
        argmax_take(best, idx, v[i].x, e);
        argmax_take(best, idx, v[i].y, e + 1);
        argmax_take(best, idx, v[i].z, e + 2);
        argmax_take(best, idx, v[i].w, e + 3);
      }
    }
    for (; g < n4; g += kArgmaxThreads) {
      const float4 v = r4[g];
      const int e = (int)(4 * g);
      argmax_take(best, idx, v.x, e);
      argmax_take(best, idx, v.y, e + 1);
      argmax_take(best, idx, v.z, e + 2);
      argmax_take(best, idx, v.w, e + 3);
    }
  } else {
    int64_t j = t;
    for (; j + (kArgmaxBatch - 1) * kArgmaxThreads < V; j += kArgmaxBatch * kArgmaxThreads) {
      float v[kArgmaxBatch];
#pragma unroll
      for (int i = 0; i < kArgmaxBatch; ++i) v[i] = r[j + i * kArgmaxThreads];
#pragma unroll
      for (int i = 0; i < kArgmaxBatch; ++i) argmax_take(best, idx, v[i], (int)(j + i * kArgmaxThreads));
    }
    for (; j < V; j += kArgmaxThreads) argmax_take(best, idx, r[j], (int)j);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int oi = __shfl_xor(idx, o);
    if (ov > best || (ov == best && oi < idx)) {
      best = ov;
      idx = oi;
    }
  }
  const int w = t >> 6;
  if ((t & 63) == 0) {
    bv[w] = best;
    bi[w] = idx;
  }
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kArgmaxThreads / 64; ++i)
      if (bv[i] > best || (bv[i] == best && bi[i] < idx)) {
        best = bv[i];
        idx = bi[i];
      }
    out[m * stride] = idx;
  }
}

// ------------------------------------------------------------------ round bookkeeping
// phase 0 (draft step j): rows b = 0..B-1 at position len[b]-1+j with token
//   vtok[b][j];
// phase 1 (verify): rows r = b*(gamma+1)+i at position len[b]-1+i with token
//   vtok[b][i]; also drafts[b][i-1] = vtok[b][i] for i >= 1.
__global__ __launch_bounds__(256) void spec_prepare_kernel(int phase, int64_t B, int gamma, int j,
                                                           const int32_t* __restrict__ len,
                                                           const int32_t* __restrict__ vtok,
                                                           int32_t* __restrict__ drafts,
                                                           int32_t* __restrict__ seq,
                                                           int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ tok) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int S = gamma + 1;
  if (phase == 0) {
    if (t >= B) return;
    seq[t] = (int32_t)t;
    pos[t] = len[t] - 1 + j;
    tok[t] = vtok[t * S + j];
  } else {
    if (t >= B * S) return;
    const int64_t b = t / S;
    const int i = (int)(t % S);
    seq[t] = (int32_t)b;
    pos[t] = len[b] - 1 + i;
    tok[t] = vtok[t];
    if (i >= 1) drafts[b * gamma + i - 1] = vtok[t];
  }
}

// Commit one round: for every sequence still short of max_gen tokens, append
// out_tok[b][0..n] (n = n_accept[b], 0 when n_accept is NULL), advance len and
// the generated count by n+1, and make out_tok[b][n] the next round's first
// input token (vtok[b][0], row stride vstride).  stats[0] += accepted drafts,
// stats[1] += active sequences this round, stats[2] = sequences still active
// afterwards.  One block; sequences b = tid, tid + 256, ...
__global__ __launch_bounds__(256) void spec_commit_kernel(int64_t B, int gamma,
                                                          const int32_t* __restrict__ n_accept,
                                                          const int32_t* __restrict__ out_tok,
                                                          int32_t* __restrict__ len,
                                                          int32_t* __restrict__ vtok,
                                                          int64_t vstride,
                                                          int32_t* __restrict__ gen,
                                                          int64_t gen_cap,
                                                          int32_t* __restrict__ n_gen,
                                                          int max_gen, int64_t* __restrict__ stats) {
  __shared__ int64_t red[4];
  int64_t acc = 0, act = 0, still = 0;
  for (int64_t b = threadIdx.x; b < B; b += 256) {
    int ng = n_gen[b];
    if (ng < max_gen) {
      const int n = n_accept ? min(max(n_accept[b], 0), gamma) : 0;
      const int32_t* o = out_tok + b * (gamma + 1);
      for (int i = 0; i <= n; ++i)
        if (ng + i < gen_cap) gen[b * gen_cap + ng + i] = o[i];
      ng += n + 1;
      n_gen[b] = ng;
      len[b] += n + 1;
      vtok[b * vstride] = o[n];
      acc += n;
      act += 1;
    }
    still += ng < max_gen ? 1 : 0;
  }
  acc = block_sum_256(acc, red);
  act = block_sum_256(act, red);
  still = block_sum_256(still, red);
  if (threadIdx.x == 0) {
    stats[0] += acc;
    stats[1] += act;
    stats[2] = still;
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_embed(const uint16_t* emb, int64_t V, int64_t d, const int32_t* tok, int64_t M,
                        float* x, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)M), dim3(256), 0, s, emb, V, d, tok, x);
  return hipGetLastError();
}

// The vector kernel wherever its alignment holds: x, add and their row
// strides in whole 16-byte groups, y 8-byte and the codes 2-byte aligned.
static bool norm_v4_ok(const float* x, int64_t xs, const float* add, int64_t as, int64_t d,
                       const uint16_t* y, const uint8_t* yq, int qalign = 2) {
#ifdef QSPEC_NORM_SCALAR
  return false;
#endif
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  return d % 4 == 0 && al(x, 16) && xs % 4 == 0 && (add == nullptr || (al(add, 16) && as % 4 == 0)) &&
         al(y, 8) && (yq == nullptr || al(yq, qalign));
}

hipError_t launch_add_rmsnorm(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                              int64_t d, double eps, uint16_t* y, hipStream_t s) {
  if (norm_v4_ok(x, xs, add, as, d, y, nullptr))
    hipLaunchKernelGGL(add_rmsnorm_v4_kernel<4>, dim3((unsigned)M), dim3(kNormThreads), 0, s, x, xs,
                       add, as, (int)d, eps, y, nullptr, nullptr);
  else
    hipLaunchKernelGGL(add_rmsnorm_kernel<4>, dim3((unsigned)M), dim3(256), 0, s, x, xs, add, as,
                       (int)d, eps, y, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm_quant(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                                    int64_t d, double eps, uint16_t* y, uint8_t* yq, float* ys,
                                    hipStream_t s) {
  if (norm_v4_ok(x, xs, add, as, d, y, yq))
    hipLaunchKernelGGL(add_rmsnorm_v4_kernel<4>, dim3((unsigned)M), dim3(kNormThreads), 0, s, x, xs,
                       add, as, (int)d, eps, y, yq, ys);
  else
    hipLaunchKernelGGL(add_rmsnorm_kernel<4>, dim3((unsigned)M), dim3(256), 0, s, x, xs, add, as,
                       (int)d, eps, y, yq, ys);
  return hipGetLastError();
}

// the W4A8 drafter's 8-bit codes: the 16-byte kernel stores a thread's four
// codes as one 4-byte word, so yq must be 4-byte aligned for it
hipError_t launch_add_rmsnorm_quant8(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                                     int64_t d, double eps, uint16_t* y, int8_t* yq, float* ys,
                                     hipStream_t s) {
  uint8_t* q = reinterpret_cast<uint8_t*>(yq);
  if (norm_v4_ok(x, xs, add, as, d, y, q, 4))
    hipLaunchKernelGGL(add_rmsnorm_v4_kernel<8>, dim3((unsigned)M), dim3(kNormThreads), 0, s, x, xs,
                       add, as, (int)d, eps, y, q, ys);
  else
    hipLaunchKernelGGL(add_rmsnorm_kernel<8>, dim3((unsigned)M), dim3(256), 0, s, x, xs, add, as,
                       (int)d, eps, y, q, ys);
  return hipGetLastError();
}

hipError_t launch_rope_kv(const float* qkv, int64_t M, int H, int Hkv, int hd, const int32_t* seq,
                          const int32_t* pos, double base, float* q, uint16_t* kc, uint16_t* vc,
                          int64_t B, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(rope_kv_kernel, dim3((unsigned)M), dim3(256), 0, s, qkv, H, Hkv, hd, seq, pos,
                     base, q, kc, vc, B, cap);
  return hipGetLastError();
}

// Query heads per block: the largest of 4, 2, 1 whose grid still has
// QSPEC_ATTN_MIN_BLOCKS blocks; a row's output does not depend on it.
// Measured on MI355X (16 q / 4 kv heads, 128 / 256 / 384 keys): 16 decode
// rows with RoPE fused 9.1 / 11.2 / 15.5 us with 4 heads per block (64
// blocks), 7.4 / 9.0 / 11.9 with 2, 6.7 / 8.1 / 10.4 with 1 (256 blocks);
// 80 verify rows 14.2 / 21.2 / 30.3 us with 4, 11.2 / 16.5 / 23.3 with 2
// (640 blocks), 13.7 / 19.1 / 26.7 with 1.  Prefill grids keep 4 (every
// key and value load shared by the whole group).
#ifndef QSPEC_ATTN_MIN_BLOCKS
#define QSPEC_ATTN_MIN_BLOCKS 512
#endif
static int attn_hpb(int64_t M, int H, int Hkv) {
  const int grp = H / Hkv;
  for (int hpb : {4, 2})
    if (M * Hkv * ((grp + hpb - 1) / hpb) >= QSPEC_ATTN_MIN_BLOCKS) return hpb;
  return 1;
}

hipError_t launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t M,
                            int H, int Hkv, const int32_t* seq, const int32_t* pos, int64_t B,
                            int64_t cap, uint16_t* out, hipStream_t s) {
  const int hpb = attn_hpb(M, H, Hkv), grp = H / Hkv;
  const dim3 grid((unsigned)M, (unsigned)(Hkv * ((grp + hpb - 1) / hpb)));
  if (hpb == 4)
    hipLaunchKernelGGL(attention_kernel<4>, grid, dim3(64 * kAttnWaves), 0, s, q, kc, vc, H, Hkv,
                       seq, pos, B, cap, out);
  else if (hpb == 2)
    hipLaunchKernelGGL(attention_kernel<2>, grid, dim3(64 * kAttnWaves), 0, s, q, kc, vc, H, Hkv,
                       seq, pos, B, cap, out);
  else
    hipLaunchKernelGGL(attention_kernel<1>, grid, dim3(64 * kAttnWaves), 0, s, q, kc, vc, H, Hkv,
                       seq, pos, B, cap, out);
  return hipGetLastError();
}

hipError_t launch_rope_attention(const float* qkv, int64_t M, int H, int Hkv, const int32_t* seq,
                                 const int32_t* pos, double base, float* q, uint16_t* kc,
                                 uint16_t* vc, int64_t B, int64_t cap, uint16_t* out,
                                 hipStream_t s) {
  const int hpb = attn_hpb(M, H, Hkv), grp = H / Hkv;
  const dim3 grid((unsigned)M, (unsigned)(Hkv * ((grp + hpb - 1) / hpb)));
  if (hpb == 4)
    hipLaunchKernelGGL(rope_attention_kernel<4>, grid, dim3(64 * kAttnWaves), 0, s, qkv, H, Hkv,
                       seq, pos, base, q, kc, vc, B, cap, out);
  else if (hpb == 2)
    hipLaunchKernelGGL(rope_attention_kernel<2>, grid, dim3(64 * kAttnWaves), 0, s, qkv, H, Hkv,
                       seq, pos, base, q, kc, vc, B, cap, out);
  else
    hipLaunchKernelGGL(rope_attention_kernel<1>, grid, dim3(64 * kAttnWaves), 0, s, qkv, H, Hkv,
                       seq, pos, base, q, kc, vc, B, cap, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gu, int64_t M, int64_t F, uint16_t* a, hipStream_t s) {
  const int64_t n = M * F;
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, s, gu, M, F, a);
  return hipGetLastError();
}

hipError_t launch_silu_mul_pairs(const float* gu, int64_t M, int64_t F, uint16_t* a,
                                 hipStream_t s) {
  const int64_t n = M * F;
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
  hipLaunchKernelGGL(silu_mul_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, gu, M, F, a);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int64_t M, int64_t V, int32_t* out, int64_t stride,
                         hipStream_t s) {
  // 16-byte loads when every row starts 16-byte aligned
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0 && (V & 3) == 0)
    hipLaunchKernelGGL((argmax_kernel<true>), dim3((unsigned)M), dim3(kArgmaxThreads), 0, s, x, V, out,
                       stride);
  else
    hipLaunchKernelGGL((argmax_kernel<false>), dim3((unsigned)M), dim3(kArgmaxThreads), 0, s, x, V,
                       out, stride);
  return hipGetLastError();
}

hipError_t launch_spec_prepare(int phase, int64_t B, int gamma, int j, const int32_t* len,
                               const int32_t* vtok, int32_t* drafts, int32_t* seq, int32_t* pos,
                               int32_t* tok, hipStream_t s) {
  const int64_t rows = phase == 0 ? B : B * (gamma + 1);
  hipLaunchKernelGGL(spec_prepare_kernel, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, s, phase,
                     B, gamma, j, len, vtok, drafts, seq, pos, tok);
  return hipGetLastError();
}

hipError_t launch_spec_commit(int64_t B, int gamma, const int32_t* n_accept, const int32_t* out_tok,
                              int32_t* len, int32_t* vtok, int64_t vstride, int32_t* gen,
                              int64_t gen_cap, int32_t* n_gen, int max_gen, int64_t* stats,
                              hipStream_t s) {
  hipLaunchKernelGGL(spec_commit_kernel, dim3(1), dim3(256), 0, s, B, gamma, n_accept, out_tok,
                     len, vtok, vstride, gen, gen_cap, n_gen, max_gen, stats);
  return hipGetLastError();
}

}  // namespace qspec
