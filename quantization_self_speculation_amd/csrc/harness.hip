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

// fp64 -> bf16 with one rounding: truncate to fp32 and set the lowest bit if
// anything was dropped (round to odd keeps the information a later rounding
// to nearest needs), then round fp32 -> bf16 to nearest even.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  float t = __double2float_rz(v);
  uint32_t u = __float_as_uint(t);
  if ((double)t != v) u |= 1u;
  return f32_to_bf16_rne(__uint_as_float(u));
}

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
template <int PER>
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
  const float s = a / 7.0f;
  const float r = 1.0f / s;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = (int)threadIdx.x + 256 * i;
    const int c = (j < n && s != 0.0f) ? quant_code_act(__uint_as_float((uint32_t)yb[i] << 16), s, r) : 0;
    const int nb = __shfl_xor(c, 1, 64);
    if (!(threadIdx.x & 1) && j < n) q[j >> 1] = (uint8_t)((c & 0xF) | ((nb & 0xF) << 4));
  }
  if (threadIdx.x == 0) *qs = s;
}

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
  if (yq != nullptr) quant_row_bf16<kNormPer>(yb, d, redf, yq + m * (d / 2), ys + m);  // uniform
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
// One 256-thread block per (row, kv head); wave w serves the query heads
// g*grp + w, w+4, ...  Each lane scores keys t = lane, lane+64, ... (a full
// 128-term dot product, fp32, fixed order), the scores sit in LDS; softmax
// with the max subtracted; then lane l accumulates output dims 2l, 2l+1 over
// t in increasing order.  Output bf16.
constexpr int kHeadDim = 128;

__global__ __launch_bounds__(256) void attention_kernel(const float* __restrict__ q,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vc, int H,
                                                        int Hkv, const int32_t* __restrict__ seq,
                                                        const int32_t* __restrict__ pos, int64_t B,
                                                        int64_t cap, uint16_t* __restrict__ out) {
  extern __shared__ float lds[];  // [4][kHeadDim + cap]
  const int64_t m = blockIdx.x;
  const int g = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = H / Hkv;
  const int64_t b = seq[m];
  // rows outside the cache attend to nothing (output 0)
  const bool ok = b >= 0 && b < B && pos[m] >= 0 && pos[m] < cap;
  const int T = ok ? pos[m] + 1 : 0;
  const int64_t bb = ok ? b : 0;
  const uint16_t* K = kc + (bb * Hkv + g) * cap * kHeadDim;
  const uint16_t* Vv = vc + (bb * Hkv + g) * cap * kHeadDim;
  float* qs = lds + w * (kHeadDim + cap);
  float* sc = qs + kHeadDim;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  for (int hh = w; hh < grp; hh += 4) {
    const int h = g * grp + hh;
    const float* qr = q + m * (H * kHeadDim) + h * kHeadDim;
    qs[lane] = qr[lane];
    qs[lane + 64] = qr[lane + 64];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float mx = -INFINITY;
    for (int t = lane; t < T; t += 64) {
      const uint16_t* kr = K + (int64_t)t * kHeadDim;
      float acc = 0.f;
#pragma unroll 4
      for (int j = 0; j < kHeadDim; j += 8) {
        const uint4 p = *reinterpret_cast<const uint4*>(kr + j);
        const uint32_t wv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(qs[j + 2 * i], __uint_as_float(wv[i] << 16), acc);
          acc = fmaf(qs[j + 2 * i + 1], __uint_as_float(wv[i] & 0xFFFF0000u), acc);
        }
      }
      const float s = acc * scale;
      sc[t] = s;
      mx = fmaxf(mx, s);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float den = 0.f;
    for (int t = lane; t < T; t += 64) {
      const float e = __expf(sc[t] - mx);
      sc[t] = e;
      den += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float o0 = 0.f, o1 = 0.f;
    const uint32_t* vcol = reinterpret_cast<const uint32_t*>(Vv) + lane;  // dims 2l, 2l+1
    int t = 0;
    for (; t + 32 <= T; t += 32) {  // 32 value rows in flight, added in order
      uint32_t vv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) vv[i] = vcol[(int64_t)(t + i) * (kHeadDim / 2)];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float pt = sc[t + i];
        o0 = fmaf(pt, __uint_as_float(vv[i] << 16), o0);
        o1 = fmaf(pt, __uint_as_float(vv[i] & 0xFFFF0000u), o1);
      }
    }
    for (; t < T; ++t) {
      const float pt = sc[t];
      const uint32_t vv = vcol[(int64_t)t * (kHeadDim / 2)];
      o0 = fmaf(pt, __uint_as_float(vv << 16), o0);
      o1 = fmaf(pt, __uint_as_float(vv & 0xFFFF0000u), o1);
    }
    const float inv = T > 0 ? 1.0f / den : 0.f;
    uint16_t* orow = out + m * (H * kHeadDim) + h * kHeadDim;
    orow[2 * lane] = f32_to_bf16_rne(o0 * inv);
    orow[2 * lane + 1] = f32_to_bf16_rne(o1 * inv);
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------ SiLU * up
// a[m][j] = bf16(silu(g) * u), g = gu[m][j], u = gu[m][F + j], fp64 inside
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ gu, int64_t M,
                                                       int64_t F, uint16_t* __restrict__ a) {
  const int64_t n = M * F;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / F, j = t % F;
    const double g = gu[m * 2 * F + j], u = gu[m * 2 * F + F + j];
    a[t] = f64_to_bf16_rne(g / (1.0 + exp(-g)) * u);
  }
}

// ------------------------------------------------------------------ argmax
// out[m * stride] = the first index of the largest value of row m
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ x, int64_t V,
                                                     int32_t* __restrict__ out, int64_t stride) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  const int64_t m = blockIdx.x;
  const float* r = x + m * V;
  float best = -INFINITY;
  int idx = 0x7FFFFFFF;
  int64_t j = threadIdx.x;
  for (; j + 3 * 256 < V; j += 4 * 256) {  // four loads in flight, compared in index order
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[j + 256 * i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v[i] > best || idx == 0x7FFFFFFF) {  // the first value counts even at -inf
        best = v[i];
        idx = (int)(j + 256 * i);
      }
  }
  for (; j < V; j += 256) {
    const float v = r[j];
    if (v > best || idx == 0x7FFFFFFF) {
      best = v;
      idx = (int)j;
    }
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
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    bv[w] = best;
    bi[w] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 4; ++i)
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

hipError_t launch_add_rmsnorm(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                              int64_t d, double eps, uint16_t* y, hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, x, xs, add, as,
                     (int)d, eps, y, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm_quant(float* x, int64_t xs, const float* add, int64_t as, int64_t M,
                                    int64_t d, double eps, uint16_t* y, uint8_t* yq, float* ys,
                                    hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, x, xs, add, as,
                     (int)d, eps, y, yq, ys);
  return hipGetLastError();
}

hipError_t launch_rope_kv(const float* qkv, int64_t M, int H, int Hkv, int hd, const int32_t* seq,
                          const int32_t* pos, double base, float* q, uint16_t* kc, uint16_t* vc,
                          int64_t B, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(rope_kv_kernel, dim3((unsigned)M), dim3(256), 0, s, qkv, H, Hkv, hd, seq, pos,
                     base, q, kc, vc, B, cap);
  return hipGetLastError();
}

size_t attention_lds_bytes(int64_t cap) { return (size_t)4 * (kHeadDim + cap) * sizeof(float); }

hipError_t launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t M,
                            int H, int Hkv, const int32_t* seq, const int32_t* pos, int64_t B,
                            int64_t cap, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)M, (unsigned)Hkv), dim3(256),
                     attention_lds_bytes(cap), s, q, kc, vc, H, Hkv, seq, pos, B, cap, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gu, int64_t M, int64_t F, uint16_t* a, hipStream_t s) {
  const int64_t n = M * F;
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 4096);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, s, gu, M, F, a);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int64_t M, int64_t V, int32_t* out, int64_t stride,
                         hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)M), dim3(256), 0, s, x, V, out, stride);
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
