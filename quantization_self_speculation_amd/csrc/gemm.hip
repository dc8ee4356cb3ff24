// The dual-mode linear layer: W4A16 (verifier) and W4A4 (drafter) GEMMs over
// the one shared packed INT4 weight buffer.
//
// Pages: "QSpec: Speculative Decoding with Complementary Quantization
// Schemes", Abstract (arXiv) -- low-precision joint quantization (W4A4) for
// drafting, high-precision weight-only quantization (W4A16) for verification,
// the same weights for both; tech-dashboard QSpec summary, paragraph 2 --
// W4A4 pays off on hardware with low-precision arithmetic units.
//
// Arithmetic (the reading of the pages, which give no formula):
//   W4A16: Y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] * q[n,k]
//   W4A4:  Y[m,n] = a[m] * sum_g s[n,g] * P[m,n,g],  P exact in int32
//
// gfx950 design
//  * Codes are widened in registers only; the shared buffer stays 4-bit.
//    W4A16 turns a nibble into the bf16 of 136 + q with one AND-OR (exact),
//    runs v_mfma_f32_16x16x32_bf16 and removes the bias with the group sum of
//    x in the fp32 epilogue.  W4A4 turns nibbles into int8 holding 16 q with
//    one AND (exact) and runs v_mfma_i32_16x16x64_i8; the int32 group partial
//    is 256 P exactly.
//  * MFMA operand A = 16 weight rows (n), operand B = 16 activation rows (m),
//    so each lane of D holds 4 consecutive n of one m: one 16-byte store.
//  * Within a 128-group, lane l feeds the 32 consecutive k starting at
//    32*(l/16) into the MFMA k-slots (one 16-byte weight load per lane per
//    group); activations are staged in LDS in the matching slot order.  The
//    sum over a group is therefore the same set of products in every kernel.
//  * Each output accumulates its groups in ascending order, one fp32
//    epilogue per group; K is split into slices only as a function of (N, K),
//    and slices are reduced in fixed order -- no atomics -- so an output row
//    is bitwise the same for every M.
#include "launch.h"

namespace qspec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// streaming (non-temporal) 16-byte load: weights are read exactly once
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ v8bf as_v8bf(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 t = {a, b, c, d};
  return __builtin_bit_cast(v8bf, t);
}
__device__ __forceinline__ v4i as_v4i(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4i t = {(int)a, (int)b, (int)c, (int)d};
  return t;
}

// Sum of a 128-element activation group held as 16 chunks of 8 by 16
// consecutive lanes (aligned to 16): fixed butterfly, identical bits in all
// 16 lanes and in every kernel that calls it.
__device__ __forceinline__ float group_sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// ============================================================================
// W4A16, MFMA "skinny" family: weights streamed straight from HBM into
// registers (each byte used by exactly one wavefront), activations of up to
// 64 rows shared by the 4 wavefronts of a workgroup through LDS.
//   grid = (ceil(N / (64 NB)), S k-slices, ceil(M / (16 MB)) m-chunks)
// ============================================================================
template <int NB, int MB, int CH>
__global__ __launch_bounds__(256) void w4a16_skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ Ws, int M, int N, int K, int gps, float* __restrict__ out,
    int64_t slice_stride) {
  constexpr int ROWS = 16 * MB;        // activation rows per m-chunk
  constexpr int XST = CH * 128 + 8;    // LDS row stride in bf16 (16-byte pad)
  constexpr int WROWS = 64 * NB;       // weight rows per workgroup
  constexpr int XCH = ROWS * CH * 16;  // 16-byte activation chunks per stage
  constexpr int XPT = XCH / 256;       // ... per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][ROWS * XST];
  __shared__ float xsum[2][ROWS * CH];
  __shared__ uint16_t wsl[2][CH * WROWS];

  const int G = K / kGroup;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n_wg = blockIdx.x * WROWS;
  const int n_w = n_wg + wave * 16 * NB;
  const int g_begin = blockIdx.y * gps;
  const int g_end = min(G, g_begin + gps);
  const int m0 = blockIdx.z * ROWS;
  const int nchunks = (g_end - g_begin + CH - 1) / CH;

  const uint8_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_w + nb * 16 + l16, N - 1);
    wrow[nb] = Wq + (int64_t)n * (K / 2) + lg * 16;
  }

  uint4 wcur[CH][NB], wnext[CH][NB];
  uint4 xr[XPT];
  uint16_t sr[(CH * WROWS + 255) / 256];

  auto load_w = [&](int c, uint4 (&w)[CH][NB]) {
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int gl = 0; gl < CH; ++gl)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        w[gl][nb] = (gc + gl < g_end)
                        ? ld_stream(wrow[nb] + (int64_t)(gc + gl) * 64)
                        : make_uint4(0, 0, 0, 0);
  };
  auto load_x = [&](int c) {
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int r = idx / (CH * 16), cc = idx % (CH * 16);
      const bool ok = (m0 + r < M) && (gc + (cc >> 4) < g_end);
      xr[i] = ok ? *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + r) * K +
                                                   (int64_t)gc * kGroup + cc * 8)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < (CH * WROWS + 255) / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < CH * WROWS) {
        const int gl = idx / WROWS, rr = idx % WROWS;
        const int n = min(n_wg + rr, N - 1);
        sr[i] = (gc + gl < g_end) ? Ws[(int64_t)n * G + gc + gl] : (uint16_t)0;
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int r = idx / (CH * 16), cc = idx % (CH * 16);
      const uint32_t v[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
      uint32_t p[4];
      bf16x8_interleave(v, p);
      *reinterpret_cast<uint4*>(&xs[buf][r * XST + cc * 8]) = make_uint4(p[0], p[1], p[2], p[3]);
      const float s = group_sum16(bf16x8_sum(v));
      if ((cc & 15) == 0) xsum[buf][r * CH + (cc >> 4)] = s;
    }
#pragma unroll
    for (int i = 0; i < (CH * WROWS + 255) / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < CH * WROWS) wsl[buf][idx] = sr[i];
    }
  };

  v4f tot[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nchunks > 0) {
    load_w(0, wcur);
    load_x(0);
    store_x(0);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1, wnext);
      load_x(c + 1);
    }
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int gl = 0; gl < CH; ++gl) {
      if (gc + gl < g_end) {
        v4f acc[NB][MB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8bf b[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            b[mb] = *reinterpret_cast<const v8bf*>(
                &xs[buf][(mb * 16 + l16) * XST + gl * 128 + lg * 32 + j * 8]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint4 w = wcur[gl][nb];
            const uint32_t wd = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
            uint32_t a4[4];
            w4_to_bf16_biased(wd, a4);
            const v8bf a = as_v8bf(a4[0], a4[1], a4[2], a4[3]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[mb], acc[nb][mb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float xsm = xsum[buf][(mb * 16 + l16) * CH + gl];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint16_t* wp = &wsl[buf][gl * WROWS + wave * 16 * NB + nb * 16 + lg * 4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float t = fmaf(-kW4Bias, xsm, acc[nb][mb][r]);
              tot[nb][mb][r] = fmaf(half_bits_to_float(wp[r]), t, tot[nb][mb][r]);
            }
          }
        }
      }
    }
    if (more) store_x(buf ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int gl = 0; gl < CH; ++gl)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wcur[gl][nb] = wnext[gl][nb];
    }
  }

  float* o = out + (int64_t)blockIdx.y * slice_stride;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + l16;
      const int n = n_w + nb * 16 + lg * 4;
      if (m < M && n < N) {
        float* dst = o + (int64_t)m * N + n;
        if (vec) {
          *reinterpret_cast<float4*>(dst) =
              make_float4(tot[nb][mb][0], tot[nb][mb][1], tot[nb][mb][2], tot[nb][mb][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = tot[nb][mb][r];
        }
      }
    }
}

// ============================================================================
// W4A4, MFMA "skinny" family: same structure; codes widened to int8 (16 q),
// v_mfma_i32_16x16x64_i8, exact int32 group partial, fp32 scale epilogue.
// ============================================================================
template <int NB, int MB, int CH>
__global__ __launch_bounds__(256) void w4a4_skinny_kernel(
    const uint8_t* __restrict__ Xq, const float* __restrict__ Xs, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ Ws, int M, int N, int K, int gps, float* __restrict__ out,
    int64_t slice_stride, int32_t* __restrict__ P, int apply_xs) {
  constexpr int ROWS = 16 * MB;
  constexpr int XST = CH * 128 + 16;   // LDS row stride in bytes (int8 codes)
  constexpr int WROWS = 64 * NB;
  constexpr int XCH = ROWS * CH * 4;   // 16-byte packed chunks (32 codes) per stage
  constexpr int XPT = (XCH + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][ROWS * XST];
  __shared__ uint16_t wsl[2][CH * WROWS];

  const int G = K / kGroup;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n_wg = blockIdx.x * WROWS;
  const int n_w = n_wg + wave * 16 * NB;
  const int g_begin = blockIdx.y * gps;
  const int g_end = min(G, g_begin + gps);
  const int m0 = blockIdx.z * ROWS;
  const int nchunks = (g_end - g_begin + CH - 1) / CH;

  const uint8_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_w + nb * 16 + l16, N - 1);
    wrow[nb] = Wq + (int64_t)n * (K / 2) + lg * 16;
  }

  uint4 wcur[CH][NB], wnext[CH][NB];
  uint4 xr[XPT];
  uint16_t sr[(CH * WROWS + 255) / 256];

  auto load_w = [&](int c, uint4 (&w)[CH][NB]) {
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int gl = 0; gl < CH; ++gl)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        w[gl][nb] = (gc + gl < g_end)
                        ? ld_stream(wrow[nb] + (int64_t)(gc + gl) * 64)
                        : make_uint4(0, 0, 0, 0);
  };
  auto load_x = [&](int c) {
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int r = idx / (CH * 4), cc = idx % (CH * 4);
      const bool ok = idx < XCH && (m0 + r < M) && (gc + (cc >> 2) < g_end);
      xr[i] = ok ? *reinterpret_cast<const uint4*>(Xq + (int64_t)(m0 + r) * (K / 2) +
                                                   (int64_t)gc * 64 + cc * 16)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < (CH * WROWS + 255) / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < CH * WROWS) {
        const int gl = idx / WROWS, rr = idx % WROWS;
        const int n = min(n_wg + rr, N - 1);
        sr[i] = (gc + gl < g_end) ? Ws[(int64_t)n * G + gc + gl] : (uint16_t)0;
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < XCH) {
        const int r = idx / (CH * 4), cc = idx % (CH * 4);
        const uint4 p = xr[i];
        uint8_t* dst = &xs[buf][r * XST + (cc >> 2) * 128 + (cc & 3) * 32];
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(w4_lo_x16(p.x), w4_hi_x16(p.x), w4_lo_x16(p.y), w4_hi_x16(p.y));
        *reinterpret_cast<uint4*>(dst + 16) =
            make_uint4(w4_lo_x16(p.z), w4_hi_x16(p.z), w4_lo_x16(p.w), w4_hi_x16(p.w));
      }
    }
#pragma unroll
    for (int i = 0; i < (CH * WROWS + 255) / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < CH * WROWS) wsl[buf][idx] = sr[i];
    }
  };

  v4f tot[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nchunks > 0) {
    load_w(0, wcur);
    load_x(0);
    store_x(0);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1, wnext);
      load_x(c + 1);
    }
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int gl = 0; gl < CH; ++gl) {
      if (gc + gl < g_end) {
        v4i acc[NB][MB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v4i b[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            b[mb] = *reinterpret_cast<const v4i*>(
                &xs[buf][(mb * 16 + l16) * XST + gl * 128 + lg * 32 + j * 16]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint4 w = wcur[gl][nb];
            const uint32_t p0 = j == 0 ? w.x : w.z, p1 = j == 0 ? w.y : w.w;
            const v4i a = as_v4i(w4_lo_x16(p0), w4_hi_x16(p0), w4_lo_x16(p1), w4_hi_x16(p1));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[nb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[mb], acc[nb][mb], 0, 0, 0);
          }
        }
        const int g = gc + gl;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* wp = &wsl[buf][gl * WROWS + wave * 16 * NB + nb * 16 + lg * 4];
          float sc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] = half_bits_to_float(wp[r]) * 0.00390625f;  // / 256
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              tot[nb][mb][r] = fmaf(sc[r], (float)acc[nb][mb][r], tot[nb][mb][r]);
            if (P != nullptr) {
              const int m = m0 + mb * 16 + l16;
              const int n = n_w + nb * 16 + lg * 4;
              if (m < M) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < N) P[((int64_t)m * N + n + r) * G + g] = acc[nb][mb][r] >> 8;
              }
            }
          }
        }
      }
    }
    if (more) store_x(buf ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int gl = 0; gl < CH; ++gl)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wcur[gl][nb] = wnext[gl][nb];
    }
  }

  float* o = out + (int64_t)blockIdx.y * slice_stride;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + l16;
      const int n = n_w + nb * 16 + lg * 4;
      if (m < M && n < N) {
        const float a = apply_xs ? Xs[m] : 1.0f;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = apply_xs ? a * tot[nb][mb][r] : tot[nb][mb][r];
        float* dst = o + (int64_t)m * N + n;
        if (vec) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = v[r];
        }
      }
    }
}

// ============================================================================
// W4A16 GEMV family (M <= 4): VALU dot products, one wavefront per row at a
// time, lanes along K (16 bytes = 32 codes each, 1 KiB per row per pass),
// cross-lane reduction per row.  Activations live in registers.
//   grid = (ceil(N / (4 RPW)), ceil(K / 2048))
// ============================================================================
template <int MM, int RPW>
__global__ __launch_bounds__(256) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ Ws, int N, int K, float* __restrict__ out, int64_t slice_stride) {
  const int G = K / kGroup;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = blockIdx.y * 2048 + lane * 32;  // this lane's 32 codes
  const bool kv = k0 < K;
  const int g = k0 / kGroup;

  // activations for the lane's 32 k, pair-interleaved to match the codes
  uint32_t xp[MM][16];
  float xsl[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = kv ? *reinterpret_cast<const uint4*>(X + (int64_t)m * K + k0 + c * 8)
                   : make_uint4(0, 0, 0, 0);
      const uint32_t n4[4] = {v.x, v.y, v.z, v.w};
      uint32_t p[4];
      bf16x8_interleave(n4, p);
#pragma unroll
      for (int i = 0; i < 4; ++i) xp[m][c * 4 + i] = p[i];
      s += bf16x8_sum(n4);
    }
    xsl[m] = s;
  }

  const int nbase = (blockIdx.x * 4 + wave) * RPW;
  float* o = out + (int64_t)blockIdx.y * slice_stride;
  constexpr int U = 4;  // rows in flight
  for (int r0 = 0; r0 < RPW; r0 += U) {
    uint4 w[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = min(nbase + r0 + u, N - 1);
      w[u] = kv ? ld_stream(Wq + (int64_t)n * (K / 2) + k0 / 2) : make_uint4(0, 0, 0, 0);
      sc[u] = kv ? half_bits_to_float(Ws[(int64_t)n * G + g]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      float acc[MM];
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[m] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t a4[4];
        w4_to_bf16_biased(wd[c], a4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v2bf a = __builtin_bit_cast(v2bf, a4[i]);
#pragma unroll
          for (int m = 0; m < MM; ++m)
            acc[m] = __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(v2bf, xp[m][c * 4 + i]),
                                                     acc[m], false);
        }
      }
      const int n = nbase + r0 + u;
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const float v = wave_sum(sc[u] * fmaf(-kW4Bias, xsl[m], acc[m]));
        if (lane == 0 && n < N) o[(int64_t)m * N + n] = v;
      }
    }
  }
}

// Fixed-order reduction of S k-slice partials; optionally times Xs[m].
__global__ __launch_bounds__(256) void reduce_slices_kernel(const float* __restrict__ part, int S,
                                                            int64_t MN, int64_t N,
                                                            const float* __restrict__ Xs,
                                                            float* __restrict__ Y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += (int64_t)gridDim.x * 256) {
    float s = part[i];
    for (int t = 1; t < S; ++t) s += part[(int64_t)t * MN + i];
    if (Xs != nullptr) s = Xs[i / N] * s;
    Y[i] = s;
  }
}

// ---------------------------------------------------------------- planning
// Split-K depends on (N, K) only: an output row's operation order is the
// same for every M within one family.
struct SkinnyPlan {
  int S, gps, MB, mchunks;
};
constexpr int kSkinnyNB = 1;

SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K) {
  SkinnyPlan p;
  const int64_t G = K / kGroup;
  const int64_t ntiles = cdiv(N, 64 * kSkinnyNB);
  int64_t S = cdiv(512, ntiles);
  if (S < 1) S = 1;
  if (S > G) S = G;
  p.gps = (int)cdiv(G, S);
  p.S = (int)cdiv(G, p.gps);
  p.MB = (int)(M >= 64 ? 4 : cdiv(M, 16));
  p.mchunks = (int)cdiv(M, 16 * p.MB);
  return p;
}

struct GemvPlan {
  int S;
};
constexpr int kGemvRPW = 16;
GemvPlan plan_gemv(int64_t K) { return GemvPlan{(int)cdiv(K, 2048)}; }

int w4a16_pick(int variant, int64_t M) {
  if (variant != QSPEC_GEMM_AUTO) return variant;
  return M <= 2 ? QSPEC_GEMM_GEMV : QSPEC_GEMM_SKINNY;
}
int w4a4_pick(int variant, int64_t /*M*/) {
  if (variant != QSPEC_GEMM_AUTO) return variant;
  return QSPEC_GEMM_SKINNY;
}

hipError_t reduce(const float* part, int S, int64_t M, int64_t N, const float* Xs, float* Y,
                  hipStream_t s) {
  const int64_t MN = M * N;
  int64_t blocks = cdiv(MN, 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(reduce_slices_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, S, MN,
                     N, Xs, Y);
  return hipGetLastError();
}

}  // namespace

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const SkinnyPlan p = plan_skinny(M, N, K);
  const GemvPlan q = plan_gemv(K);
  size_t a = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  size_t b = q.S > 1 ? (size_t)q.S * std::min<int64_t>(M, 4) * N * sizeof(float) : 0;
  return std::max(a, b);
}

hipError_t launch_w4a16(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                        int64_t N, int64_t K, int variant, float* Y, void* ws, hipStream_t s) {
  const int v = w4a16_pick(variant, M);
  if (v == QSPEC_GEMM_GEMV) {
    const GemvPlan q = plan_gemv(K);
    // rows of X in chunks of up to 4
    for (int64_t m0 = 0; m0 < M; m0 += 4) {
      const int mm = (int)std::min<int64_t>(4, M - m0);
      float* out = q.S > 1 ? static_cast<float*>(ws) : Y + m0 * N;
      const int64_t stride = (int64_t)mm * N;
      dim3 grid((unsigned)cdiv(N, 4 * kGemvRPW), (unsigned)q.S);
      const uint16_t* Xm = X + m0 * K;
      switch (mm) {
        case 1: hipLaunchKernelGGL((w4a16_gemv_kernel<1, kGemvRPW>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        case 2: hipLaunchKernelGGL((w4a16_gemv_kernel<2, kGemvRPW>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        case 3: hipLaunchKernelGGL((w4a16_gemv_kernel<3, kGemvRPW>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        default: hipLaunchKernelGGL((w4a16_gemv_kernel<4, kGemvRPW>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (q.S > 1) {
        e = reduce(out, q.S, mm, N, nullptr, Y + m0 * N, s);
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }
  // SKINNY (TILED shares it until the prefill family lands)
  const SkinnyPlan p = plan_skinny(M, N, K);
  float* out = p.S > 1 ? static_cast<float*>(ws) : Y;
  const int64_t stride = M * N;
  dim3 grid((unsigned)cdiv(N, 64 * kSkinnyNB), (unsigned)p.S, (unsigned)p.mchunks);
  switch (p.MB) {
    case 1: hipLaunchKernelGGL((w4a16_skinny_kernel<kSkinnyNB, 1, 4>), grid, dim3(256), 0, s, X, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride); break;
    case 2: hipLaunchKernelGGL((w4a16_skinny_kernel<kSkinnyNB, 2, 2>), grid, dim3(256), 0, s, X, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride); break;
    case 3: hipLaunchKernelGGL((w4a16_skinny_kernel<kSkinnyNB, 3, 1>), grid, dim3(256), 0, s, X, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride); break;
    default: hipLaunchKernelGGL((w4a16_skinny_kernel<kSkinnyNB, 4, 1>), grid, dim3(256), 0, s, X, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.S > 1) return reduce(out, p.S, M, N, nullptr, Y, s);
  return hipSuccess;
}

size_t w4a4_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const SkinnyPlan p = plan_skinny(M, N, K);
  return p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
}

hipError_t launch_w4a4(const uint8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, int32_t* P,
                       void* ws, hipStream_t s) {
  (void)w4a4_pick(variant, M);
  const SkinnyPlan p = plan_skinny(M, N, K);
  float* out = p.S > 1 ? static_cast<float*>(ws) : Y;
  const int apply = p.S > 1 ? 0 : 1;
  const int64_t stride = M * N;
  dim3 grid((unsigned)cdiv(N, 64 * kSkinnyNB), (unsigned)p.S, (unsigned)p.mchunks);
  switch (p.MB) {
    case 1: hipLaunchKernelGGL((w4a4_skinny_kernel<kSkinnyNB, 1, 4>), grid, dim3(256), 0, s, Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride, P, apply); break;
    case 2: hipLaunchKernelGGL((w4a4_skinny_kernel<kSkinnyNB, 2, 2>), grid, dim3(256), 0, s, Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride, P, apply); break;
    case 3: hipLaunchKernelGGL((w4a4_skinny_kernel<kSkinnyNB, 3, 2>), grid, dim3(256), 0, s, Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride, P, apply); break;
    default: hipLaunchKernelGGL((w4a4_skinny_kernel<kSkinnyNB, 4, 2>), grid, dim3(256), 0, s, Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, p.gps, out, stride, P, apply); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.S > 1) return reduce(out, p.S, M, N, Xs, Y, s);
  return hipSuccess;
}

}  // namespace qspec
