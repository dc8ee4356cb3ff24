// Ceiling probes: what this GPU sustains for the two resources the hot path
// is bound by, measured with the same kinds of instructions the kernels use.
//   * HBM read: every byte of a buffer read once with 16-byte non-temporal
//     loads, several loads in flight per lane (the decode GEMMs' weight
//     stream is this access with arithmetic on top);
//   * MFMA: independent chains of v_mfma_i32_16x16x64_i8 (the drafter's
//     instruction) or v_mfma_f32_16x16x32_bf16 (the verifier's), enough per
//     wavefront to keep the matrix pipe busy;
//   * an empty kernel, for the cost of one more launch in a graph.
// The results are the denominators a measured fraction is quoted against,
// next to the published peaks; nothing here is on the hot path.
#include "launch.h"

namespace qspec {
namespace {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

// Each thread reads 16-byte units u = base + (i * grid_threads) for the
// units of the buffer, UNR at a time (all issued before any is used).  The
// XOR of everything read is written only where it equals `never` (the host
// passes a value the data cannot give), so the loads stay live and nothing
// is stored.
template <int UNR>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4p* __restrict__ buf,
                                                         int64_t units, uint32_t never,
                                                         uint32_t* __restrict__ sink) {
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  int64_t u = t;
  for (; u + (UNR - 1) * nthr < units; u += UNR * nthr) {
    u32x4p v[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) v[i] = __builtin_nontemporal_load(buf + u + i * nthr);
#pragma unroll
    for (int i = 0; i < UNR; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  for (; u < units; u += nthr) {
    const u32x4p v = __builtin_nontemporal_load(buf + u);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[t & 255] = acc;
}

// Eight independent accumulators per wavefront, `iters` rounds of one MFMA
// each (four rounds per loop trip); eight named chains rather than an array,
// so every accumulator keeps its registers from round to round.
#define QSPEC_PROBE_ROUND(F) \
  c0 = F(a, b, c0, 0, 0, 0); c1 = F(a, b, c1, 0, 0, 0); c2 = F(a, b, c2, 0, 0, 0); \
  c3 = F(a, b, c3, 0, 0, 0); c4 = F(a, b, c4, 0, 0, 0); c5 = F(a, b, c5, 0, 0, 0); \
  c6 = F(a, b, c6, 0, 0, 0); c7 = F(a, b, c7, 0, 0, 0);

__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int iters, float never,
                                                            float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane + 1, lane + 2, lane + 3};
  const v4i b = {lane ^ 5, lane ^ 7, lane ^ 9, lane ^ 11};
  v4i c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; it += 4) {
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_i32_16x16x64_i8)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_i32_16x16x64_i8)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_i32_16x16x64_i8)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_i32_16x16x64_i8)
  }
  const v4i t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const int s = t[0] + t[1] + t[2] + t[3];
  if ((float)s == never) sink[threadIdx.x] = (float)s;
}

__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float never,
                                                              float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const uint32_t w = 0x3F803F80u + (uint32_t)lane;  // small bf16 values
  const u4 ta = {w, w + 1, w + 2, w + 3}, tb = {w ^ 1, w ^ 2, w ^ 3, w ^ 4};
  const v8bf a = __builtin_bit_cast(v8bf, ta), b = __builtin_bit_cast(v8bf, tb);
  v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int it = 0; it < iters; it += 4) {
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_f32_16x16x32_bf16)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_f32_16x16x32_bf16)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_f32_16x16x32_bf16)
    QSPEC_PROBE_ROUND(__builtin_amdgcn_mfma_f32_16x16x32_bf16)
  }
  const v4f t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = t[0] + t[1] + t[2] + t[3];
  if (s == never) sink[threadIdx.x] = s;
}
#undef QSPEC_PROBE_ROUND

__global__ void probe_empty_kernel() {}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t bytes, int blocks, int unroll,
                             uint32_t* sink, hipStream_t s) {
  const int64_t units = bytes / 16;
  const u32x4p* p = static_cast<const u32x4p*>(buf);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(probe_read_kernel<1>, dim3(blocks), dim3(256), 0, s, p, units, 0x5A5A5A5Au, sink); break;
    case 2: hipLaunchKernelGGL(probe_read_kernel<2>, dim3(blocks), dim3(256), 0, s, p, units, 0x5A5A5A5Au, sink); break;
    case 4: hipLaunchKernelGGL(probe_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, units, 0x5A5A5A5Au, sink); break;
    case 8: hipLaunchKernelGGL(probe_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, units, 0x5A5A5A5Au, sink); break;
    default: hipLaunchKernelGGL(probe_read_kernel<16>, dim3(blocks), dim3(256), 0, s, p, units, 0x5A5A5A5Au, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* sink, hipStream_t s) {
  // iters rounds to a multiple of four (the loop's trip)
  if (kind == 0)
    hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3(blocks), dim3(256), 0, s, iters, -1.5f, sink);
  else
    hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(blocks), dim3(256), 0, s, iters, -1.5f, sink);
  return hipGetLastError();
}

hipError_t launch_probe_empty(hipStream_t s) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace qspec
