// The dual-mode linear layer: W4A16 (verifier) and W4A4 (drafter) GEMMs over
// the one shared packed INT4 weight buffer, and a W4A8 middle tier on the
// same buffer (8-bit activation codes; the skinny and stream families).
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
//   W4A8:  the same with 8-bit activation codes
//
// gfx950 design
//  * Codes are widened in registers only; the shared buffer stays 4-bit.
//    W4A16 turns a nibble into the bf16 of 136 + q with one AND-XOR
//    (exact), runs v_mfma_f32_16x16x32_bf16 and removes the bias in fp32
//    before the scale: with a second MFMA chain whose A operand is the
//    constant -136 (skinny, stream and prefill kernels; the prefill kernel
//    runs it once per activation block and seeds every weight block's
//    accumulator with it) or with the group sum of x (GEMV).  W4A4 turns
//    nibbles into int8 holding 16 q (a mask, and a shift for the low
//    nibbles; exact) and runs v_mfma_i32_16x16x64_i8; the int32 group
//    partial is 256 P exactly (16 P for W4A8, whose codes are staged as
//    they are, in the same k order).
//  * Outputs are fp32, or, for the W4A4 drafter on request, the bf16
//    rounding (to nearest even) of that fp32 value.
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
#include <atomic>
#include <type_traits>

#include "launch.h"

// Tile parameters (activation chunk CH, weight ring depth PD) per m-block
// count; measured on MI355X.  Overridable at build time for tuning sweeps.
#ifndef QSPEC_SK_A1
#define QSPEC_SK_A1 4, 4   // W4A4,  M <= 16: CH, PD
#endif
#ifndef QSPEC_SK_A2
#define QSPEC_SK_A2 4, 4
#endif
#ifndef QSPEC_SK_A3
#define QSPEC_SK_A3 2, 4
#endif
#ifndef QSPEC_SK_A4
#define QSPEC_SK_A4 2, 4
#endif
#ifndef QSPEC_SK_B1
#define QSPEC_SK_B1 4, 4   // W4A16, M <= 16: CH, PD
#endif
#ifndef QSPEC_SK_B2
#define QSPEC_SK_B2 2, 4
#endif
#ifndef QSPEC_SK_B3
#define QSPEC_SK_B3 2, 4
#endif
#ifndef QSPEC_SK_B4
#define QSPEC_SK_B4 1, 4
#endif
#ifndef QSPEC_SK_NB16
#define QSPEC_SK_NB16 1    // W4A16, M > 16: 16-row blocks per wavefront
#endif
#ifndef QSPEC_SK_SPLIT_WG
#define QSPEC_SK_SPLIT_WG 128  // k-split until about this many workgroups (a function of N, K)
#endif
#ifndef QSPEC_SK_VBIAS_N
#define QSPEC_SK_VBIAS_N 16384  // W4A16 from this many rows: the bias term from staged group sums
#endif
#ifndef QSPEC_SK_MIN_GPS
#define QSPEC_SK_MIN_GPS 4     // the k-split leaves at least this many groups per slice
#endif
#ifndef QSPEC_SK_BIG_NWV
#define QSPEC_SK_BIG_NWV 4      // wavefronts per workgroup on grids of more than 768 64-row tiles
#endif
#ifndef QSPEC_SK_TARGET_WG
#define QSPEC_SK_TARGET_WG 256  // M <= 16 below this many 64-row tiles: the stream family
#endif

// wavefronts per SIMD the register budget of a skinny instantiation must
// allow (the most that compiles without spills)
constexpr int skinny_wpe(int mode, int mb) {
#ifdef QSPEC_SK_NO_WPE
  return 1;
#else
  return mb <= 2 ? 4 : (mode == 0 && mb == 3) ? 3 : 2;
#endif
}


namespace qspec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// two bf16 -136.0 (0xC308): removes the +136 bias of the widened codes
constexpr uint32_t kNegBiasPair = 0xC308C308u;

// streaming (non-temporal) 16-byte load: weights are read exactly once
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Output of a linear layer: fp32 Yf, or, when a bf16 destination Yb is
// given (the W4A4 drafter's chaining output), the round-to-nearest-even
// bf16 of exactly the fp32 value that would have been stored.  out_store4
// writes the outputs o .. o + 3 of one row (those below nvalid); vec: o is a
// multiple of 4 and all four are valid.
__device__ __forceinline__ void out_store4(float* Yf, uint16_t* Yb, int64_t o, const float (&v)[4],
                                           int nvalid, bool vec) {
  if (Yb != nullptr) {
    if (vec) {
      *reinterpret_cast<uint2*>(Yb + o) =
          make_uint2((uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                     (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < nvalid) Yb[o + r] = f32_to_bf16_rne(v[r]);
    }
  } else {
    if (vec) {
      *reinterpret_cast<float4*>(Yf + o) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < nvalid) Yf[o + r] = v[r];
    }
  }
}

__device__ __forceinline__ void out_store1(float* Yf, uint16_t* Yb, int64_t o, float v) {
  if (Yb != nullptr)
    Yb[o] = f32_to_bf16_rne(v);
  else
    Yf[o] = v;
}

__device__ __forceinline__ v8bf as_v8bf(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 t = {a, b, c, d};
  return __builtin_bit_cast(v8bf, t);
}
__device__ __forceinline__ v4i as_v4i(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4i t = {(int)a, (int)b, (int)c, (int)d};
  return t;
}

// 16 8-bit codes k0 .. k15 (natural order) -> the order the widened 4-bit
// codes take in an MFMA operand (even k of each 8, then odd k), so 8-bit
// activations meet the weights' lo/hi widening in the same k order
__device__ __forceinline__ uint4 i8x16_to_widened_order(const uint4 p) {
  return make_uint4(
      (p.x & 0xFFu) | ((p.x >> 8) & 0xFF00u) | ((p.y & 0xFFu) << 16) | ((p.y << 8) & 0xFF000000u),
      ((p.x >> 8) & 0xFFu) | ((p.x >> 16) & 0xFF00u) | ((p.y << 8) & 0xFF0000u) | (p.y & 0xFF000000u),
      (p.z & 0xFFu) | ((p.z >> 8) & 0xFF00u) | ((p.w & 0xFFu) << 16) | ((p.w << 8) & 0xFF000000u),
      ((p.z >> 8) & 0xFFu) | ((p.z >> 16) & 0xFF00u) | ((p.w << 8) & 0xFF0000u) | (p.w & 0xFF000000u));
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
// MFMA "skinny" family (all three modes): the decode / verify shapes.
//   * a workgroup = 4 wavefronts x 16 weight rows = one 64-row n-tile, one
//     k-slice of the groups, one m-chunk of up to 64 activation rows;
//   * weights go straight from HBM into a register ring PD groups deep (each
//     byte is used by exactly one wavefront; PD-1 groups of compute cover the
//     latency of every load);
//   * activations of the m-chunk are staged through LDS, CH groups at a time,
//     double-buffered, in the MFMA k-slot order, once per workgroup;
//   * split-K (S slices, a function of N and K only) is reduced inside the
//     kernel by the last slice to arrive, in fixed slice order; arrival is
//     counted with one atomic add on a 64-bit counter per tile in the
//     caller's (zero-filled) workspace, which the last slice resets to 0;
//   * block -> (tile, slice) mapping deals the S slices of a tile to one XCD
//     when blocks go round-robin to the 8 XCDs (a locality hint only: the
//     hand-off of partials is correct on any placement).
// ============================================================================
enum { kW4A16 = 0, kW4A4 = 1, kW4A8 = 2 };  // W4A8: skinny and stream families

struct SkinnyArgs {
  const void* X;            // W4A16: bf16 [M][K]; W4A4: packed codes [M][K/2]; W4A8: int8 [M][K]
  const float* Xs;          // W4A4 / W4A8: [M]
  const uint8_t* Wq;
  const uint16_t* Ws;
  float* Y;
  uint16_t* Yb;             // bf16 output instead of Y (W4A4 only), else null
  float* part;              // [S][M][N] when S > 1
  unsigned long long* cnt;  // [T] when S > 1
  int32_t* P;               // W4A4 / W4A8 int32 group partials (optional)
  uint16_t* A;              // W4A16 gate|up in pair order: bf16 SwiGLU [M][N/2] instead of Y
  int M, N, K, S, gps, ntiles, T;
};

// End of a (tile, slice): store Y (times Xs for W4A4) when the k-range is not
// split, else publish this slice's partial and let the last slice to arrive
// reduce all S partials in slice order.  Partials are written and read with
// system-scope atomic accesses (coherent whatever XCD each slice ran on: they
// do not stay in an XCD's L2), the writer waits for its stores to complete
// before the arrival count, and the arrival counter (in the caller's
// workspace, zero at rest) is reset by the last slice.
template <int MODE, int MB, int NB, int NWV, bool SW>
__device__ __forceinline__ void finish_tile(const SkinnyArgs& a, const v4f (&tot)[NB][MB], int t,
                                            int slice, int m0, int n_wg, int n_w, int l16, int lg,
                                            int* s_last_ptr) {
  constexpr int ROWS = 16 * MB;
  constexpr int WROWS = 16 * NB * NWV;
  constexpr int NT = 64 * NWV;
  const int M = a.M, N = a.N;
  int& s_last = *s_last_ptr;
  const bool vec = (N & 3) == 0;
  if (SW && a.S == 1) {
    // W4A16 gate|up with the SwiGLU output (a.A): lanes lg = 0, 1 hold gate
    // columns 0 .. 7 of each 16-row block, lanes lg = 2, 3 (32 lanes on)
    // the matching up columns; after the exchange both lanes of a pair hold
    // its four gate / up values, and each finishes two of them
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = __shfl_xor(tot[nb][mb][r], 32, 64);
        const int m = m0 + mb * 16 + l16;
        const int n16 = n_w + nb * 16;  // the block's first row
        if (m < M && n16 < N) {
          const bool gate_lane = lg < 2;
          const int r0 = gate_lane ? 0 : 2;  // the two pairs this lane finishes
          const int j = n16 / 2 + (lg & 1) * 4 + r0;
          uint16_t h[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float g = gate_lane ? tot[nb][mb][r0 + k] : o[r0 + k];
            const float u = gate_lane ? o[r0 + k] : tot[nb][mb][r0 + k];
            h[k] = swiglu_bf16(g, u);
          }
          *reinterpret_cast<uint32_t*>(a.A + (int64_t)m * (N / 2) + j) =
              (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        }
      }
    return;
  }
  if (a.S == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 16 + l16;
        const int n = n_w + nb * 16 + lg * 4;
        if (m < M && n < N) {
          const float xsc = MODE != kW4A16 ? a.Xs[m] : 1.0f;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = MODE != kW4A16 ? xsc * tot[nb][mb][r] : tot[nb][mb][r];
          out_store4(a.Y, a.Yb, (int64_t)m * N + n, v, N - n, vec);
        }
      }
    return;
  }

  float* o = a.part + (int64_t)slice * M * N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + l16;
      const int n = n_w + nb * 16 + lg * 4;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N)
            __hip_atomic_store(o + (int64_t)m * N + n + r, tot[nb][mb][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  // Each partial store is a relaxed system-scope atomic (written through to
  // memory, never held dirty in an XCD's L2), and every thread waits for its
  // stores to be acknowledged before the barrier that precedes the arrival
  // count; the last slice reads the partials with system-scope atomic loads.
  // A release/acquire fence pair around the count would also write back and
  // invalidate the XCD's whole L2 on every arrival: measured on MI355X, that
  // made the split shapes up to 1.6x slower (the M = 128 verify pass of the
  // batched sweep 197 -> 323 us), so the hand-off relies on the completion
  // wait, as the hardware's own release sequence does for written-through
  // data.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One atomic add per slice: slices that finish together queue at the
  // counter instead of retrying (a compare-and-swap loop costs one memory
  // round trip per competitor, quadratic in S).
  if (threadIdx.x == 0) {
    const unsigned long long old = __hip_atomic_fetch_add(a.cnt + t, 1ull, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_SYSTEM);
    s_last = old + 1ull == (unsigned long long)a.S;
  }
  __syncthreads();
  if (!s_last) return;
  const int64_t MN = (int64_t)M * N;
  if constexpr (SW) {
    // SwiGLU epilogue: each thread takes gate / up pairs (columns c and c + 8
    // of a 16-row block) and sums both over the slices exactly as the
    // element loop below sums one column
    constexpr int PPT = ROWS * WROWS / 2 / NT;
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const int pr = threadIdx.x + NT * e;
      const int m = m0 + pr / (WROWS / 2), qq = pr % (WROWS / 2);
      const int ng = n_wg + (qq >> 3) * 16 + (qq & 7);
      if (m < M && ng < N) {
        const float* sg = a.part + (int64_t)m * N + ng;
        float g = 0.f, u = 0.f;
        for (int s = 0; s < a.S; ++s) {
          const float vg = __hip_atomic_load(sg + s * MN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          const float vu = __hip_atomic_load(sg + 8 + s * MN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          g = s == 0 ? vg : g + vg;
          u = s == 0 ? vu : u + vu;
        }
        a.A[(int64_t)m * (N / 2) + n_wg / 2 + qq] = swiglu_bf16(g, u);
      }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(a.cnt + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return;
  }
  // all partials of an element are requested before any is added (in slice
  // order), 8 slices per batch
  constexpr int EPT = ROWS * WROWS / NT;
  float acc[EPT];
  const float* src[EPT];
  bool ok[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = threadIdx.x + NT * e;
    const int m = m0 + i / WROWS, n = n_wg + i % WROWS;
    ok[e] = m < M && n < N;
    src[e] = a.part + (int64_t)min(m, M - 1) * N + min(n, N - 1);
    acc[e] = 0.f;
  }
  for (int s0 = 0; s0 < a.S; s0 += 8) {
    float v[EPT][8];
#pragma unroll
    for (int e = 0; e < EPT; ++e)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[e][k] = __hip_atomic_load(src[e] + (int64_t)min(s0 + k, a.S - 1) * MN, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
    for (int e = 0; e < EPT; ++e)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < a.S) acc[e] = (s0 + k == 0) ? v[e][k] : acc[e] + v[e][k];
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = threadIdx.x + NT * e;
    const int m = m0 + i / WROWS, n = n_wg + i % WROWS;
    if (ok[e]) out_store1(a.Y, a.Yb, (int64_t)m * N + n, MODE != kW4A16 ? a.Xs[m] * acc[e] : acc[e]);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.cnt + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Straight-line main loop: every global load is issued unconditionally (from
// a clamped, valid address) so the compiler keeps exact load counters and the
// weight ring stays in flight across waits; only the arithmetic of groups past
// the end of the slice is skipped (a branch uniform over the workgroup).
template <int MODE, int MB, int NB, int CH, int PD, bool XOUT, int NWV = 4, bool VB = false>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(skinny_wpe(MODE, MB)))) void skinny_kernel(const SkinnyArgs a) {
  static_assert(PD % CH == 0, "prefetch depth must be a multiple of the chunk");
  // XOUT: the extra output -- the int32 group partials (a.P) in the integer
  // modes, the SwiGLU of gate|up rows in pair order (a.A) in W4A16.
  // VB (W4A16): the bias term from group sums staged with the activations
  // instead of a second MFMA chain
  constexpr int NT = 64 * NWV;             // threads of a workgroup
  constexpr int ROWS = 16 * MB;            // activation rows of an m-chunk
  constexpr int WROWS = 16 * NB * NWV;     // weight rows of a tile (NWV wavefronts x NB blocks of 16)
  constexpr int XSTB = (MODE == kW4A16 ? CH * 256 : CH * 128) + 16;  // LDS row bytes
  constexpr int XCH = MODE == kW4A16 ? ROWS * CH * 16 : MODE == kW4A8 ? ROWS * CH * 8 : ROWS * CH * 4;  // 16-B chunks
  constexpr int XPT = (XCH + NT - 1) / NT;
  constexpr int SPT = (CH * WROWS + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][ROWS * XSTB];
  __shared__ uint16_t wsl[2][CH * WROWS];
  static_assert(!VB || MODE == kW4A16, "the staged bias sums are a W4A16 path");
  // W4A16 with VB: each staged row's activation sum per group (the bias term)
  __shared__ float xsum[2][VB ? ROWS * CH : 1];
  __shared__ int s_last;

  const int b = blockIdx.x;
  const int t = 8 * ((b >> 3) / a.S) + (b & 7);
  const int slice = (b >> 3) % a.S;
  if (t >= a.T) return;  // padding block (uniform)
  const int ntile = t % a.ntiles, mchunk = t / a.ntiles;
  const int G = a.K / kGroup;
  const int g_begin = slice * a.gps, g_end = min(G, g_begin + a.gps);
  const int ng = g_end - g_begin;
  const int nblk = (ng + PD - 1) / PD;  // PD-group blocks, the last may be partial
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n_wg = ntile * WROWS, n_w = n_wg + wave * 16 * NB;
  const int m0 = mchunk * ROWS;
  const int M = a.M, N = a.N, K = a.K;

  // tiled weights: 16 rows x one group = one contiguous 1 KiB tile; lane l's
  // 16 bytes = row l%16, codes 32*(l/16) .. +32 of the group
  const int nrb = (N + 15) / 16;
  const uint8_t* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    wrow[nb] = a.Wq + ((int64_t)min(n_w / 16 + nb, nrb - 1) * G + g_begin) * 1024 + lane * 16;
  auto wload = [&](int nb, int gi) {
    return ld_stream(wrow[nb] + (int64_t)min(gi, ng - 1) * 1024);
  };

  uint4 xr[XPT];
  uint16_t sr[SPT];
  // every load below is unconditional: groups past the slice read clamped
  // (valid) addresses whose results are never used; the activation rows go
  // through a buffer resource over this m-chunk's rows, and rows past M read
  // an out-of-range offset (zeros, no memory access)
  const int xrb = MODE == kW4A16 ? K * 2 : MODE == kW4A8 ? K : K / 2;  // activation row bytes
  const int mrows = min(ROWS, M - m0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(a.X) + (int64_t)m0 * xrb), (short)0,
      mrows * xrb, 0x00020000);
  auto x_load = [&](int c) {
    const int gc = g_begin + c * CH;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = min((int)threadIdx.x + NT * i, XCH - 1);
      uint32_t off;
      if (MODE == kW4A16) {
        const int r = idx / (CH * 16), cc = idx % (CH * 16);
        off = r < mrows ? (uint32_t)(r * xrb + min(gc + (cc >> 4), G - 1) * (kGroup * 2) + (cc & 15) * 16)
                        : 0x80000000u;
      } else if (MODE == kW4A8) {
        const int r = idx / (CH * 8), cc = idx % (CH * 8);
        off = r < mrows ? (uint32_t)(r * xrb + min(gc + (cc >> 3), G - 1) * kGroup + (cc & 7) * 16)
                        : 0x80000000u;
      } else {
        const int r = idx / (CH * 4), cc = idx % (CH * 4);
        off = r < mrows ? (uint32_t)(r * xrb + min(gc + (cc >> 2), G - 1) * 64 + (cc & 3) * 16)
                        : 0x80000000u;
      }
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0);
      xr[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int idx = min((int)threadIdx.x + NT * i, CH * WROWS - 1);
      const int gl = idx / WROWS, rr = idx % WROWS;
      const int rb = min((n_wg + rr) >> 4, nrb - 1);
      sr[i] = a.Ws[((int64_t)rb * G + min(gc + gl, G - 1)) * 16 + (rr & 15)];
    }
  };
  auto x_store = [&](int buf) {
    if constexpr (VB) {
      // each staged row's group sums: a group's 16 chunks of a row sit in
      // the 16 lanes of one DPP row (chunk = lane % 16); eight values per
      // lane by a fixed dot2 chain, then the row's fixed tree -- the same
      // for every M.  All lanes take part (rows past M hold zeros, chunks
      // past the tile repeat the last one and are not stored).
      const v2bf one2 = __builtin_bit_cast(v2bf, 0x3F803F80u);
      float sx[XPT];
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        float s8 = 0.f;
        const uint32_t v[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s8 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, v[e]), one2, s8, false);
        sx[i] = s8;
      }
#pragma unroll
      for (int i = 0; i < XPT; ++i) sx[i] = row16_sum_dpp(sx[i]);
#pragma unroll
      for (int i = 0; i < XPT; ++i) {
        const int idx = threadIdx.x + NT * i;
        if (l16 == 0 && idx < XCH) xsum[buf][(idx / (CH * 16)) * CH + (idx % (CH * 16)) / 16] = sx[i];
      }
    }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + NT * i;
      if (XCH % NT != 0 && idx >= XCH) continue;  // workgroup sizes that do not divide the chunk
      // rows past M are not staged: their LDS rows feed only the MFMA
      // output columns of rows past M, which are never stored
      if (MODE == kW4A16) {
        const int r = idx / (CH * 16), cc = idx % (CH * 16);
        if (r >= mrows) continue;
        const uint32_t v[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        uint32_t p[4];
        bf16x8_interleave(v, p);
        *reinterpret_cast<uint4*>(&xs[buf][r * XSTB + cc * 16]) = make_uint4(p[0], p[1], p[2], p[3]);
      } else if (MODE == kW4A8) {
        // 16 codes k0 .. k15 of the group slot cc & 7, reordered to the order
        // the widened 4-bit path stages (even k of each 8, then odd k), so
        // both modes meet the weights' lo/hi widening in the same k order
        if (idx >= XCH) continue;
        const int r = idx / (CH * 8), cc = idx % (CH * 8);
        if (r >= mrows) continue;
        *reinterpret_cast<uint4*>(&xs[buf][r * XSTB + (cc >> 3) * 128 + (cc & 7) * 16]) =
            i8x16_to_widened_order(xr[i]);
      } else if (idx < XCH) {
        const int r = idx / (CH * 4), cc = idx % (CH * 4);
        if (r >= mrows) continue;
        const uint4 p = xr[i];
        uint8_t* dst = &xs[buf][r * XSTB + (cc >> 2) * 128 + (cc & 3) * 32];
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(w4_lo_x16(p.x), w4_hi_x16(p.x), w4_lo_x16(p.y), w4_hi_x16(p.y));
        *reinterpret_cast<uint4*>(dst + 16) =
            make_uint4(w4_lo_x16(p.z), w4_hi_x16(p.z), w4_lo_x16(p.w), w4_hi_x16(p.w));
      }
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int idx = threadIdx.x + NT * i;
      if (idx < CH * WROWS) wsl[buf][idx] = sr[i];
    }
  };

  v4f tot[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 wr[PD][NB];

  // the weight ring is issued before the first activation chunk is stored,
  // so the weight stream starts at once instead of one L2 round trip later
  x_load(0);
#pragma unroll
  for (int s = 0; s < PD; ++s) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wr[s][nb] = wload(nb, s);
    __builtin_amdgcn_sched_barrier(0);  // slot order, as in the steady state
  }
  x_store(0);
  __syncthreads();
  x_load(1);

  for (int bi = 0; bi < nblk; ++bi) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int gi = bi * PD + s;
      const int gl = s % CH;  // compile-time after unrolling
      const int c = gi / CH;
      const int buf = c & 1;
      if (gi >= ng) {
        // past the end of the slice: nothing to add
      } else if (MODE == kW4A16) {
        // acc = sum x (136 + q) per row; the bias term -136 sum x per m comes
        // from one more MFMA chain with a constant A operand, or with VB
        // from the group sums staged with the activations (one FMA)
        v4f acc[NB][MB], corr[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          corr[mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        const v8bf cneg = as_v8bf(kNegBiasPair, kNegBiasPair, kNegBiasPair, kNegBiasPair);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8bf bv[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            bv[mb] = *reinterpret_cast<const v8bf*>(
                &xs[buf][(mb * 16 + l16) * XSTB + gl * 256 + lg * 64 + j * 16]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint4 w = wr[s][nb];
            const uint32_t wd = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
            uint32_t a4[4];
            w4_to_bf16_biased(wd, a4);
            const v8bf av = as_v8bf(a4[0], a4[1], a4[2], a4[3]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[mb], acc[nb][mb], 0, 0, 0);
          }
          // with one weight block the bias chain runs into the same
          // accumulator; with several it is shared and added per group
          if constexpr (!VB) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              if (NB == 1)
                acc[0][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cneg, bv[mb], acc[0][mb], 0, 0, 0);
              else
                corr[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cneg, bv[mb], corr[mb], 0, 0, 0);
            }
          }
        }
        if constexpr (VB) {
          (void)cneg;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float sx = xsum[buf][(mb * 16 + l16) * CH + gl];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[nb][mb][r] = fmaf(-kW4Bias, sx, acc[nb][mb][r]);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* wp = &wsl[buf][gl * WROWS + wave * 16 * NB + nb * 16 + lg * 4];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              tot[nb][mb][r] = fmaf(half_bits_to_float(wp[r]),
                                    (NB == 1 || VB) ? acc[nb][mb][r] : acc[nb][mb][r] + corr[mb][r],
                                    tot[nb][mb][r]);
        }
      } else {
        v4i acc[NB][MB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v4i bv[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            bv[mb] = *reinterpret_cast<const v4i*>(
                &xs[buf][(mb * 16 + l16) * XSTB + gl * 128 + lg * 32 + j * 16]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint4 w = wr[s][nb];
            const uint32_t p0 = j == 0 ? w.x : w.z, p1 = j == 0 ? w.y : w.w;
            const v4i av = as_v4i(w4_lo_x16(p0), w4_hi_x16(p0), w4_lo_x16(p1), w4_hi_x16(p1));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[nb][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv[mb], acc[nb][mb], 0, 0, 0);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* wp = &wsl[buf][gl * WROWS + wave * 16 * NB + nb * 16 + lg * 4];
          float sc[4];
#pragma unroll
          // / 256 when both operands carry the x16 of the widening, / 16 for
          // 8-bit activation codes
          for (int r = 0; r < 4; ++r) sc[r] = half_bits_to_float(wp[r]) * (MODE == kW4A8 ? 0.0625f : 0.00390625f);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              tot[nb][mb][r] = fmaf(sc[r], (float)acc[nb][mb][r], tot[nb][mb][r]);
            if (XOUT) {
              const int m = m0 + mb * 16 + l16, n = n_w + nb * 16 + lg * 4;
              if (m < M) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < N)
                    a.P[((int64_t)m * N + n + r) * G + g_begin + gi] =
                        acc[nb][mb][r] >> (MODE == kW4A8 ? 4 : 8);
              }
            }
          }
        }
      }
      // refill the slot only after its old value is dead, so the new load can
      // land in the same registers (no copies, no drain at the loop edge)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wr[s][nb] = wload(nb, gi + PD);
      if (gl == CH - 1) {  // end of activation chunk c: publish chunk c+1, fetch c+2
        x_store((c + 1) & 1);
        __syncthreads();
        x_load(c + 2);
      }
    }
  }
  finish_tile<MODE, MB, NB, NWV, MODE == kW4A16 && XOUT>(a, tot, t, slice, m0, n_wg, n_w, l16, lg,
                                                        &s_last);
}

// ============================================================================
// MFMA "tiled" family: the prefill shapes, compute-bound.  One kernel per
// mode, both on the same grid and data flow:
//   * a workgroup = WN wavefronts side by side in N; each wavefront owns 64
//     rows of N (4 weight blocks of 16) for all the workgroup's rows of M;
//   * weight tiles (flat 1 KiB per 16 rows x group, exactly one MFMA operand
//     per lane) and their scales go from global memory straight into a
//     register ring, PD groups ahead, and are widened in registers: every
//     weight byte is read by one wavefront of a workgroup;
//   * the activation group slice is staged in LDS once per workgroup,
//     double-buffered, one barrier per group;
//   * block order: n-tiles are dealt round-robin to the 8 XCDs and each XCD
//     walks all m-tiles of an n-tile in a row, so a weight tile is fetched
//     from HBM about once per XCD and then served by that XCD's L2 (the W4A4
//     kernel walks the same order with a persistent grid, several tiles
//     per workgroup);
//   * all loads go through buffer resources with the group as a uniform
//     offset.
// ============================================================================
struct TiledArgs {
  const void* X;
  const float* Xs;
  const uint8_t* Wq;
  const uint16_t* Ws;
  float* Y;
  uint16_t* Yb;  // bf16 output instead of Y (W4A4 only), else null
  int32_t* P;    // W4A4 int32 group partials [M][N][K/128] (optional)
  int M, N, K, ntn, ntm;
};

// ----------------------------------------------------------------------------
// W4A4 prefill kernel, register-direct weights: WN wavefronts, each owning a
// 64 (n) x 64 (m) output block, so a workgroup computes BN = 64 WN rows of N
// for 64 rows of M.
//   * weights: the 1 KiB tile of (16-row block, group) is exactly one MFMA
//     A-operand pair (lane l = slot l), so each wavefront loads its four
//     tiles per group straight into registers (PD groups ahead) and widens
//     them there; no LDS for the larger operand;
//   * activations: the 64 x 64-byte group slice is staged in LDS once per
//     workgroup, widened to int8 (16 q), double-buffered, one barrier per
//     group;
//   * persistent grid (two workgroups per CU): each workgroup walks its
//     tiles one after the other with the group pipeline running on across
//     tile boundaries, so a finished tile's fp32 stores drain while the next
//     tile's loads and MFMAs proceed (3 % faster than one tile per
//     workgroup; the stores of a wave of tiles otherwise all land at once);
//   * epilogue without an int -> float conversion (with one, convert then
//     FMA, the kernel runs at a third of this rate on MI355X): the first MFMA
//     of each group starts from the integer bit pattern of B = 1.5 * 2^23, so
//     its int32 result bits(B) + P' (P' = 256 P, the partial of the 16 q
//     operands, |P'| <= 2^21) read as fp32 is exactly B + P', and one FMA per
//     output and group adds s (B + P') to the running sum (s = scale / 256).
//     After every CH groups the sum drops B times the sum of those CH
//     scales, which the thread staging that column accumulates as it stages
//     the scales.  P stays exact; what changes is that each FMA rounds at the
//     magnitude the bias gives the running sum, up to CH B s: at most
//     CH * scale / 341 per FMA, i.e. CH / 341 of one unit of P.
// ----------------------------------------------------------------------------
#ifndef QSPEC_PF_SHAPE
#define QSPEC_PF_SHAPE 4, 2, 4  // WN, PD (weight ring depth), CH (groups per bias chunk)
#endif
#ifndef QSPEC_PF_RST
#define QSPEC_PF_RST 144  // LDS row stride of the widened activation slice (bytes)
#endif

template <int WN, int PD, int CH, bool BOUT, bool WITHP>
__global__ __launch_bounds__(64 * WN, 2) void w4a4_prefill_kernel(const TiledArgs a) {
  constexpr int BN = 64 * WN, BM = 64, NT = 64 * WN, RST = QSPEC_PF_RST;
  constexpr int BCH = BM * 4;                          // 16-byte activation chunks per group
  constexpr int BC = BCH >= NT ? BCH / NT : 1;         // chunks per staging thread
  static_assert(BCH % NT == 0 || NT % BCH == 0, "staging split");
  constexpr int U = PD;                                // unroll: ring slot and LDS buffer static
  static_assert(PD == 2 || PD == 4, "ring depth");
  constexpr uint32_t kBiasBits = 0x4B400000u;          // 1.5 * 2^23
  constexpr float kBias = 12582912.0f;
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BM * RST];
  __shared__ __attribute__((aligned(16))) float Ss[2][BN];
  __shared__ __attribute__((aligned(16))) float Cs[2][BN];

  const int M = a.M, N = a.N, K = a.K;
  const int G = K / kGroup;
  const int ntn = a.ntn, ntm = a.ntm;
  const int P = gridDim.x;  // a multiple of 8
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int l16 = lane & 15, lg = lane >> 4;
  const int nrb = (N + 15) / 16;

  // Tiles of this workgroup: tile k is tau = blockIdx.x + k P of the
  // XCD-dealt order (tau & 7 stays this block's XCD; each XCD walks the m-tiles
  // of an n-tile together).  nt does not decrease with k, so the valid tiles
  // (nt < ntn) are the first nk.
  const int ntau = 8 * ((ntn + 7) / 8) * ntm;
  auto tile_nt = [&](int kk) {
    const int tau = (int)blockIdx.x + kk * P;
    return 8 * ((tau >> 3) / ntm) + (tau & 7);
  };
  auto tile_m0 = [&](int kk) {
    const int tau = (int)blockIdx.x + kk * P;
    return ((tau >> 3) % ntm) * BM;
  };
  int nk = 0;
  while ((int)blockIdx.x + nk * P < ntau && tile_nt(nk) < ntn) ++nk;
  if (nk == 0) return;  // uniform
  const int S = nk * G;  // group steps of this workgroup, tile after tile

  // Three streams walk the steps (tile k, group g) in order, each with its
  // own position: the weight ring (PD steps ahead of the MFMAs), the
  // activation and scale loads (3 ahead) and the compute.  Buffer resources
  // start at the current tile of their stream, so offsets stay 32-bit; past
  // the last step a stream re-reads its last step (never used).
  // weights: row blocks rbw .. rbw + 3 of the tile (clamped), slot `lane`
  __amdgpu_buffer_rsrc_t wres;
  int woff[4];  // wavefront-uniform block offsets; the lane's slot is lane * 16
  const uint32_t wlane = (uint32_t)lane * 16;
  int wk = 0, wg = 0;
  auto w_tile = [&](int kk) {
    const int nt = tile_nt(kk);
    const int rbw = min(nt * (BN / 16) + wn * 4, nrb - 1);
    wres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.Wq) + (int64_t)rbw * G * 1024,
                                             (short)0, min(4, nrb - rbw) * G * 1024, 0x00020000);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      woff[nb] = (min(nt * (BN / 16) + wn * 4 + nb, nrb - 1) - rbw) * G * 1024;
  };
  auto w_advance = [&]() {
    const bool wrap = wg + 1 == G, more = wk + 1 < nk;
    wg = wrap ? (more ? 0 : G - 1) : wg + 1;
    if (wrap && more) {  // uniform
      wk = wk + 1;
      w_tile(wk);
    }
  };
  auto wload = [&](int nb) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wres, wlane, woff[nb] + wg * 1024, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  // activations: chunk c = (row (c % 16) + 16 (c / 64), 16 packed bytes
  // (c / 16) % 4 of the group): 16 consecutive lanes write 16 rows of one
  // column of chunks, the pattern of the MFMA operand reads; scales: thread
  // tid stages column tid of the tile
  const bool bstager = tid < BCH;
  __amdgpu_buffer_rsrc_t xres, sres;
  uint32_t boff[BC];
  int bdst[BC];
  uint32_t soff;
  int xk = 0, xg = 0;
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = min(tid + NT * i, BCH - 1);
    const int row = (c & 15) | ((c >> 6) << 4), part = (c >> 4) & 3;
    bdst[i] = row * RST + part * 32;
  }
  auto x_tile = [&](int kk) {
    const int nt = tile_nt(kk), m0 = tile_m0(kk);
    xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.X)) + (int64_t)m0 * (K / 2), (short)0,
        min(BM, M - m0) * (K / 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int c = min(tid + NT * i, BCH - 1);
      const int row = (c & 15) | ((c >> 6) << 4), part = (c >> 4) & 3;
      boff[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * (K / 2) + part * 16);
    }
    const int scol = nt * BN + tid;
    const int srb0 = min(nt * (BN / 16), nrb - 1);
    sres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.Ws) + (int64_t)srb0 * G * 16,
                                             (short)0, min(BN / 16, nrb - srb0) * G * 32, 0x00020000);
    soff = (uint32_t)(((min(scol >> 4, nrb - 1) - srb0) * G * 16 + (scol & 15)) * 2);
  };
  auto x_advance = [&]() {
    const bool wrap = xg + 1 == G, more = xk + 1 < nk;
    xg = wrap ? (more ? 0 : G - 1) : xg + 1;
    if (wrap && more) {  // uniform
      xk = xk + 1;
      x_tile(xk);
    }
  };
  struct BStage {
    uint4 x[BC];
    uint16_t s;
  };
  auto bload = [&](BStage& st) {
    if (bstager) {
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xres, boff[i], xg * 64, 0);
        st.x[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
    st.s = __builtin_amdgcn_raw_buffer_load_b16(sres, soff, xg * 32, 0);
    x_advance();
  };
  float ssum = 0.f;  // this thread's column: sum of the scales of the open chunk
  // stage a step whose group index in its tile is gs
  auto bstore = [&](const BStage& st, int buf, int gs) {
    if (bstager) {
#pragma unroll
      for (int i = 0; i < BC; ++i) {
        const uint4 p = st.x[i];
        uint8_t* d = &Bs[buf][bdst[i]];
        *reinterpret_cast<uint4*>(d) =
            make_uint4(w4_lo_x16(p.x), w4_hi_x16(p.x), w4_lo_x16(p.y), w4_hi_x16(p.y));
        *reinterpret_cast<uint4*>(d + 16) =
            make_uint4(w4_lo_x16(p.z), w4_hi_x16(p.z), w4_lo_x16(p.w), w4_hi_x16(p.w));
      }
    }
    const float sv = half_bits_to_float(st.s) * 0.00390625f;  // / 256 (both operands are 16 q)
    Ss[buf][tid] = sv;
    ssum += sv;
    if (gs % CH == CH - 1 || gs == G - 1) {  // uniform: the chunk closes with group gs
      Cs[buf][tid] = kBias * ssum;
      ssum = 0.f;
    }
  };

  v4f tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i cbias = {(int)kBiasBits, (int)kBiasBits, (int)kBiasBits, (int)kBiasBits};

  w_tile(0);
  x_tile(0);
  uint4 ring[PD][4];
#pragma unroll
  for (int i = 0; i < PD; ++i) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) ring[i][nb] = wload(nb);
    w_advance();
  }
  BStage bst[2];
  bload(bst[0]);  // step 0
  bload(bst[1]);  // step 1
  bstore(bst[0], 0, 0);
  bload(bst[0]);  // step 2
  __syncthreads();

  int ck = 0, cg = 0;  // the compute stream's tile and group
  const bool vec = (N & 3) == 0;
  // one group step; u = s mod U fixes the ring slot and the LDS buffer at
  // compile time
  auto step = [&](auto uc, int s) {
    constexpr int u = decltype(uc)::value;
    const int buf = u & 1;
    const uint8_t* Bb = &Bs[buf][l16 * RST + lg * 32];
    v4i bf[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      bf[mb][0] = *reinterpret_cast<const v4i*>(Bb + mb * 16 * RST);
      bf[mb][1] = *reinterpret_cast<const v4i*>(Bb + mb * 16 * RST + 16);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // this step's weights of block nb, widened; the ring slot then takes
      // the weight stream's next step
      const uint4 p = ring[u % PD][nb];
      const v4i a0 = {(int)w4_lo_x16(p.x), (int)w4_hi_x16(p.x), (int)w4_lo_x16(p.y), (int)w4_hi_x16(p.y)};
      const v4i a1 = {(int)w4_lo_x16(p.z), (int)w4_hi_x16(p.z), (int)w4_lo_x16(p.w), (int)w4_hi_x16(p.w)};
      ring[u % PD][nb] = wload(nb);
      const float4 sc = *reinterpret_cast<const float4*>(&Ss[buf][wn * 64 + nb * 16 + lg * 4]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bf[mb][0], cbias, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bf[mb][1], acc, 0, 0, 0);
        if constexpr (WITHP) {
          // the same accumulator, as integers: bits(B) + 256 P exactly
          const int m = tile_m0(ck) + mb * 16 + l16;
          const int n = tile_nt(ck) * BN + wn * 64 + nb * 16 + lg * 4;
          if (m < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) a.P[((int64_t)m * N + n + r) * G + cg] = (acc[r] - (int)kBiasBits) >> 8;
          }
        }
        tot[nb][mb][0] = fmaf(sc.x, __int_as_float(acc[0]), tot[nb][mb][0]);
        tot[nb][mb][1] = fmaf(sc.y, __int_as_float(acc[1]), tot[nb][mb][1]);
        tot[nb][mb][2] = fmaf(sc.z, __int_as_float(acc[2]), tot[nb][mb][2]);
        tot[nb][mb][3] = fmaf(sc.w, __int_as_float(acc[3]), tot[nb][mb][3]);
      }
    }
    w_advance();
    if (cg % CH == CH - 1 || cg == G - 1) {  // uniform: drop the chunk's bias
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float4 cr = *reinterpret_cast<const float4*>(&Cs[buf][wn * 64 + nb * 16 + lg * 4]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          tot[nb][mb][0] -= cr.x;
          tot[nb][mb][1] -= cr.y;
          tot[nb][mb][2] -= cr.z;
          tot[nb][mb][3] -= cr.w;
        }
      }
    }
    if (cg == G - 1) {  // uniform: the tile is complete; its stores drain
                        // while the next tile computes
      const int m0 = tile_m0(ck), n0 = tile_nt(ck) * BN + wn * 64 + lg * 4;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int m = m0 + mb * 16 + l16;
          const int n = n0 + nb * 16;
          if (m < M && n < N) {
            const float xsc = a.Xs[m];
            const float v[4] = {xsc * tot[nb][mb][0], xsc * tot[nb][mb][1], xsc * tot[nb][mb][2],
                                xsc * tot[nb][mb][3]};
            // the output type is a template argument: the stores sit inside
            // the main loop, so only one kind is compiled into it
            out_store4(BOUT ? nullptr : a.Y, BOUT ? a.Yb : nullptr, (int64_t)m * N + n, v, N - n,
                       vec);
          }
          tot[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    {
      const bool last = cg == G - 1;
      ck = ck + (last ? 1 : 0);
      cg = last ? 0 : cg + 1;
    }
    // stage step s + 1 into the other buffer (its readers, step s - 1, all
    // passed the previous barrier), then fetch step s + 3
    if (s + 1 < S) bstore(bst[(u + 1) & 1], buf ^ 1, cg);
    bload(bst[(u + 1) & 1]);
    __syncthreads();
  };
  int s0 = 0;
  for (; s0 + U <= S; s0 += U) {
    step(std::integral_constant<int, 0>{}, s0);
    step(std::integral_constant<int, 1>{}, s0 + 1);
    if constexpr (U > 2) {
      step(std::integral_constant<int, 2>{}, s0 + 2);
      step(std::integral_constant<int, 3>{}, s0 + 3);
    }
  }
  // tail: fewer than U steps left, s0 is a multiple of U
  if (s0 < S) step(std::integral_constant<int, 0>{}, s0);
  if constexpr (U > 2) {
    if (s0 + 1 < S) step(std::integral_constant<int, 1>{}, s0 + 1);
    if (s0 + 2 < S) step(std::integral_constant<int, 2>{}, s0 + 2);
  }
}

#ifndef QSPEC_PF_GRID
#define QSPEC_PF_GRID 512  // persistent workgroups: two per CU
#endif
template <int WN, int PD, int CH>
hipError_t launch_w4a4_prefill(TiledArgs a, hipStream_t s) {
  a.ntn = (int)cdiv(a.N, 64 * WN);
  a.ntm = (int)cdiv(a.M, 64);
  const int64_t tiles = 8 * cdiv(a.ntn, 8) * a.ntm;  // a multiple of 8, as is the grid
  const int64_t grid = std::min<int64_t>(tiles, QSPEC_PF_GRID);
  if (a.Yb != nullptr)
    hipLaunchKernelGGL((w4a4_prefill_kernel<WN, PD, CH, true, false>), dim3((unsigned)grid),
                       dim3(64 * WN), 0, s, a);
  else if (a.P != nullptr)
    hipLaunchKernelGGL((w4a4_prefill_kernel<WN, PD, CH, false, true>), dim3((unsigned)grid),
                       dim3(64 * WN), 0, s, a);
  else
    hipLaunchKernelGGL((w4a4_prefill_kernel<WN, PD, CH, false, false>), dim3((unsigned)grid),
                       dim3(64 * WN), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// W4A16 prefill kernel: the W4A4 prefill kernel's grid and data flow with
// bf16 operands.  WN wavefronts, each owning a 64 (n) x 16 MBW (m) block;
// weights (and their scales) go straight from global memory into a
// register ring and are widened there to bf16 (136 + q); the activation
// group slice (16 MBW rows x 128 bf16 per wavefront row block) is staged
// in LDS once per workgroup, pair-interleaved, double-buffered.  Per group
// and 16-row activation block the -136 chain runs once (4 MFMAs) and seeds
// the accumulator of every weight block, so each output costs one FMA per
// group in the scale epilogue.
// ----------------------------------------------------------------------------
#ifndef QSPEC_PF16_SHAPE
#define QSPEC_PF16_SHAPE 4, 2, 2  // WN, MBW (16-row activation blocks per wavefront), PD
#endif

template <int WN, int MBW, int PD>
__global__ __launch_bounds__(64 * WN, 2) void w4a16_prefill_kernel(const TiledArgs a) {
  constexpr int BN = 64 * WN, BM = 16 * MBW, NT = 64 * WN;
  constexpr int RST = 272;               // LDS row stride: 256 B of bf16 + 16 (odd in 16-B units)
  constexpr int BCH = BM * 16;           // 16-byte chunks of the group slice
  constexpr int BC = BCH / NT;           // chunks per staging thread
  static_assert(BCH % NT == 0 && BC >= 1, "staging split");
  static_assert(PD == 2 || PD == 4, "ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BM * RST];

  const int b = blockIdx.x;
  const int xcd = b & 7, loc = b >> 3;
  const int nt = 8 * (loc / a.ntm) + xcd, mt = loc % a.ntm;
  if (nt >= a.ntn) return;  // padding block (uniform)
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / kGroup;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int l16 = lane & 15, lg = lane >> 4;
  const int nrb = (N + 15) / 16;
  const int m0 = mt * BM;

  // weight tiles and scales of this wavefront: row blocks rbw .. rbw + 3
  const int rbw = min(nt * (BN / 16) + wn * 4, nrb - 1);
  const int nbv = min(4, nrb - rbw);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.Wq) + (int64_t)rbw * G * 1024, (short)0, nbv * G * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.Ws) + (int64_t)rbw * G * 16, (short)0, nbv * G * 32, 0x00020000);
  uint32_t woff[4], soff[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int rel = min(nt * (BN / 16) + wn * 4 + nb, nrb - 1) - rbw;
    woff[nb] = (uint32_t)(rel * G * 1024 + lane * 16);
    soff[nb] = (uint32_t)((rel * G * 16 + lg * 4) * 2);
  }
  // activation staging: chunk c = (row (c % 16) + 16 (c / 256), 16 bytes
  // (c / 16) % 16 of the row's 256-byte group slice): 16 consecutive lanes
  // write 16 rows of one column of chunks, the pattern of the operand reads
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(a.X)) + (int64_t)m0 * K * 2, (short)0,
      min(BM, M - m0) * K * 2, 0x00020000);  // this tile's rows: 32-bit offsets suffice
  uint32_t boff[BC];
  int bdst[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + NT * i;
    const int row = (c & 15) | ((c >> 8) << 4), part = (c >> 4) & 15;
    boff[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * K * 2 + part * 16);
    bdst[i] = row * RST + part * 16;
  }
  struct BStage {
    uint4 x[BC];
  };
  auto bload = [&](BStage& st, int g) {
    const int gg = min(g, G - 1);
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xres, boff[i], gg * 256, 0);
      st.x[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto bstore = [&](const BStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const uint32_t v[4] = {st.x[i].x, st.x[i].y, st.x[i].z, st.x[i].w};
      uint32_t p[4];
      bf16x8_interleave(v, p);
      *reinterpret_cast<uint4*>(&Bs[buf][bdst[i]]) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  };

  v4f tot[4][MBW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) tot[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v8bf cneg = as_v8bf(kNegBiasPair, kNegBiasPair, kNegBiasPair, kNegBiasPair);

  uint4 ring[PD][4];
  uint2 sring[PD][4];
  auto wload = [&](int slot, int g) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[nb], g * 1024, 0);
      ring[slot][nb] = make_uint4(v.x, v.y, v.z, v.w);
      const auto sv = __builtin_amdgcn_raw_buffer_load_b64(sres, soff[nb], g * 32, 0);
      sring[slot][nb] = make_uint2(sv[0], sv[1]);
    }
  };
#pragma unroll
  for (int i = 0; i < PD; ++i) wload(i, min(i, G - 1));
  BStage bst[2];
  bload(bst[0], 0);
  bload(bst[1], 1);
  bstore(bst[0], 0);
  bload(bst[0], 2);
  __syncthreads();

  auto step = [&](auto uc, int g) {
    constexpr int u = decltype(uc)::value;
    const int buf = u & 1;
    const uint8_t* Bb = &Bs[buf][l16 * RST + lg * 64];
    v8bf bv[MBW][4];
    v4f corr[MBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[mb][j] = *reinterpret_cast<const v8bf*>(Bb + mb * 16 * RST + j * 16);
      corr[mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        corr[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cneg, bv[mb][j], corr[mb], 0, 0, 0);
    }
    const int gn = min(g + PD, G - 1);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint4 p = ring[u % PD][nb];
      const uint2 sp = sring[u % PD][nb];
      const uint32_t wv[4] = {p.x, p.y, p.z, p.w};
      v8bf av[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a4[4];
        w4_to_bf16_biased(wv[j], a4);
        av[j] = as_v8bf(a4[0], a4[1], a4[2], a4[3]);
      }
      const float s0 = half_bits_to_float((uint16_t)(sp.x & 0xFFFF));
      const float s1 = half_bits_to_float((uint16_t)(sp.x >> 16));
      const float s2 = half_bits_to_float((uint16_t)(sp.y & 0xFFFF));
      const float s3 = half_bits_to_float((uint16_t)(sp.y >> 16));
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        v4f acc = corr[mb];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], bv[mb][j], acc, 0, 0, 0);
        tot[nb][mb][0] = fmaf(s0, acc[0], tot[nb][mb][0]);
        tot[nb][mb][1] = fmaf(s1, acc[1], tot[nb][mb][1]);
        tot[nb][mb][2] = fmaf(s2, acc[2], tot[nb][mb][2]);
        tot[nb][mb][3] = fmaf(s3, acc[3], tot[nb][mb][3]);
      }
    }
    wload(u % PD, gn);  // the ring slot takes group g + PD
    // stage group g + 1 into the other buffer (its readers, group g - 1,
    // all passed the previous barrier), then fetch group g + 3
    if (g + 1 < G) bstore(bst[(u + 1) & 1], buf ^ 1);
    bload(bst[(u + 1) & 1], g + 3);
    __syncthreads();
  };
  int g = 0;
  for (; g + PD <= G; g += PD) {
    step(std::integral_constant<int, 0>{}, g);
    step(std::integral_constant<int, 1>{}, g + 1);
    if constexpr (PD > 2) {
      step(std::integral_constant<int, 2>{}, g + 2);
      step(std::integral_constant<int, 3>{}, g + 3);
    }
  }
  // tail: fewer than PD groups left, g is a multiple of PD
  if (g < G) step(std::integral_constant<int, 0>{}, g);
  if constexpr (PD > 2) {
    if (g + 1 < G) step(std::integral_constant<int, 1>{}, g + 1);
    if (g + 2 < G) step(std::integral_constant<int, 2>{}, g + 2);
  }

  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int m = m0 + mb * 16 + l16;
      const int n = nt * BN + wn * 64 + nb * 16 + lg * 4;
      if (m < M && n < N) {
        float* dst = a.Y + (int64_t)m * N + n;
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

template <int WN, int MBW, int PD>
hipError_t launch_w4a16_prefill(TiledArgs a, hipStream_t s) {
  a.ntn = (int)cdiv(a.N, 64 * WN);
  a.ntm = (int)cdiv(a.M, 16 * MBW);
  const int64_t blocks = 8 * cdiv(a.ntn, 8) * a.ntm;
  hipLaunchKernelGGL((w4a16_prefill_kernel<WN, MBW, PD>), dim3((unsigned)blocks), dim3(64 * WN), 0,
                     s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_tiled(const void* X, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                        int64_t M, int64_t N, int64_t K, float* Y, uint16_t* Yb, int32_t* P,
                        hipStream_t s) {
  TiledArgs a{X, Xs, Wq, Ws, Y, Yb, P, (int)M, (int)N, (int)K, 0, 0};  // the launcher sets the grid
  if (MODE == kW4A16) return launch_w4a16_prefill<QSPEC_PF16_SHAPE>(a, s);
  return launch_w4a4_prefill<QSPEC_PF_SHAPE>(a, s);
}

// ============================================================================
// "Stream" family (all three modes, M <= 16): the decode shapes, HBM-bound.
//   * a workgroup = nw wavefronts on ONE 16-row weight block; wavefront w
//     takes groups w, w + nw, w + 2 nw, ... (dealt round-robin: at each step
//     the workgroup reads nw adjacent tiles), so the k-split is reduced inside
//     the workgroup (LDS, fixed order) -- no partials leave the chip;
//   * nw depends on (N, K) only: about 4096 wavefronts in flight, at most 16
//     per workgroup, at least 2 groups per wavefront;
//   * weights stream HBM -> registers through a PD-deep ring (one flat 1 KiB
//     tile per wavefront per group); the activation rows and the group scales
//     come from L2 in the same ring stages (every wavefront reads the same few
//     KiB of activations; buffer loads, so lanes of rows >= M fetch nothing);
//     W4A16 with at most 8 (4) rows takes two (one) 16-byte activation loads
//     per lane and group instead of four, and DPP row shifts move each MFMA's
//     fragment into place (stream_xfrag);
//   * the per-group arithmetic is the skinny family's: W4A16 runs
//     v_mfma_f32_16x16x32_bf16 on bf16(136 + q) with a -136 constant-operand
//     chain; W4A4 runs v_mfma_i32_16x16x64_i8 on 16 q; fp32 scale epilogue.
//   A row's operation order does not depend on M (rows past M are clamped
//   duplicates whose outputs are not stored).
// ============================================================================
struct StreamArgs {
  const void* X;    // W4A16: bf16 [M][K]; W4A4: packed codes [M][K/2]; W4A8: int8 [M][K]
  const float* Xs;  // W4A4 / W4A8: [M]
  const uint8_t* Wq;
  const uint16_t* Ws;
  float* Y;
  uint16_t* Yb;  // bf16 output instead of Y (W4A4 only), else null
  int32_t* P;    // W4A4 / W4A8 int32 group partials [M][N][K/128] (optional)
  int M, N, K, nrb;
  uint16_t* A;   // integer modes, gate|up rows in pair order: bf16 SwiGLU [M][N/2] instead of Y
};

// Ring depth (groups) of the stream kernels: measured on MI355X, a shallow
// ring (fewer registers, more resident wavefronts) streams faster than a deep
// one for these shapes.
#ifndef QSPEC_ST_PD4
#define QSPEC_ST_PD4 2   // W4A4
#endif
#ifndef QSPEC_ST_PD16
#define QSPEC_ST_PD16 2  // W4A16
#endif
#ifndef QSPEC_ST_PD16X
#define QSPEC_ST_PD16X 2  // W4A16 with one or two activation loads per group
#endif
#ifndef QSPEC_ST_PDL
#define QSPEC_ST_PDL 1    // ring depth where each wavefront walks at least 6 groups (a long K)
#endif
#ifndef QSPEC_ST_SMALL
#define QSPEC_ST_SMALL 192  // integer modes: grids of at most this many row blocks take PDL
#endif
#ifndef QSPEC_ST_TARGET
#define QSPEC_ST_TARGET 4096  // wavefronts the k-split aims for
#endif
#ifndef QSPEC_ST_WIDE
#define QSPEC_ST_WIDE 512     // integer modes: row blocks from which the ring is three deep
#endif
constexpr int kStreamMaxM = 16;
constexpr int kStreamMaxW = 16;

// One ring stage: the weight tile slot of this lane, its four group scales
// and its activation loads (XL 16-byte loads), all for one group.
template <int MODE, int XL>
struct StreamStage {
  uint4 w;
  uint2 s;
  uint4 x[MODE == kW4A16 ? XL : MODE == kW4A8 ? 2 : 1];
};

// W4A16 activation fragments of few rows.  MFMA j of a group reads, in lane
// (l16, lg), the 16-byte chunk 4 lg + j of activation row l16.  With XL = 4
// every lane loads its own four chunks (one load each, whether or not its
// row exists).  With M <= 8 (XL = 2) load i gives lane (8 t + m, lg) chunk
// 4 lg + 2 i + t of row m, and with M <= 4 (XL = 1) the one load gives lane
// (4 j + m, lg) chunk 4 lg + j of row m; a DPP shift left inside each
// 16-lane row (lane l takes lane l + d) then hands chunk j to lane (m, lg).
// Lanes of rows >= M receive other rows' values there, which only reach
// output columns that are not stored, so each row's operands -- and its
// result -- are bitwise those of XL = 4.
template <int D>
__device__ __forceinline__ uint4 row_shl(uint4 v) {
  constexpr int ctrl = 0x100 + D;  // DPP row_shl:D
  return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, ctrl, 0xF, 0xF, false));
}
template <int XL>
__device__ __forceinline__ uint4 stream_xfrag(const uint4 (&x)[XL], int j) {
  if constexpr (XL == 4) {
    return x[j];
  } else if constexpr (XL == 2) {
    return (j & 1) ? row_shl<8>(x[j >> 1]) : x[j >> 1];
  } else {
    return j == 0 ? x[0] : j == 1 ? row_shl<4>(x[0]) : j == 2 ? row_shl<8>(x[0]) : row_shl<12>(x[0]);
  }
}


template <int MODE, bool WITHP, int PD = (MODE == kW4A16 ? QSPEC_ST_PD16 : QSPEC_ST_PD4),
          bool SW = false, int XL = 4>
__global__ __launch_bounds__(1024) void stream_kernel(const StreamArgs a) {
  static_assert(MODE == kW4A16 || XL == 4, "few-row activation loads are a W4A16 path");
  static_assert(!(WITHP && MODE == kW4A16), "the int32 partials output is an integer-mode path");
  extern __shared__ __attribute__((aligned(16))) float red_[];  // [nw][64][4] when nw > 1
  float(*red)[64][4] = reinterpret_cast<float(*)[64][4]>(red_);
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int rb = blockIdx.x;
  const int M = a.M, K = a.K, G = K / kGroup;
  // groups dealt round-robin: wavefront w takes groups w, w + nw, w + 2 nw,
  // ... (local index i -> group w + nw i), so at each step the workgroup's
  // loads cover nw adjacent tiles; gl clamps the local index
  const int g0 = 0, g1 = w < G ? (G - 1 - w) / nw + 1 : 0;
  const int gl = max(0, g1 - 1);

  const uint8_t* wt = a.Wq + (int64_t)rb * G * 1024 + lane * 16;
  const uint16_t* sc = a.Ws + (int64_t)rb * G * 16 + lg * 4;
  // activation rows through a buffer resource: lanes of rows >= M read an
  // out-of-range offset, which returns zeros without a memory access
  const int xrow_bytes = MODE == kW4A16 ? K * 2 : MODE == kW4A8 ? K : K / 2;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.X), (short)0, M * xrow_bytes, 0x00020000);
  // the row this lane loads and the chunk offset of its first load (W4A16:
  // see stream_xfrag; XL = 4 and the integer modes: row l16)
  const int xr = XL == 4 ? l16 : XL == 2 ? (l16 & 7) : (l16 & 3);
  const int xc = XL == 4 ? 0 : XL == 2 ? (l16 >> 3) : (l16 >> 2);
  const uint32_t xoff0 = (xr < M ? (uint32_t)(xr * xrow_bytes) : 0x80000000u) +
                         (uint32_t)(lg * (MODE == kW4A16 ? 64 : MODE == kW4A8 ? 32 : 16) + 16 * xc);
  // activation bytes per group
  constexpr int xgb = MODE == kW4A16 ? kGroup * 2 : MODE == kW4A8 ? kGroup : kGroup / 2;
  constexpr int nxl = MODE == kW4A16 ? XL : MODE == kW4A8 ? 2 : 1;  // 16-byte loads per stage
  constexpr int xstep = MODE == kW4A16 ? 64 / XL : 16;               // bytes between them

  auto load = [&](StreamStage<MODE, XL>& st, int g) {
    const int gg = min(w + nw * min(g, gl), G - 1);
    st.w = ld_stream(wt + (int64_t)gg * 1024);
    st.s = *reinterpret_cast<const uint2*>(sc + (int64_t)gg * 16);
    const uint32_t o = xoff0 + (uint32_t)(gg * xgb);
#pragma unroll
    for (int i = 0; i < nxl; ++i) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xres, o + xstep * i, 0, 0);
      st.x[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };

  v4f tot = {0.f, 0.f, 0.f, 0.f};
  StreamStage<MODE, XL> ring[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) load(ring[i], g0 + i);
  const v8bf negb = as_v8bf(kNegBiasPair, kNegBiasPair, kNegBiasPair, kNegBiasPair);

  // one group from ring stage i, holding this wavefront's local group li
  auto group = [&](int i, int li) {
    const StreamStage<MODE, XL>& st = ring[i];
    const uint32_t s01 = st.s.x, s23 = st.s.y;
    if constexpr (MODE == kW4A16) {
      // bf16(136 + q) x activations, then the -136 chain into the same
      // accumulator: acc = sum_k x (136 + q) - 136 sum_k x
      const uint32_t wv[4] = {st.w.x, st.w.y, st.w.z, st.w.w};
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      v8bf B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t aw[4], xi[4];
        const uint4 xf = stream_xfrag<XL>(st.x, j);
        const uint32_t xw[4] = {xf.x, xf.y, xf.z, xf.w};
        w4_to_bf16_biased(wv[j], aw);
        bf16x8_interleave(xw, xi);
        B[j] = as_v8bf(xi[0], xi[1], xi[2], xi[3]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(aw[0], aw[1], aw[2], aw[3]), B[j],
                                                      acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(negb, B[j], acc, 0, 0, 0);
      tot[0] = fmaf(half_bits_to_float((uint16_t)(s01 & 0xFFFF)), acc[0], tot[0]);
      tot[1] = fmaf(half_bits_to_float((uint16_t)(s01 >> 16)), acc[1], tot[1]);
      tot[2] = fmaf(half_bits_to_float((uint16_t)(s23 & 0xFFFF)), acc[2], tot[2]);
      tot[3] = fmaf(half_bits_to_float((uint16_t)(s23 >> 16)), acc[3], tot[3]);
    } else {
      const uint4 p = st.w;
      const v4i a0 = {(int)w4_lo_x16(p.x), (int)w4_hi_x16(p.x), (int)w4_lo_x16(p.y), (int)w4_hi_x16(p.y)};
      const v4i a1 = {(int)w4_lo_x16(p.z), (int)w4_hi_x16(p.z), (int)w4_lo_x16(p.w), (int)w4_hi_x16(p.w)};
      v4i b0, b1;
      if (MODE == kW4A8) {
        const uint4 x0 = i8x16_to_widened_order(st.x[0]);
        const uint4 x1 = i8x16_to_widened_order(st.x[nxl - 1]);
        b0 = as_v4i(x0.x, x0.y, x0.z, x0.w);
        b1 = as_v4i(x1.x, x1.y, x1.z, x1.w);
      } else {
        const uint4 x = st.x[0];
        b0 = as_v4i(w4_lo_x16(x.x), w4_hi_x16(x.x), w4_lo_x16(x.y), w4_hi_x16(x.y));
        b1 = as_v4i(w4_lo_x16(x.z), w4_hi_x16(x.z), w4_lo_x16(x.w), w4_hi_x16(x.w));
      }
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
      if constexpr (WITHP) {
        // the accumulator is 256 P (both operands x16) or 16 P (8-bit codes)
        const int n = rb * 16 + lg * 4;
        if (l16 < M) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < a.N)
              a.P[((int64_t)l16 * a.N + n + r) * G + w + nw * li] = acc[r] >> (MODE == kW4A8 ? 4 : 8);
        }
      }
      // / 256 when both operands carry the x16 of the widening, / 16 for
      // 8-bit activation codes
      constexpr float f = MODE == kW4A8 ? 0.0625f : 0.00390625f;
      tot[0] = fmaf(half_bits_to_float((uint16_t)(s01 & 0xFFFF)) * f, (float)acc[0], tot[0]);
      tot[1] = fmaf(half_bits_to_float((uint16_t)(s01 >> 16)) * f, (float)acc[1], tot[1]);
      tot[2] = fmaf(half_bits_to_float((uint16_t)(s23 & 0xFFFF)) * f, (float)acc[2], tot[2]);
      tot[3] = fmaf(half_bits_to_float((uint16_t)(s23 >> 16)) * f, (float)acc[3], tot[3]);
    }
  };
  // Full rounds of PD groups carry no condition, so the compiler keeps every
  // ring load in flight across the waits (a conditional use of a ring stage
  // inside the loop made it wait for all outstanding loads each round).
  int gb = g0;
  for (; gb + PD <= g1; gb += PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      group(i, gb + i);
      load(ring[i], gb + i + PD);  // refill this stage, PD groups ahead
      // issue the refill here, before the next group's arithmetic (left to
      // itself the scheduler sinks every refill to the end of the round, so
      // the next round waits for all of them)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < PD - 1; ++i)
    if (gb + i < g1) group(i, gb + i);  // tail: fewer than PD groups

  // per-wavefront sums -> one sum per output, in wavefront order
  if (nw > 1) {
    *reinterpret_cast<v4f*>(&red[w][lane][0]) = tot;
    __syncthreads();
    if (w != 0) return;
    tot = *reinterpret_cast<const v4f*>(&red[0][lane][0]);
    for (int j = 1; j < nw; ++j) {
      const v4f t = *reinterpret_cast<const v4f*>(&red[j][lane][0]);
      tot[0] += t[0];
      tot[1] += t[1];
      tot[2] += t[2];
      tot[3] += t[3];
    }
  }
  if constexpr (SW) {
    // gate|up rows in pair order, the SwiGLU output (a.A): the same values
    // as the stored Y, paired across the two halves of the wavefront (lanes
    // lg = 0, 1 hold gate columns 0 .. 7 of the block, lanes lg = 2, 3 the
    // matching up columns); each lane of a pair finishes two of its four
    // (gate lanes take outputs 0, 1 of their four, up lanes 2, 3; each
    // sends the two its partner takes)
    const float xs = l16 < M ? a.Xs[l16] : 0.f;
    const float v0 = xs * tot[0], v1 = xs * tot[1], v2 = xs * tot[2], v3 = xs * tot[3];
    const bool gate_lane = lg < 2;
    const float o0 = __shfl_xor(gate_lane ? v2 : v0, 32, 64);
    const float o1 = __shfl_xor(gate_lane ? v3 : v1, 32, 64);
    if (l16 >= M) return;
    const int N = a.N;
    const int j = rb * 8 + (lg & 1) * 4 + (gate_lane ? 0 : 2);
    const uint16_t h0 = swiglu_bf16(gate_lane ? v0 : o0, gate_lane ? o0 : v2);
    const uint16_t h1 = swiglu_bf16(gate_lane ? v1 : o1, gate_lane ? o1 : v3);
    *reinterpret_cast<uint32_t*>(a.A + (int64_t)l16 * (N / 2) + j) = (uint32_t)h0 | ((uint32_t)h1 << 16);
    return;
  }
  if (l16 >= M) return;
  const int n = rb * 16 + lg * 4;
  const int N = a.N;
  if (n >= N) return;
  float xs = 1.f;
  if (MODE != kW4A16) xs = a.Xs[l16];
  const float v[4] = {xs * tot[0], xs * tot[1], xs * tot[2], xs * tot[3]};
  out_store4(a.Y, a.Yb, (int64_t)l16 * N + n, v, N - n, (N & 3) == 0);
}

int stream_waves(int64_t N, int64_t K) {
  const int64_t nrb = cdiv(N, 16), G = K / kGroup;
  int nw = 1;
  while (nw < kStreamMaxW && nrb * nw < QSPEC_ST_TARGET && G / (2 * nw) >= 2) nw *= 2;
  return nw;
}

template <int MODE>
hipError_t launch_stream(const void* X, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                         int64_t M, int64_t N, int64_t K, float* Y, uint16_t* Yb, int32_t* P,
                         hipStream_t s, uint16_t* A = nullptr) {
  StreamArgs a{X, Xs, Wq, Ws, Y, Yb, P, (int)M, (int)N, (int)K, (int)cdiv(N, 16), A};
  const int nw = stream_waves(N, K);
  const size_t lds = nw > 1 ? (size_t)nw * 64 * 4 * sizeof(float) : 0;
  if constexpr (MODE != kW4A16) {
    if (A != nullptr) {  // the SwiGLU output (the gate|up layer of a drafter)
      if (a.nrb >= QSPEC_ST_WIDE)
        hipLaunchKernelGGL((stream_kernel<MODE, false, 3, true>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      else
        hipLaunchKernelGGL((stream_kernel<MODE, false, QSPEC_ST_PD4, true>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
    if (P != nullptr) {
      hipLaunchKernelGGL((stream_kernel<MODE, true>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
    // integer modes on wide grids (at least QSPEC_ST_WIDE row blocks, few
    // groups per wavefront): a three-group ring.  Measured on MI355X at
    // M = 16, K = 2048: N = 11264 7.35 -> 5.72 us.  Where each wavefront
    // walks at least 6 groups (a long K) one group: the Qwen2.5-7B down
    // projection (9 groups per wavefront) at M = 8 / 16 10.0 / 11.0 us
    // against 10.2 / 12.1 (two groups) and 10.6 / 12.7 (three), one box.
    // The narrower shapes with 3-4 groups per wavefront keep two (O at M = 8
    // 4.2 against 4.8 us with one).  The ring depth changes when loads are
    // issued, not what is computed: the rows are bitwise the same either way.
    if (a.nrb >= QSPEC_ST_WIDE) {
      hipLaunchKernelGGL((stream_kernel<MODE, false, 3>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
    // The same one-group ring on grids of at most 192 row blocks (each
    // workgroup alone on its compute unit): on the 2048-wide decoder's
    // drafter layers at M = 16 (128-192 row blocks) 0.1-0.35 us faster per
    // launch in both integer modes (W4A8 QKV 4.81 -> 4.53 us, down 7.2 ->
    // 6.8 us), while the 224-row-block Qwen2.5-7B O projection lost 0.6 us.
    if ((K / kGroup) / nw >= 6 || a.nrb <= QSPEC_ST_SMALL) {
      hipLaunchKernelGGL((stream_kernel<MODE, false, QSPEC_ST_PDL>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (MODE == kW4A16) {
    // few rows: one or two activation loads per group instead of four
    // (stream_xfrag); the rows are bitwise those of the four-load kernel
    if (M <= 4) {
      hipLaunchKernelGGL((stream_kernel<MODE, false, QSPEC_ST_PD16X, false, 1>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
    if (M <= 8) {
      // where each wavefront walks at least 6 groups (a long K), the next
      // group is requested only once the current one is consumed: measured
      // on the down projection (9 groups per wavefront) at M = 5 / 8, one
      // box, 12.3 / 14.5 us against 12.7 / 15.6 (two groups) and 13.2 / 16.9
      // (three); on 3-4 groups per wavefront one group helps QKV (6.7 ->
      // 6.1 us at M = 5) but costs O 0.4-0.8 us, so those keep two
      if ((K / kGroup) / nw >= 6)
        hipLaunchKernelGGL((stream_kernel<MODE, false, QSPEC_ST_PDL, false, 2>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      else
        hipLaunchKernelGGL((stream_kernel<MODE, false, QSPEC_ST_PD16X, false, 2>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((stream_kernel<MODE, false>), dim3((unsigned)a.nrb), dim3(64 * nw), lds, s, a);
  return hipGetLastError();
}

// ============================================================================
// W4A16 GEMV family (M <= 4 per launch): VALU dot products, no MFMA.
//   * a wavefront owns one 16-row block for a k-slice of up to 32 groups;
//     lane l reads the tile slot of row l%16, codes 32*(l/16) .. +32 of each
//     group -- one flat 1 KiB load per wavefront per group;
//   * the activation slice (pair-interleaved to match the codes) and its
//     32-element sums live in LDS, staged once per workgroup;
//   * each lane accumulates ws * (x . (136 + q) - 136 * sum(x)) over its
//     groups with v_dot2_f32_bf16; the four lanes of a row are reduced with
//     two cross-lane steps at the end (the wavefront reduction).
//   grid = (ceil(N / 64), ceil(G / 32))
// ============================================================================
constexpr int kGemvGroups = 32;  // groups per k-slice

template <int MM, int PD>
__global__ __launch_bounds__(256) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ Ws, int N, int K, float* __restrict__ out, int64_t slice_stride) {
  constexpr int KS = kGemvGroups * kGroup;  // k per slice
  __shared__ __attribute__((aligned(16))) uint32_t xs[MM][KS / 2];
  __shared__ float xsum[MM][KS / 32];
  const int G = K / kGroup;
  const int g0 = blockIdx.y * kGemvGroups;
  const int ng = min(G - g0, kGemvGroups);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;

  // stage the activation slice: MM rows x KS/8 chunks of 8
#pragma unroll
  for (int i = 0; i < MM * (KS / 8) / 256; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int m = idx / (KS / 8), c8 = idx % (KS / 8);
    const int k = g0 * kGroup + c8 * 8;
    uint4 v = *reinterpret_cast<const uint4*>(X + (int64_t)m * K + min(k, K - 8));
    if (k >= K) v = make_uint4(0, 0, 0, 0);
    const uint32_t nv[4] = {v.x, v.y, v.z, v.w};
    uint32_t p[4];
    bf16x8_interleave(nv, p);
    *reinterpret_cast<uint4*>(&xs[m][c8 * 4]) = make_uint4(p[0], p[1], p[2], p[3]);
    float s8 = bf16x8_sum(nv);  // four consecutive 8-chunks = one 32-chunk (a DPP quad)
    s8 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s8), 0xB1, 0xF, 0xF, false));
    s8 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s8), 0x4E, 0xF, 0xF, false));
    if ((c8 & 3) == 0) xsum[m][c8 >> 2] = s8;
  }
  __syncthreads();

  const int nrb = (N + 15) / 16;
  const int rb = min(blockIdx.x * 4 + wave, nrb - 1);
  const uint8_t* wrow = Wq + ((int64_t)rb * G + g0) * 1024 + lane * 16;
  const uint16_t* srow = Ws + ((int64_t)rb * G + g0) * 16 + r;  // tiled scales
  auto wload = [&](int gi) { return ld_stream(wrow + (int64_t)min(gi, ng - 1) * 1024); };

  float tot[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) tot[m] = 0.f;
  uint4 wr[PD];
  uint16_t sr[PD];
#pragma unroll
  for (int s = 0; s < PD; ++s) {
    wr[s] = wload(s);
    sr[s] = srow[min(s, ng - 1) * 16];
    __builtin_amdgcn_sched_barrier(0);  // slot order, as in the steady state
  }
  for (int b0 = 0; b0 < ng; b0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int gi = b0 + s;
      const uint4 w = wr[s];
      const float sc = half_bits_to_float(sr[s]);
      if (gi < ng) {
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
        float acc[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[m] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t a4[4];
          w4_to_bf16_biased(wd[j], a4);
#pragma unroll
          for (int m = 0; m < MM; ++m) {
            const uint4 xv = *reinterpret_cast<const uint4*>(&xs[m][gi * 64 + c * 16 + j * 4]);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a4[i]),
                                                       __builtin_bit_cast(v2bf, xw[i]), acc[m],
                                                       false);
          }
        }
#pragma unroll
        for (int m = 0; m < MM; ++m)
          tot[m] = fmaf(sc, fmaf(-kW4Bias, xsum[m][gi * 4 + c], acc[m]), tot[m]);
      }
      wr[s] = wload(gi + PD);
      sr[s] = srow[min(gi + PD, ng - 1) * 16];
    }
  }
  // the four lanes of a row (r, r+16, r+32, r+48) hold disjoint 32-chunks
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    tot[m] += __shfl_xor(tot[m], 16, 64);
    tot[m] += __shfl_xor(tot[m], 32, 64);
  }
  const int nn = rb * 16 + r;
  if (c == 0 && blockIdx.x * 4 + wave < nrb && nn < N) {
    float* o = out + (int64_t)blockIdx.y * slice_stride;
#pragma unroll
    for (int m = 0; m < MM; ++m) o[(int64_t)m * N + nn] = tot[m];
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
  int S, gps, MB, NB, NWV, mchunks, ntiles, T;
  bool VB;  // W4A16: the bias term from staged group sums (a function of N)
  int64_t blocks;
  size_t cnt_bytes, part_bytes;
};

// Wavefronts per workgroup of the one-activation-block kernels (decode
// shapes): when every workgroup is resident at once (up to 768 four-wavefront
// tiles), a CU that holds one workgroup more than another streams that many
// more weight bytes through its own load queue, so take the count whose
// workgroups spread most evenly over the 256 CUs -- fewest wavefronts on the
// busiest CU, ties to the larger workgroup (its activation staging serves
// more weight rows).  Larger grids run in several waves of workgroups and
// balance themselves; they keep four wavefronts (measured on MI355X).
constexpr int kSkinnyNWV[] = {4, 5, 8, 10};
int skinny_nwv(int64_t N, int64_t S, int NB) {
  if (cdiv(N, 64 * NB) * S > 768) return QSPEC_SK_BIG_NWV;
  int best = 4;
  int64_t best_cost = -1;
  for (int nwv : kSkinnyNWV) {
    const int64_t wgs = cdiv(N, 16 * NB * nwv) * S;
    const int64_t cost = cdiv(wgs, 256) * nwv;
    if (best_cost < 0 || cost <= best_cost) {
      best = nwv;
      best_cost = cost;
    }
  }
  return best;
}

// max_tiles: the plan with four-wavefront tiles (the most arrival counters),
// which sizes the workspace for every plan of these (M, N, K)
SkinnyPlan plan_skinny(int mode, int64_t M, int64_t N, int64_t K, bool max_tiles = false) {
  SkinnyPlan p;
  const int64_t G = K / kGroup;
  const int64_t t64 = cdiv(N, 64);  // the split depends on N and K only
  int64_t S = 1;
  if (t64 < QSPEC_SK_SPLIT_WG) {
    S = cdiv(QSPEC_SK_SPLIT_WG, t64);
    const int64_t smax = std::max<int64_t>(1, G / QSPEC_SK_MIN_GPS);  // groups per slice
    if (S > smax) S = smax;
  }
  p.gps = (int)cdiv(G, S);
  p.S = (int)cdiv(G, p.gps);
  p.MB = (int)(M >= 64 ? 4 : cdiv(M, 16));
#ifndef QSPEC_SK_NO_MB5
  // W4A16 at 65-80 rows (a verify pass of 16 sequences, 5 rows each): one
  // 80-row block reads every weight tile once instead of twice (64 + 16)
  if (mode == 0 && cdiv(M, 16) == 5) p.MB = 5;
#endif
  // W4A16 with a k-split: one 16-row activation block per workgroup (more,
  // lighter workgroups; the weight tile is re-read from L2 per block)
  if (mode == 0 && p.S > 1) p.MB = 1;
  // two 16-row blocks per wavefront halve the LDS activation reads once the
  // activation tile spans several m-blocks (the bf16 verifier shapes)
  p.NB = (mode == 0 && p.MB >= 2) ? QSPEC_SK_NB16 : 1;
  p.NWV = ((p.MB == 1 || (mode == 0 && p.MB == 3)) && !max_tiles) ? skinny_nwv(N, p.S, p.NB) : 4;
  p.ntiles = (int)cdiv(N, 16 * p.NB * p.NWV);
  p.mchunks = (int)cdiv(M, 16 * p.MB);
  p.T = p.ntiles * p.mchunks;
  p.blocks = 8 * cdiv(p.T, 8) * p.S;
  // W4A16 on wide layers: the bias term from group sums staged with the
  // activations instead of a second MFMA chain per 16-row block (measured:
  // gate|up N = 37888 at M = 5 / 16 / 40 17.1 / 18.1 / 32.3 -> 15.2 / 16.6 /
  // 30.6 us, the 128256-row lm_head at M = 1 47.7 -> 47.2 us; on the narrow
  // layers it is level or slower, e.g. N = 11264, K = 2048 at M = 80 17.2 ->
  // 19.7 us).  A function of N alone, so a row's bits do not depend on M.
  p.VB = mode == 0 && N >= QSPEC_SK_VBIAS_N;
  p.cnt_bytes = p.S > 1 ? round_up((size_t)p.T * 8, 256) : 0;
  p.part_bytes = p.S > 1 ? (size_t)p.S * M * N * sizeof(float) : 0;
  return p;
}

template <int MODE, bool XOUT, bool VB>
hipError_t launch_skinny_t(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.blocks), blk(64 * p.NWV);
  // W4A16 with three activation blocks, or any mode with one: the workgroup
  // size balanced over the CUs (5, 8 or 10 wavefronts; 4 is the generic case)
  if (MODE == kW4A16 && p.MB == 3 && p.NWV != 4) {
    switch (p.NWV) {
      case 5: hipLaunchKernelGGL((skinny_kernel<kW4A16, 3, QSPEC_SK_NB16, QSPEC_SK_B3, XOUT, 5, VB>), grid, blk, 0, s, a); break;
      case 8: hipLaunchKernelGGL((skinny_kernel<kW4A16, 3, QSPEC_SK_NB16, QSPEC_SK_B3, XOUT, 8, VB>), grid, blk, 0, s, a); break;
      default: hipLaunchKernelGGL((skinny_kernel<kW4A16, 3, QSPEC_SK_NB16, QSPEC_SK_B3, XOUT, 10, VB>), grid, blk, 0, s, a); break;
    }
    return hipGetLastError();
  }
  if (p.MB == 1 && p.NWV != 4) {
    if constexpr (MODE == kW4A16) {
      switch (p.NWV) {
        case 5: hipLaunchKernelGGL((skinny_kernel<kW4A16, 1, 1, QSPEC_SK_B1, XOUT, 5, VB>), grid, blk, 0, s, a); break;
        case 8: hipLaunchKernelGGL((skinny_kernel<kW4A16, 1, 1, QSPEC_SK_B1, XOUT, 8, VB>), grid, blk, 0, s, a); break;
        default: hipLaunchKernelGGL((skinny_kernel<kW4A16, 1, 1, QSPEC_SK_B1, XOUT, 10, VB>), grid, blk, 0, s, a); break;
      }
    } else {  // W4A4 and W4A8 share the int8 data flow and its parameters
      switch (p.NWV) {
        case 5: hipLaunchKernelGGL((skinny_kernel<MODE, 1, 1, QSPEC_SK_A1, XOUT, 5, VB>), grid, blk, 0, s, a); break;
        case 8: hipLaunchKernelGGL((skinny_kernel<MODE, 1, 1, QSPEC_SK_A1, XOUT, 8, VB>), grid, blk, 0, s, a); break;
        default: hipLaunchKernelGGL((skinny_kernel<MODE, 1, 1, QSPEC_SK_A1, XOUT, 10, VB>), grid, blk, 0, s, a); break;
      }
    }
    return hipGetLastError();
  }
  if constexpr (MODE == kW4A16) {
    switch (p.MB) {
      case 1: hipLaunchKernelGGL((skinny_kernel<kW4A16, 1, 1, QSPEC_SK_B1, XOUT, 4, VB>), grid, blk, 0, s, a); break;
      case 2: hipLaunchKernelGGL((skinny_kernel<kW4A16, 2, QSPEC_SK_NB16, QSPEC_SK_B2, XOUT, 4, VB>), grid, blk, 0, s, a); break;
      case 3: hipLaunchKernelGGL((skinny_kernel<kW4A16, 3, QSPEC_SK_NB16, QSPEC_SK_B3, XOUT, 4, VB>), grid, blk, 0, s, a); break;
      case 5: hipLaunchKernelGGL((skinny_kernel<kW4A16, 5, QSPEC_SK_NB16, QSPEC_SK_B4, XOUT, 4, VB>), grid, blk, 0, s, a); break;
      default: hipLaunchKernelGGL((skinny_kernel<kW4A16, 4, QSPEC_SK_NB16, QSPEC_SK_B4, XOUT, 4, VB>), grid, blk, 0, s, a); break;
    }
  } else {
    switch (p.MB) {
      case 1: hipLaunchKernelGGL((skinny_kernel<MODE, 1, 1, QSPEC_SK_A1, XOUT>), grid, blk, 0, s, a); break;
      case 2: hipLaunchKernelGGL((skinny_kernel<MODE, 2, 1, QSPEC_SK_A2, XOUT>), grid, blk, 0, s, a); break;
      case 3: hipLaunchKernelGGL((skinny_kernel<MODE, 3, 1, QSPEC_SK_A3, XOUT>), grid, blk, 0, s, a); break;
      default: hipLaunchKernelGGL((skinny_kernel<MODE, 4, 1, QSPEC_SK_A4, XOUT>), grid, blk, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_skinny(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t s) {
  // the extra output: partials in the integer modes, the SwiGLU in W4A16
  if constexpr (MODE == kW4A16) {
    if (p.VB) {
      if (a.A != nullptr) return launch_skinny_t<MODE, true, true>(a, p, s);
      return launch_skinny_t<MODE, false, true>(a, p, s);
    }
  }
  if (MODE != kW4A16 ? a.P != nullptr : a.A != nullptr) return launch_skinny_t<MODE, true, false>(a, p, s);
  return launch_skinny_t<MODE, false, false>(a, p, s);
}

// A GEMM workspace of ws_bytes holds the k-split arrival counters in its
// first half and every family's partials in its second half.  The split
// depends on ws_bytes alone, so no call's partials can land on the counters
// of a later call that shares the workspace, whatever the two calls' shapes
// (a counter must read zero when its call starts).
struct WsSplit {
  unsigned long long* cnt;
  float* part;
};
WsSplit ws_split(void* ws, size_t ws_bytes) {
  const size_t half = ws_bytes / 2 / 256 * 256;
  return WsSplit{static_cast<unsigned long long*>(ws),
                 reinterpret_cast<float*>(static_cast<char*>(ws) + half)};
}
// bytes that hold both halves: twice the larger of counters and partials
size_t ws_need(size_t cnt_bytes, size_t part_bytes) {
  const size_t h = round_up(std::max(cnt_bytes, part_bytes), 256);
  return 2 * h;
}

struct GemvPlan {
  int S;
};
GemvPlan plan_gemv(int64_t K) { return GemvPlan{(int)cdiv(K / kGroup, kGemvGroups)}; }

// AUTO: for M <= 16 the stream family where the skinny family would have
// few workgroups (fewer than QSPEC_SK_TARGET_WG 64-row tiles), the skinny
// family otherwise up to skinny_max rows, the tiled family beyond.  The
// crossover measured on the Qwen2.5-7B projections lies between 128 and 192
// rows for W4A16 and between 256 and 384 for W4A4 (whose skinny kernel has
// half the MFMA work per weight byte).  Up to 512 rows the skinny family
// stays where the tiled grid would leave most of the chip idle on a long K
// (fewer than 128 tiles of bm x 256 and at least 64 groups): it splits K,
// the tiled kernel walks it on few workgroups (measured on the Qwen2.5-7B
// and Llama-3-8B down projections at M = 160 ... 512: W4A16 at M = 160
// 83 / 74 us against 129 / 98 us, W4A4 at M = 288 79 / 76 us against
// 123 / 95 us).  Below the skinny limit the tiled family takes over from
// tiled_min rows when its grid fills the chip (at least 256 tiles): on the
// gate|up projection (N = 37888) W4A16 at M = 64 / 96 / 128 runs 45 / 45 /
// 65 us tiled against 52 / 78 / 80 us skinny, W4A4 at M = 96 / 128 40 / 42
// against 46 / 48 us, while at M = 40 the skinny family is ahead (32 against
// 44 us).  W4A16 takes the stream family up to 8 rows only: from 9 rows its
// four activation loads per group cost more than the skinny family's LDS
// staging (measured at M = 16: down 25.8 against 20.0 us, QKV 13.0 against
// 9.4 us; at M = 5 down 12.3 against 18.3 us).  The choice depends on M, N
// and K only.
int auto_pick(int64_t M, int64_t N, int64_t K, int64_t stream_max, int64_t skinny_max, int64_t bm,
              int64_t tiled_min) {
  if (M <= stream_max && cdiv(N, 64) < QSPEC_SK_TARGET_WG) return QSPEC_GEMM_STREAM;
  const int64_t tiles = cdiv(N, 256) * cdiv(M, bm);
  if (M <= skinny_max)
    return (M >= tiled_min && tiles >= 256) ? QSPEC_GEMM_TILED : QSPEC_GEMM_SKINNY;
  if (M <= 512 && K / kGroup >= 64 && tiles < 128) return QSPEC_GEMM_SKINNY;
  return QSPEC_GEMM_TILED;
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

int w4a16_pick(int variant, int64_t M, int64_t N, int64_t K) {
  return variant != QSPEC_GEMM_AUTO ? variant : auto_pick(M, N, K, 8, 128, 32, 64);
}
int w4a4_pick(int variant, int64_t M, int64_t N, int64_t K) {
  return variant != QSPEC_GEMM_AUTO ? variant : auto_pick(M, N, K, kStreamMaxM, 256, 64, 96);
}
// W4A8 runs the stream family where W4A4 would, the skinny family otherwise
int w4a8_pick(int variant, int64_t M, int64_t N, int64_t K) {
  return w4a4_pick(variant, M, N, K) == QSPEC_GEMM_STREAM ? QSPEC_GEMM_STREAM : QSPEC_GEMM_SKINNY;
}

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const SkinnyPlan p = plan_skinny(0, M, N, K, true);  // four-wavefront tiles: the most counters
  const GemvPlan q = plan_gemv(K);
  const size_t gemv_part = q.S > 1 ? (size_t)q.S * std::min<int64_t>(M, 4) * N * sizeof(float) : 0;
  const size_t part = std::max(p.part_bytes, gemv_part);
  return p.cnt_bytes + part == 0 ? 0 : ws_need(p.cnt_bytes, part);
}

hipError_t launch_w4a16(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                        int64_t N, int64_t K, int variant, float* Y, void* ws, size_t ws_bytes,
                        hipStream_t s) {
  const int v = w4a16_pick(variant, M, N, K);
  const WsSplit w = ws_split(ws, ws_bytes);
  if (v == QSPEC_GEMM_STREAM)
    return launch_stream<kW4A16>(X, nullptr, Wq, Ws, M, N, K, Y, nullptr, nullptr, s);
  if (v == QSPEC_GEMM_GEMV) {
    const GemvPlan q = plan_gemv(K);
    // rows of X in chunks of up to 4
    for (int64_t m0 = 0; m0 < M; m0 += 4) {
      const int mm = (int)std::min<int64_t>(4, M - m0);
      float* out = q.S > 1 ? w.part : Y + m0 * N;
      const int64_t stride = (int64_t)mm * N;
      dim3 grid((unsigned)cdiv(N, 64), (unsigned)q.S);
      const uint16_t* Xm = X + m0 * K;
      switch (mm) {
        case 1: hipLaunchKernelGGL((w4a16_gemv_kernel<1, 8>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        case 2: hipLaunchKernelGGL((w4a16_gemv_kernel<2, 8>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        case 3: hipLaunchKernelGGL((w4a16_gemv_kernel<3, 8>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
        default: hipLaunchKernelGGL((w4a16_gemv_kernel<4, 8>), grid, dim3(256), 0, s, Xm, Wq, Ws, (int)N, (int)K, out, stride); break;
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
  if (v == QSPEC_GEMM_TILED)
    return launch_tiled<kW4A16>(X, nullptr, Wq, Ws, M, N, K, Y, nullptr, nullptr, s);
  const SkinnyPlan p = plan_skinny(0, M, N, K);
  SkinnyArgs a{};
  a.X = X;
  a.Wq = Wq;
  a.Ws = Ws;
  a.Y = Y;
  a.cnt = p.S > 1 ? w.cnt : nullptr;
  a.part = p.S > 1 ? w.part : nullptr;
  a.M = (int)M; a.N = (int)N; a.K = (int)K; a.S = p.S; a.gps = p.gps; a.ntiles = p.ntiles; a.T = p.T;
  return launch_skinny<kW4A16>(a, p, s);
}

// The gate|up layer with the SwiGLU in the epilogue: the SKINNY family's
// plan for (M, N, K) -- the same k-split as qspec_gemm_w4a16 with the
// SKINNY variant, so A is bitwise the pair-order SiLU * up of that Y.
hipError_t launch_w4a16_swiglu(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                               int64_t N, int64_t K, uint16_t* A, void* ws, size_t ws_bytes,
                               hipStream_t s) {
  const WsSplit w = ws_split(ws, ws_bytes);
  const SkinnyPlan p = plan_skinny(0, M, N, K);
  SkinnyArgs a{};
  a.X = X;
  a.Wq = Wq;
  a.Ws = Ws;
  a.A = A;
  a.cnt = p.S > 1 ? w.cnt : nullptr;
  a.part = p.S > 1 ? w.part : nullptr;
  a.M = (int)M; a.N = (int)N; a.K = (int)K; a.S = p.S; a.gps = p.gps; a.ntiles = p.ntiles; a.T = p.T;
  return launch_skinny<kW4A16>(a, p, s);
}

// The drafters' gate|up layer with the SwiGLU in the STREAM epilogue (M <=
// 16): A bitwise the pair-order silu_mul of that family's Y.
hipError_t launch_w4a4_swiglu(const uint8_t* Xq, const float* Xs, const uint8_t* Wq,
                              const uint16_t* Ws, int64_t M, int64_t N, int64_t K, uint16_t* A,
                              hipStream_t s) {
  return launch_stream<kW4A4>(Xq, Xs, Wq, Ws, M, N, K, nullptr, nullptr, nullptr, s, A);
}

hipError_t launch_w4a8_swiglu(const int8_t* Xq, const float* Xs, const uint8_t* Wq,
                              const uint16_t* Ws, int64_t M, int64_t N, int64_t K, uint16_t* A,
                              hipStream_t s) {
  return launch_stream<kW4A8>(Xq, Xs, Wq, Ws, M, N, K, nullptr, nullptr, nullptr, s, A);
}

size_t w4a4_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const SkinnyPlan p = plan_skinny(1, M, N, K, true);  // four-wavefront tiles: the most counters
  return p.cnt_bytes + p.part_bytes == 0 ? 0 : ws_need(p.cnt_bytes, p.part_bytes);
}

hipError_t launch_w4a4(const uint8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, uint16_t* Yb,
                       int32_t* P, void* ws, size_t ws_bytes, hipStream_t s) {
  // exactly one of Y (fp32) and Yb (bf16) is given; the int32 partials P
  // (with Y only) come from the family that computes Y, the same kernel
  // code instantiated with its partials store
  const int v = w4a4_pick(variant, M, N, K);
  if (v == QSPEC_GEMM_TILED) return launch_tiled<kW4A4>(Xq, Xs, Wq, Ws, M, N, K, Y, Yb, P, s);
  if (v == QSPEC_GEMM_STREAM) return launch_stream<kW4A4>(Xq, Xs, Wq, Ws, M, N, K, Y, Yb, P, s);
  const SkinnyPlan p = plan_skinny(1, M, N, K);
  const WsSplit w = ws_split(ws, ws_bytes);
  SkinnyArgs a{};
  a.X = Xq;
  a.Xs = Xs;
  a.Wq = Wq;
  a.Ws = Ws;
  a.Y = Y;
  a.Yb = Yb;
  a.P = P;
  a.cnt = p.S > 1 ? w.cnt : nullptr;
  a.part = p.S > 1 ? w.part : nullptr;
  a.M = (int)M; a.N = (int)N; a.K = (int)K; a.S = p.S; a.gps = p.gps; a.ntiles = p.ntiles; a.T = p.T;
  return launch_skinny<kW4A4>(a, p, s);
}

// W4A8: the stream family where AUTO picks it for W4A4 (M <= 16, N < 16384)
// or on request, else the skinny family, on the W4A4 plan (same k-split,
// same workspace); AUTO, SKINNY and STREAM are the accepted variants.
hipError_t launch_w4a8(const int8_t* Xq, const float* Xs, const uint8_t* Wq, const uint16_t* Ws,
                       int64_t M, int64_t N, int64_t K, int variant, float* Y, int32_t* P,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  if (w4a8_pick(variant, M, N, K) == QSPEC_GEMM_STREAM)
    return launch_stream<kW4A8>(Xq, Xs, Wq, Ws, M, N, K, Y, nullptr, P, s);
  const SkinnyPlan p = plan_skinny(1, M, N, K);
  const WsSplit w = ws_split(ws, ws_bytes);
  SkinnyArgs a{};
  a.X = Xq;
  a.Xs = Xs;
  a.Wq = Wq;
  a.Ws = Ws;
  a.Y = Y;
  a.P = P;
  a.cnt = p.S > 1 ? w.cnt : nullptr;
  a.part = p.S > 1 ? w.part : nullptr;
  a.M = (int)M; a.N = (int)N; a.K = (int)K; a.S = p.S; a.gps = p.gps; a.ntiles = p.ntiles; a.T = p.T;
  return launch_skinny<kW4A8>(a, p, s);
}

}  // namespace qspec
