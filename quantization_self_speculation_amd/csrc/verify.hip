// The draft/verify acceptance step.
//
// Pages: tech-dashboard QSpec summary, paragraph 3 (a draft proposes several
// tokens, the target verifies them in one parallel pass, the output
// distribution equals the target's); agihunt.info review of SpecQuant, method
// paragraph (a full match is accepted, the first mismatch is rewritten by the
// parent); "QSpec: Speculative Decoding with Complementary Quantization
// Schemes", Builds on (the speculative decoding / speculative sampling papers
// whose acceptance rule this is -- the pages name it but print no formula).
//
// The work is one streaming pass over the logits (HBM-bound) plus, when
// sampling, one pass over the one or two rows each sequence samples from:
//   greedy:   pass1 (chunk argmax, lowest index on ties) -> decide
//   sampling: pass1 (chunk max and sum of exp) -> decide (merge chunks,
//             accept tests) -> residual chunk sums -> inverse-CDF select
// Chunks are reduced in fixed order (no atomics): the same inputs give the
// same bits.
#include <atomic>
#include <mutex>

#include "launch.h"

namespace qspec {
namespace {

// Scratch of qspec_verify_noalloc, for callers that cannot allocate: one
// array per device, allocated with the code object and held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in); the device address comes from hipGetSymbolAddress,
// once per device, and is cached below.
static __device__ __align__(256) uint8_t scratch[kVerifyScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[64];

// chunk sizes (measured on MI355X; overridable at build time for sweeps)
#ifndef QSPEC_VF_QPC
#define QSPEC_VF_QPC 1024
#endif
#ifndef QSPEC_VF_RCW
#define QSPEC_VF_RCW 2048
#endif
constexpr int kQPC = QSPEC_VF_QPC;  // float4 quads per pass-1 chunk (4096 logits)
constexpr int kRCW = QSPEC_VF_RCW;  // logits per residual chunk (8 per thread)
constexpr int kMaxRChunks = 4096; // V <= kRCW * kMaxRChunks

__device__ __forceinline__ void argmax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// exp(a - b) for fp32 a, b <= a + 88: the rounding error of the subtraction
// is carried (Knuth's two-sum), s log2(e) is split into its fp32 rounding h
// and the remainder l (the FMA error-free product, TwoProduct of Ogita, Rump
// and Oishi, with log2(e) itself as a two-float constant), the hardware
// exp2 (v_exp_f32, about 1 ulp) takes h, and the remainder and the
// subtraction error are applied to first order: exp(x) = 2^h (1 + l ln 2 +
// err) up to terms below 1e-10 relative.  The result is within about 2 ulp
// of exp of the exact difference; a == -inf gives 0, and results below the
// fp32 normal range may be flushed to zero (they cannot move a sum of terms
// of which the largest is 1).
__device__ __forceinline__ float exp_diff(float a, float b) {
  if (a == -INFINITY) return 0.f;
  constexpr float kLog2eHi = 1.44269502162933349609375f;    // fp32 rounding of log2(e)
  constexpr float kLog2eLo = 1.925962991126e-8f;          // log2(e) - kLog2eHi
  constexpr float kLn2 = 0.693147182464599609375f;          // fp32 rounding of ln(2)
  const float s = a - b;
  const float bb = s - a;
  const float err = (a - (s - bb)) + (-b - bb);
  const float h = s * kLog2eHi;
  const float l = fmaf(s, kLog2eHi, -h) + s * kLog2eLo;
  const float e = __builtin_amdgcn_exp2f(h);
  return fmaf(e, fmaf(l, kLn2, err), e);
}

// Geometry of a row's pass-1 split: elements [0, a0) are a scalar head, then
// nq aligned float4 quads, then a scalar tail.  Chunk c takes quads
// [c*kQPC, (c+1)*kQPC); chunk 0 also takes the head, the last chunk the tail.
__device__ __forceinline__ void row_geom(int64_t base, int64_t V, int64_t& a0, int64_t& nq) {
  a0 = (4 - (base & 3)) & 3;
  if (a0 > V) a0 = V;
  nq = (V - a0) >> 2;
}

// pass 1.  grid = (nck, rows); rows = target rows then (sampling) draft rows.
// Each thread keeps its (at most 8) quads in registers: greedy takes the
// argmax (lowest index on ties); sampling takes the local max and the fp64
// sum of exp(x - max) over the same values.
template <bool GREEDY>
__global__ __launch_bounds__(256) void pass1_kernel(const float* __restrict__ tgt,
                                                    const float* __restrict__ drf, int64_t rows_t,
                                                    int64_t V, int nck, float* __restrict__ pm,
                                                    double* __restrict__ ps, int* __restrict__ pi) {
  constexpr int QPT = kQPC / 256;
  __shared__ float sm[4];
  __shared__ double ss[4];
  __shared__ int si[4];
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  const bool is_t = row < rows_t;
  const int64_t rr = is_t ? row : row - rows_t;
  const float* rp = (is_t ? tgt : drf) + rr * V;
  int64_t a0, nq;
  row_geom(rr * V, V, a0, nq);
  const int tid = threadIdx.x;

  const int64_t q0 = (int64_t)c * kQPC;
  const int64_t q1 = min(nq, q0 + kQPC);
  const float4* qp = reinterpret_cast<const float4*>(rp + a0);
  float4 v[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int64_t q = q0 + tid + 256 * k;
    v[k] = q < q1 ? qp[q] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  // scalar head (chunk 0) and tail (last chunk) elements: one thread may
  // hold one of each when the row has a single chunk
  float hv = -INFINITY, tv = -INFINITY;
  int hi = 0x7FFFFFFF, ti = 0x7FFFFFFF;
  if (c == 0 && tid < a0) {
    hv = rp[tid];
    hi = tid;
  }
  if (c == nck - 1) {
    const int64_t t0 = a0 + 4 * nq;
    if (t0 + tid < V) {
      tv = rp[t0 + tid];
      ti = (int)(t0 + tid);
    }
  }

  const int lane = tid & 63, w = tid >> 6;
  if (GREEDY) {
    float bv = hv;
    int bi = hi;
    argmax_merge(bv, bi, tv, ti);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = (int)(a0 + 4 * (q0 + tid + 256 * k));
      argmax_merge(bv, bi, v[k].x, i);
      argmax_merge(bv, bi, v[k].y, i + 1);
      argmax_merge(bv, bi, v[k].z, i + 2);
      argmax_merge(bv, bi, v[k].w, i + 3);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) {
      sm[w] = bv;
      si[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float m = sm[0];
      int ib = si[0];
      for (int k = 1; k < 4; ++k) argmax_merge(m, ib, sm[k], si[k]);
      pm[row * nck + c] = m;
      pi[row * nck + c] = ib;
    }
    return;
  }
  // sampling: the chunk max first, then every exponential relative to it
  float mx = fmaxf(hv, tv);
#pragma unroll
  for (int k = 0; k < QPT; ++k) mx = fmaxf(mx, fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w)));
  mx = wave_max_dpp(mx);
  if (lane == 0) sm[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  double s = 0.0;
  if (mx != -INFINITY) {
    s = (double)exp_diff(hv, mx) + (double)exp_diff(tv, mx);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      // four terms in fp32 (each within ~1 ulp), then into the fp64 sum
      const float e = (exp_diff(v[k].x, mx) + exp_diff(v[k].y, mx)) +
                      (exp_diff(v[k].z, mx) + exp_diff(v[k].w, mx));
      s += (double)e;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) ss[w] = s;
  __syncthreads();
  if (tid == 0) {
    pm[row * nck + c] = mx;
    ps[row * nck + c] = (ss[0] + ss[1]) + (ss[2] + ss[3]);
  }
}

// greedy decision: one wavefront per sequence.
__global__ __launch_bounds__(64) void greedy_decide_kernel(const int32_t* __restrict__ dt,
                                                           int gamma, int nck,
                                                           const float* __restrict__ pm,
                                                           const int* __restrict__ pi,
                                                           int32_t* __restrict__ n_accept,
                                                           int32_t* __restrict__ out_tok) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  int n = gamma;
  int emit = -1;
  for (int i = 0; i <= gamma; ++i) {
    const int64_t row = b * (gamma + 1) + i;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = lane; c < nck; c += 64) argmax_merge(bv, bi, pm[row * nck + c], pi[row * nck + c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      argmax_merge(bv, bi, v2, i2);
    }
    if (i == gamma || dt[b * gamma + i] != bi) {
      n = i;
      emit = bi;
      break;
    }
  }
  if (lane <= gamma) {
    int v = -1;
    if (lane < n) v = dt[b * gamma + lane];
    else if (lane == n) v = emit;
    out_tok[b * (gamma + 1) + lane] = v;
  }
  if (lane == 0) n_accept[b] = n;
}

// Merge the pass-1 (max, sum) pairs of one row across chunks (fixed order:
// lanes over chunks, then a butterfly that leaves identical bits in all lanes).
__device__ __forceinline__ void row_lse(const float* pm, const double* ps, int64_t row, int nck,
                                        int lane, float& M, double& S) {
  float m = -INFINITY;
  for (int c = lane; c < nck; c += 64) m = fmaxf(m, pm[row * nck + c]);
  m = wave_max_dpp(m);
  double s = 0.0;
  for (int c = lane; c < nck; c += 64) {
    const float mc = pm[row * nck + c];
    s += ps[row * nck + c] * (double)exp_diff(mc, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  S = s;
  M = m;
}

struct Decision {
  int n, kind;  // kind 0: rejected at n (residual max(0, p - q)); 1: all accepted (p_gamma)
  float Mt, Md;
  double St, Sd;
};

// The sampling decision of sequence b, taken by a whole 256-thread block and
// returned to every thread: the 2*gamma+1 row normalizers are merged in
// parallel (one wavefront per row), the logits at the drafted tokens are
// fetched in parallel, then lane i of the first wavefront runs the accept
// test of draft i and the lowest rejecting lane decides.  p(x) and q(x) are
// fp64: exact fp64 exponent of the exact difference over the pass-1 sums.
// Taken once per sequence (sample_decide_kernel): repeated at the start of
// every residual block it cost more than the launch it saved (measured).
__device__ Decision block_decide(const float* __restrict__ tgt, const float* __restrict__ drf,
                                 const int32_t* __restrict__ dt, const float* __restrict__ ua,
                                 int gamma, int64_t V, int nck, const float* __restrict__ pm,
                                 const double* __restrict__ ps, int64_t rows_t, int64_t b) {
  __shared__ float lm[2 * QSPEC_MAX_GAMMA + 1];
  __shared__ double lsum[2 * QSPEC_MAX_GAMMA + 1];
  __shared__ float lxt[QSPEC_MAX_GAMMA], lxd[QSPEC_MAX_GAMMA];
  __shared__ Decision sdec;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nr = 2 * gamma + 1;  // target rows 0..gamma, then draft rows
  auto row_of = [&](int r) -> int64_t {
    return r <= gamma ? b * (gamma + 1) + r : rows_t + b * gamma + (r - gamma - 1);
  };
  // the drafted tokens' logits are requested first: they do not depend on
  // the merges
  float xt = 0.f, xd = 0.f;
  if (tid < gamma) {
    const int x = min(max(dt[b * gamma + tid], 0), (int)(V - 1));
    xt = tgt[(b * (gamma + 1) + tid) * V + x];
    xd = drf[(b * gamma + tid) * V + x];
  }
  if (nck <= 64) {
    // every row of this wavefront (rows w, w + 4, ...) with its chunk pairs
    // requested at once, one chunk per lane, then merged row by row
    constexpr int RPW = (2 * QSPEC_MAX_GAMMA + 1 + 3) / 4;
    float pmv[RPW];
    double psv[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = w + 4 * k;
      pmv[k] = -INFINITY;
      psv[k] = 0.0;
      if (r < nr && lane < nck) {
        pmv[k] = pm[row_of(r) * nck + lane];
        psv[k] = ps[row_of(r) * nck + lane];
      }
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = w + 4 * k;
      if (r >= nr) break;  // uniform over the wavefront
      const float M = wave_max_dpp(pmv[k]);
      double S = psv[k] * (double)exp_diff(pmv[k], M);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) S += __shfl_xor(S, o, 64);
      if (lane == 0) {
        lm[r] = M;
        lsum[r] = S;
      }
    }
  } else {
    for (int r = w; r < nr; r += 4) {
      float M;
      double S;
      row_lse(pm, ps, row_of(r), nck, lane, M, S);
      if (lane == 0) {
        lm[r] = M;
        lsum[r] = S;
      }
    }
  }
  if (tid < gamma) {
    lxt[tid] = xt;
    lxd[tid] = xd;
  }
  __syncthreads();
  if (w == 0) {
    // every accept test at once (lane i tests draft i); the first rejection
    // ends the run, as in the sequential rule
    bool rej = false;
    if (lane < gamma) {
      const float mt = lm[lane], md = lm[gamma + 1 + lane];
      const double st = lsum[lane], sd = lsum[gamma + 1 + lane];
      const double p = exp((double)lxt[lane] - (double)mt) / st;
      const double q = exp((double)lxd[lane] - (double)md) / sd;
      const bool acc = q > 0.0 ? ((double)ua[b * gamma + lane] <= p / q) : (p > 0.0);
      rej = !acc;
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) {
      if (mask == 0) {
        sdec = Decision{gamma, 1, lm[gamma], 0.f, lsum[gamma], 1.0};
      } else {
        const int i = __builtin_ctzll(mask);
        sdec = Decision{i, 0, lm[i], lm[gamma + 1 + i], lsum[i], lsum[gamma + 1 + i]};
      }
    }
  }
  __syncthreads();
  return sdec;
}

// The sampling decision of each sequence, once (one block per sequence), for
// the residual and select passes to read.
__global__ __launch_bounds__(256) void sample_decide_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, const int32_t* __restrict__ dt,
    const float* __restrict__ ua, int gamma, int64_t V, int nck, const float* __restrict__ pm,
    const double* __restrict__ ps, int64_t rows_t, Decision* __restrict__ dec) {
  const int64_t b = blockIdx.x;
  const Decision D = block_decide(tgt, drf, dt, ua, gamma, V, nck, pm, ps, rows_t, b);
  if (threadIdx.x == 0) dec[b] = D;
}

// r_j of the row a sequence samples from, in fp64
__device__ __forceinline__ double resid(const float* rt, const float* rd, int64_t j, int kind,
                                        float Mt, double iSt, float Md, double iSd) {
  const double p = (double)exp_diff(rt[j], Mt) * iSt;
  if (kind == 1) return p;
  const double q = (double)exp_diff(rd[j], Md) * iSd;
  return p > q ? p - q : 0.0;
}

// residual chunk sums: grid = (rnck, B), kRCW logits per block (8 per
// thread, coalesced).  rs[b][c] = sum r, pp[b][c] = sum p (fp64).
__global__ __launch_bounds__(256) void resid_sums_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, const int32_t* __restrict__ dt,
    int gamma, int64_t V, int rnck, const Decision* __restrict__ dec, double* __restrict__ rs,
    double* __restrict__ pp) {
  constexpr int EPT = kRCW / 256;
  __shared__ double red[2][4];
  const int c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const Decision D = dec[b];
  const double iSt = 1.0 / D.St, iSd = 1.0 / D.Sd;
  const float* rt = tgt + (b * (gamma + 1) + D.n) * V;
  const float* rd = drf + (b * gamma + min(D.n, gamma - 1)) * V;
  const int64_t j0 = (int64_t)c * kRCW;
  float lt[EPT], ld[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int64_t j = j0 + threadIdx.x + 256 * k;
    lt[k] = j < V ? rt[j] : -INFINITY;
    ld[k] = (j < V && D.kind == 0) ? rd[j] : -INFINITY;
  }
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const double p = (double)exp_diff(lt[k], D.Mt) * iSt;
    const double q = (double)exp_diff(ld[k], D.Md) * iSd;
    sp += p;
    sr += D.kind == 1 ? p : (p > q ? p - q : 0.0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sr += __shfl_xor(sr, o, 64);
    sp += __shfl_xor(sp, o, 64);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][w] = sr;
    red[1][w] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    rs[b * rnck + c] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    pp[b * rnck + c] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// inverse-CDF select: one 256-thread block per sequence, fp64 cumulative sums.
// One wavefront finds the chunk holding the threshold from the chunk totals
// (each lane sums a run of chunks in order, a fixed-order scan over the lanes
// gives each run its start, each lane walks its run, the lowest crossing
// wins); inside that chunk each thread takes 8 consecutive logits, and a
// block-wide exclusive scan gives every thread its starting cumulative sum.
__global__ __launch_bounds__(256) void sample_select_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, const int32_t* __restrict__ dt,
    const float* __restrict__ us, int gamma, int64_t V, int rnck, const Decision* __restrict__ dec,
    const double* __restrict__ rs, const double* __restrict__ pp, int32_t* __restrict__ n_accept,
    int32_t* __restrict__ out_tok) {
  constexpr int EPT = kRCW / 256;
  __shared__ double wsum[4];
  __shared__ int found;
  __shared__ int lastj;
  __shared__ int sh_cs, sh_cc, sh_kind;
  __shared__ double sh_base, sh_thr;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const double* tr = rs + b * rnck;  // chunk totals, read by the first wavefront
  const double* tp = pp + b * rnck;
  const int per = (rnck + 63) / 64;
  const int c0 = min(rnck, lane * per), c1 = min(rnck, c0 + per);
  // the first wavefront's totals depend on b alone: with at most two chunks
  // per lane they are requested together with the decision (one memory
  // round trip instead of two)
  double r0 = 0.0, r1 = 0.0, p0 = 0.0, p1 = 0.0;  // chunks c0, c0 + 1: residual, target
  if (w == 0 && per <= 2) {
    if (c0 < c1) {
      r0 = tr[c0];
      p0 = tp[c0];
    }
    if (c0 + 1 < c1) {
      r1 = tr[c0 + 1];
      p1 = tp[c0 + 1];
    }
  }
  const float ub = us[b];
  const Decision D = dec[b];
  const double iSt = 1.0 / D.St, iSd = 1.0 / D.Sd;
  const float* rt = tgt + (b * (gamma + 1) + D.n) * V;
  const float* rd = drf + (b * gamma + min(D.n, gamma - 1)) * V;

  if (w == 0) {
    // chunk totals, one wavefront: lane l sums its run of `per` consecutive
    // chunks in order, then an inclusive scan over the lanes (fixed order)
    int kind = D.kind;
    int sel = 0;  // 0: residual totals, 1: target-probability totals
    // total of chunk c (c0 <= c < c1) of the selected kind
#define QSPEC_TOT(c) (per <= 2 ? (sel == 0 ? ((c) == c0 ? r0 : r1) : ((c) == c0 ? p0 : p1)) \
                               : (sel == 0 ? tr : tp)[(c)])
    double excl = 0.0, R = 0.0;
    for (int pass = 0; pass < 2; ++pass) {  // a second pass only to fall back to p
      double v = 0.0;
      for (int c = c0; c < c1; ++c) v += QSPEC_TOT(c);
      double incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.0;
      R = __shfl(incl, 63, 64);
      if (!(R == 0.0 && kind == 0)) break;  // uniform
      kind = 1;  // p == q everywhere: sample from p
      sel = 1;
    }
    const double thr = (double)ub * R;
    // each lane walks its run from its exclusive start; the lowest lane
    // whose walk passes the threshold holds the chunk
    int cs = -1;
    double base = 0.0;
    {
      double run = excl;
      for (int c = c0; c < c1; ++c) {
        const double nx = run + QSPEC_TOT(c);
        if (nx > thr) {
          cs = c;
          base = run;
          break;
        }
        run = nx;
      }
    }
    const unsigned long long hit = __ballot(cs >= 0);
    // last chunk with mass (fallback when the threshold is at or past the total)
    int last_c = -1;
    for (int c = c1 - 1; c >= c0; --c)
      if (QSPEC_TOT(c) > 0.0) {
        last_c = c;
        break;
      }
#undef QSPEC_TOT
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last_c = max(last_c, __shfl_xor(last_c, o, 64));
    if (lane == (hit ? __builtin_ctzll(hit) : 0)) {
      sh_cs = hit ? cs : -1;
      sh_cc = hit ? cs : (last_c >= 0 ? last_c : 0);
      sh_kind = kind;
      sh_base = hit ? base : 0.0;
      sh_thr = thr;
    }
  }
  __syncthreads();
  const int cs = sh_cs, cc = sh_cc, kind = sh_kind;
  const double base = sh_base, thr = sh_thr;
  const int64_t js = (int64_t)cc * kRCW + (int64_t)tid * EPT;  // this thread's 8 logits
  double r[EPT];
  double ls = 0.0;
  int mylast = -1;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int64_t j = js + k;
    double v = 0.0;
    if (j < V) {
      const double p = (double)exp_diff(rt[j], D.Mt) * iSt;
      if (kind == 1) {
        v = p;
      } else {
        const double q = (double)exp_diff(rd[j], D.Md) * iSd;
        v = p > q ? p - q : 0.0;
      }
    }
    r[k] = v;
    ls += v;
    if (v > 0.0) mylast = (int)j;
  }
  // inclusive scan of the thread sums within the wavefront, then across waves
  double inc = ls;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  double exc = __shfl_up(inc, 1, 64);  // exclusive prefix within the wavefront
  if (lane == 0) exc = 0.0;
  if (lane == 63) wsum[w] = inc;
  if (tid == 0) {
    found = 0x7FFFFFFF;
    lastj = -1;
  }
  __syncthreads();
  double wbase = 0.0;
  for (int k = 0; k < w; ++k) wbase += wsum[k];
  int my = 0x7FFFFFFF;
  if (cs >= 0) {
    double cum = base + wbase + exc;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      cum += r[k];
      if (my == 0x7FFFFFFF && cum > thr) my = (int)(js + k);
    }
  }
  atomicMin(&found, my);  // LDS min / max of candidate indices: order-independent
  atomicMax(&lastj, mylast);
  __syncthreads();
  int pick = found;
  if (pick == 0x7FFFFFFF) pick = lastj >= 0 ? lastj : 0;  // threshold at or past the total
  if (tid <= gamma) {
    int v = -1;
    if (tid < D.n) v = dt[b * gamma + tid];
    else if (tid == D.n) v = pick;
    out_tok[b * (gamma + 1) + tid] = v;
  }
  if (tid == 0) n_accept[b] = D.n;
}

struct VerifyLayout {
  int nck, rnck;
  size_t pm, ps, pi, dec, rs, pp, total;  // byte offsets
};

VerifyLayout layout(int64_t B, int gamma, int64_t V) {
  VerifyLayout L;
  L.nck = (int)std::max<int64_t>(1, cdiv(V / 4, kQPC));
  L.rnck = (int)cdiv(V, kRCW);
  const int64_t rows = B * (2 * gamma + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, 256);
    return o;
  };
  L.pm = take((size_t)rows * L.nck * sizeof(float));
  L.ps = take((size_t)rows * L.nck * sizeof(double));
  L.pi = take((size_t)B * (gamma + 1) * L.nck * sizeof(int));
  L.dec = take((size_t)B * sizeof(Decision));
  L.rs = take((size_t)B * L.rnck * sizeof(double));
  L.pp = take((size_t)B * L.rnck * sizeof(double));
  L.total = off;
  return L;
}

}  // namespace

size_t verify_ws_bytes(int64_t B, int gamma, int64_t V) { return layout(B, gamma, V).total; }

// The device address of this device's scratch array, looked up once per
// device with that device current.
hipError_t verify_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// qspec_verify on this device's scratch array.  The kernels write every
// scratch element they read later in the same call, so nothing is cleared;
// calls that overlap in time on one device share the array and race.
hipError_t launch_verify_noalloc(int mode, int64_t B, int gamma, int64_t V,
                                 const int32_t* draft_tok, const float* draft_logits,
                                 const float* target_logits, const float* u_accept,
                                 const float* u_sample, int32_t* n_accept, int32_t* out_tok,
                                 hipStream_t s) {
  if (verify_ws_bytes(B, gamma, V) > kVerifyScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = verify_scratch_ptr(&ws);
  if (e != hipSuccess) return e;
  return launch_verify(mode, B, gamma, V, draft_tok, draft_logits, target_logits, u_accept,
                       u_sample, n_accept, out_tok, ws, s);
}

hipError_t launch_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                         const float* draft_logits, const float* target_logits,
                         const float* u_accept, const float* u_sample, int32_t* n_accept,
                         int32_t* out_tok, void* ws, hipStream_t s) {
  const VerifyLayout L = layout(B, gamma, V);
  char* w = static_cast<char*>(ws);
  float* pm = reinterpret_cast<float*>(w + L.pm);
  double* ps = reinterpret_cast<double*>(w + L.ps);
  int* pi = reinterpret_cast<int*>(w + L.pi);
  Decision* dec = reinterpret_cast<Decision*>(w + L.dec);
  double* rs = reinterpret_cast<double*>(w + L.rs);
  double* pp = reinterpret_cast<double*>(w + L.pp);
  const int64_t rows_t = B * (gamma + 1);
  if (mode == QSPEC_VERIFY_GREEDY) {
    hipLaunchKernelGGL(pass1_kernel<true>, dim3(L.nck, (unsigned)rows_t), dim3(256), 0, s,
                       target_logits, target_logits, rows_t, V, L.nck, pm, ps, pi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(greedy_decide_kernel, dim3((unsigned)B), dim3(64), 0, s, draft_tok, gamma,
                       L.nck, pm, pi, n_accept, out_tok);
    return hipGetLastError();
  }
  const int64_t rows = rows_t + B * gamma;
  hipLaunchKernelGGL(pass1_kernel<false>, dim3(L.nck, (unsigned)rows), dim3(256), 0, s,
                     target_logits, draft_logits, rows_t, V, L.nck, pm, ps, pi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_decide_kernel, dim3((unsigned)B), dim3(256), 0, s, target_logits,
                     draft_logits, draft_tok, u_accept, gamma, V, L.nck, pm, ps, rows_t, dec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(resid_sums_kernel, dim3(L.rnck, (unsigned)B), dim3(256), 0, s,
                     target_logits, draft_logits, draft_tok, gamma, V, L.rnck, dec, rs, pp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sample_select_kernel, dim3((unsigned)B), dim3(256), 0, s, target_logits,
                     draft_logits, draft_tok, u_sample, gamma, V, L.rnck, dec, rs, pp, n_accept,
                     out_tok);
  return hipGetLastError();
}

}  // namespace qspec
