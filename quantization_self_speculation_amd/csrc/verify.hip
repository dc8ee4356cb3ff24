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
#include "launch.h"

namespace qspec {
namespace {

constexpr int kQPC = 2048;        // float4 quads per pass-1 chunk (8192 logits)
constexpr int kRCW = 8192;        // logits per residual chunk
constexpr int kDecWords = 8;      // per-sequence decision record (32-bit words)

__device__ __forceinline__ void argmax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  // (m, s) represents sum exp(x - m) = s; merge two such pairs
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s = s + s2 * __expf(m2 - m);
  }
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
template <bool GREEDY>
__global__ __launch_bounds__(256) void pass1_kernel(const float* __restrict__ tgt,
                                                    const float* __restrict__ drf, int64_t rows_t,
                                                    int64_t V, int nck, float* __restrict__ pm,
                                                    float* __restrict__ ps, int* __restrict__ pi) {
  __shared__ float sm[4];
  __shared__ float ss[4];
  __shared__ int si[4];
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  const bool is_t = row < rows_t;
  const int64_t rr = is_t ? row : row - rows_t;
  const float* rp = (is_t ? tgt : drf) + rr * V;
  int64_t a0, nq;
  row_geom(rr * V, V, a0, nq);
  const int tid = threadIdx.x;

  float bv = -INFINITY;  // greedy: best value / sampling: running max
  int bi = 0x7FFFFFFF;
  float s = 0.f;
  auto visit = [&](float v, int idx) {
    if (GREEDY) {
      argmax_merge(bv, bi, v, idx);
    } else {
      if (v > bv) {
        s = s * __expf(bv - v) + 1.0f;
        bv = v;
      } else {
        s += __expf(v - bv);
      }
    }
  };
  if (c == 0 && tid < a0) visit(rp[tid], tid);
  const int64_t q0 = (int64_t)c * kQPC;
  const int64_t q1 = min(nq, q0 + kQPC);
  const float4* qp = reinterpret_cast<const float4*>(rp + a0);
  for (int64_t q = q0 + tid; q < q1; q += 256) {
    const float4 v = qp[q];
    const int i = (int)(a0 + 4 * q);
    visit(v.x, i);
    visit(v.y, i + 1);
    visit(v.z, i + 2);
    visit(v.w, i + 3);
  }
  if (c == nck - 1) {
    const int64_t t0 = a0 + 4 * nq;
    if (t0 + tid < V) visit(rp[t0 + tid], (int)(t0 + tid));
  }

  // wavefront then block reduction, fixed order
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o, 64);
    if (GREEDY) {
      const int i2 = __shfl_xor(bi, o, 64);
      argmax_merge(bv, bi, v2, i2);
    } else {
      const float s2 = __shfl_xor(s, o, 64);
      // symmetric merge so every lane holds identical bits
      const float m = fmaxf(bv, v2);
      const float a = (bv == -INFINITY) ? 0.f : s * __expf(bv - m);
      const float b = (v2 == -INFINITY) ? 0.f : s2 * __expf(v2 - m);
      s = (lane & o) ? b + a : a + b;
      bv = m;
    }
  }
  if (lane == 0) {
    sm[w] = bv;
    ss[w] = s;
    si[w] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float m = sm[0], sacc = ss[0];
    int ib = si[0];
    for (int k = 1; k < 4; ++k) {
      if (GREEDY) argmax_merge(m, ib, sm[k], si[k]);
      else lse_merge(m, sacc, sm[k], ss[k]);
    }
    const int64_t o = row * nck + c;
    pm[o] = m;
    if (GREEDY) pi[o] = ib;
    else ps[o] = sacc;
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

// Merge the pass-1 (max, sum) pairs of one row across chunks (fixed order).
__device__ __forceinline__ void row_lse(const float* pm, const float* ps, int64_t row, int nck,
                                        int lane, float& M, float& S) {
  float m = -INFINITY;
  for (int c = lane; c < nck; c += 64) m = fmaxf(m, pm[row * nck + c]);
  m = wave_max(m);
  float s = 0.f;
  for (int c = lane; c < nck; c += 64) s += ps[row * nck + c] * __expf(pm[row * nck + c] - m);
  S = wave_sum(s);
  M = m;
}

// sampling decision: one wavefront per sequence.  Writes the decision record
// dec[b] = {n, kind (0 reject, 1 all accepted), Mt, St, Md, Sd, -, -}.
__global__ __launch_bounds__(64) void sample_decide_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, const int32_t* __restrict__ dt,
    const float* __restrict__ ua, int gamma, int64_t V, int nck, const float* __restrict__ pm,
    const float* __restrict__ ps, int64_t rows_t, float* __restrict__ dec) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  int n = gamma, kind = 1;
  float Mt = 0.f, St = 1.f, Md = 0.f, Sd = 1.f;
  for (int i = 0; i < gamma; ++i) {
    const int64_t rt = b * (gamma + 1) + i;
    const int64_t rd = rows_t + b * gamma + i;
    float mt, st, md, sd;
    row_lse(pm, ps, rt, nck, lane, mt, st);
    row_lse(pm, ps, rd, nck, lane, md, sd);
    int x = dt[b * gamma + i];
    x = min(max(x, 0), (int)(V - 1));
    const float p = expf(tgt[rt * V + x] - mt) / st;
    const float q = expf(drf[(b * gamma + i) * V + x] - md) / sd;
    const bool acc = q > 0.f ? (ua[b * gamma + i] <= p / q) : (p > 0.f);
    if (!acc) {
      n = i;
      kind = 0;
      Mt = mt; St = st; Md = md; Sd = sd;
      break;
    }
  }
  if (kind == 1) row_lse(pm, ps, b * (gamma + 1) + gamma, nck, lane, Mt, St);
  if (lane == 0) {
    float* d = dec + b * kDecWords;
    d[0] = __int_as_float(n);
    d[1] = __int_as_float(kind);
    d[2] = Mt; d[3] = St; d[4] = Md; d[5] = Sd;
  }
}

__device__ __forceinline__ float resid(const float* rt, const float* rd, int64_t j, int kind,
                                       float Mt, float iSt, float Md, float iSd) {
  const float p = __expf(rt[j] - Mt) * iSt;
  if (kind == 1) return p;
  const float q = __expf(rd[j] - Md) * iSd;
  return fmaxf(p - q, 0.f);
}

// residual chunk sums: grid = (rnck, B).  rs[b][c] = sum r, pp[b][c] = sum p.
__global__ __launch_bounds__(256) void resid_sums_kernel(const float* __restrict__ tgt,
                                                         const float* __restrict__ drf, int gamma,
                                                         int64_t V, int rnck,
                                                         const float* __restrict__ dec,
                                                         float* __restrict__ rs,
                                                         float* __restrict__ pp) {
  __shared__ float red[2][4];
  const int c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const float* d = dec + b * kDecWords;
  const int n = __float_as_int(d[0]), kind = __float_as_int(d[1]);
  const float Mt = d[2], iSt = 1.0f / d[3], Md = d[4], iSd = 1.0f / d[5];
  const float* rt = tgt + (b * (gamma + 1) + n) * V;
  const float* rd = drf + (b * gamma + min(n, gamma - 1)) * V;
  const int64_t j0 = (int64_t)c * kRCW, j1 = min(V, j0 + kRCW);
  float sr = 0.f, sp = 0.f;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) {
    const float p = __expf(rt[j] - Mt) * iSt;
    sp += p;
    sr += kind == 1 ? p : fmaxf(p - __expf(rd[j] - Md) * iSd, 0.f);
  }
  sr = wave_sum(sr);
  sp = wave_sum(sp);
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

// inverse-CDF select: one 256-thread block per sequence.
__global__ __launch_bounds__(256) void sample_select_kernel(
    const float* __restrict__ tgt, const float* __restrict__ drf, const int32_t* __restrict__ dt,
    const float* __restrict__ us, int gamma, int64_t V, int rnck, const float* __restrict__ dec,
    const float* __restrict__ rs, const float* __restrict__ pp, int32_t* __restrict__ n_accept,
    int32_t* __restrict__ out_tok) {
  __shared__ float seg[256];
  __shared__ int found;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const float* d = dec + b * kDecWords;
  const int n = __float_as_int(d[0]);
  int kind = __float_as_int(d[1]);
  const float Mt = d[2], iSt = 1.0f / d[3], Md = d[4], iSd = 1.0f / d[5];
  const float* rt = tgt + (b * (gamma + 1) + n) * V;
  const float* rd = drf + (b * gamma + min(n, gamma - 1)) * V;

  // chunk totals in fixed sequential order (every thread computes the same)
  float R = 0.f;
  for (int c = 0; c < rnck; ++c) R += rs[b * rnck + c];
  const float* tot = rs + b * rnck;
  if (R == 0.f && kind == 0) {  // p == q everywhere: sample from p
    kind = 1;
    tot = pp + b * rnck;
    R = 0.f;
    for (int c = 0; c < rnck; ++c) R += tot[c];
  }
  const float thr = us[b] * R;
  int cs = -1;
  float base = 0.f, run = 0.f;
  for (int c = 0; c < rnck; ++c) {
    const float nx = run + tot[c];
    if (nx > thr) {
      cs = c;
      base = run;
      break;
    }
    run = nx;
  }
  int last_c = -1;  // fallback: last chunk with mass
  for (int c = rnck - 1; c >= 0; --c)
    if (tot[c] > 0.f) {
      last_c = c;
      break;
    }
  const int cc = cs >= 0 ? cs : (last_c >= 0 ? last_c : 0);
  const int64_t j0 = (int64_t)cc * kRCW, j1 = min(V, j0 + kRCW);
  const int64_t len = j1 - j0;
  const int64_t per = (len + 255) / 256;  // contiguous segment per thread
  const int64_t s0 = j0 + tid * per, s1 = min(j1, s0 + per);

  // per-thread segment sums, then exclusive scan over threads (sequential)
  float ls = 0.f;
  for (int64_t j = s0; j < s1; ++j) ls += resid(rt, rd, j, kind, Mt, iSt, Md, iSd);
  seg[tid] = ls;
  if (tid == 0) found = 0x7FFFFFFF;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int t = 0; t < 256; ++t) {
      const float v = seg[t];
      seg[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int my = 0x7FFFFFFF;
  int mylast = -1;
  if (cs >= 0) {
    float cum = base + seg[tid];
    for (int64_t j = s0; j < s1; ++j) {
      const float r = resid(rt, rd, j, kind, Mt, iSt, Md, iSd);
      cum += r;
      if (cum > thr) {
        my = (int)j;
        break;
      }
    }
  }
  for (int64_t j = s0; j < s1; ++j)
    if (resid(rt, rd, j, kind, Mt, iSt, Md, iSd) > 0.f) mylast = (int)j;
  atomicMin(&found, my);  // LDS min of candidate indices: order-independent
  __syncthreads();
  int pick = found;
  if (pick == 0x7FFFFFFF) {
    // no crossing (threshold at or beyond the total): last index with mass
    __shared__ int lastj;
    if (tid == 0) lastj = -1;
    __syncthreads();
    atomicMax(&lastj, mylast);
    __syncthreads();
    pick = lastj >= 0 ? lastj : 0;
  }
  if (tid <= gamma) {
    int v = -1;
    if (tid < n) v = dt[b * gamma + tid];
    else if (tid == n) v = pick;
    out_tok[b * (gamma + 1) + tid] = v;
  }
  if (tid == 0) n_accept[b] = n;
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
  L.pm = take((size_t)rows * L.nck * 4);
  L.ps = take((size_t)rows * L.nck * 4);
  L.pi = take((size_t)B * (gamma + 1) * L.nck * 4);
  L.dec = take((size_t)B * kDecWords * 4);
  L.rs = take((size_t)B * L.rnck * 4);
  L.pp = take((size_t)B * L.rnck * 4);
  L.total = off;
  return L;
}

}  // namespace

size_t verify_ws_bytes(int64_t B, int gamma, int64_t V) { return layout(B, gamma, V).total; }

hipError_t launch_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                         const float* draft_logits, const float* target_logits,
                         const float* u_accept, const float* u_sample, int32_t* n_accept,
                         int32_t* out_tok, void* ws, hipStream_t s) {
  const VerifyLayout L = layout(B, gamma, V);
  char* w = static_cast<char*>(ws);
  float* pm = reinterpret_cast<float*>(w + L.pm);
  float* ps = reinterpret_cast<float*>(w + L.ps);
  int* pi = reinterpret_cast<int*>(w + L.pi);
  float* dec = reinterpret_cast<float*>(w + L.dec);
  float* rs = reinterpret_cast<float*>(w + L.rs);
  float* pp = reinterpret_cast<float*>(w + L.pp);
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
  hipLaunchKernelGGL(sample_decide_kernel, dim3((unsigned)B), dim3(64), 0, s, target_logits,
                     draft_logits, draft_tok, u_accept, gamma, V, L.nck, pm, ps, rows_t, dec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(resid_sums_kernel, dim3(L.rnck, (unsigned)B), dim3(256), 0, s,
                     target_logits, draft_logits, gamma, V, L.rnck, dec, rs, pp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sample_select_kernel, dim3((unsigned)B), dim3(256), 0, s, target_logits,
                     draft_logits, draft_tok, u_sample, gamma, V, L.rnck, dec, rs, pp, n_accept,
                     out_tok);
  return hipGetLastError();
}

}  // namespace qspec
