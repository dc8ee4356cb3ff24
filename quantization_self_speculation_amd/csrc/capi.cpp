// C-ABI layer of libqspec.so: argument validation, the device check, status
// codes and dispatch to the HIP launchers.  Nothing here allocates device
// memory; validation finishes before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "launch.h"
#include "qspec_harness.h"
#include "qspec_probe.h"

namespace qspec {

namespace {
thread_local char g_err[512] = "";
std::atomic<int> g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other
}  // namespace

const char* last_error() { return g_err; }

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

qspec_status fail(qspec_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

qspec_status device_check() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QSPEC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    const int k = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (k == 1) return QSPEC_OK;
    if (k == 2) return fail(QSPEC_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(QSPEC_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(QSPEC_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return QSPEC_OK;
}

}  // namespace qspec

using namespace qspec;

namespace {

constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;  // sizes reach kernels as int

qspec_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QSPEC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  set_error("%s", "");
  return QSPEC_OK;
}

#define QS_REQUIRE(cond, status, ...)              \
  do {                                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

qspec_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(QSPEC_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(QSPEC_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return QSPEC_OK;
}

#define QS_TRY(expr)                   \
  do {                                 \
    const qspec_status _s = (expr);    \
    if (_s != QSPEC_OK) return _s;     \
  } while (0)

#define QS_PTR(p) QS_TRY(check_ptr((p), #p))

qspec_status check_k(int64_t K) {
  QS_REQUIRE(K >= QSPEC_GROUP && K % QSPEC_GROUP == 0 && K <= QSPEC_MAX_K, QSPEC_ERR_SHAPE,
             "K must be a multiple of 128 in [128, %d] (got %lld)", QSPEC_MAX_K, (long long)K);
  return QSPEC_OK;
}

qspec_status check_gemm(int64_t M, int64_t N, int64_t K, int group, int variant, bool w4a16) {
  QS_REQUIRE(group == QSPEC_GROUP, QSPEC_ERR_UNSUPPORTED, "group must be 128 (got %d)", group);
  QS_REQUIRE(M >= 1 && N >= 1, QSPEC_ERR_SHAPE, "need M >= 1 and N >= 1 (got %lld, %lld)",
             (long long)M, (long long)N);
  QS_TRY(check_k(K));
  QS_REQUIRE(M <= kMaxDim && N <= kMaxDim && M * N <= ((int64_t)1 << 40) &&
                 N * (K / 2) <= ((int64_t)1 << 42),
             QSPEC_ERR_SHAPE, "size too large");
  QS_REQUIRE(cdiv(M, 64) <= 65535, QSPEC_ERR_SHAPE, "M too large (at most 65535*64 rows)");
  const bool ok = variant == QSPEC_GEMM_AUTO || variant == QSPEC_GEMM_SKINNY ||
                  variant == QSPEC_GEMM_TILED || variant == QSPEC_GEMM_STREAM ||
                  (w4a16 && variant == QSPEC_GEMM_GEMV);
  QS_REQUIRE(ok, QSPEC_ERR_UNSUPPORTED, "unknown variant %d", variant);
  QS_REQUIRE(variant != QSPEC_GEMM_STREAM || M <= 16, QSPEC_ERR_UNSUPPORTED,
             "the STREAM family takes M <= 16 (got %lld)", (long long)M);
  return QSPEC_OK;
}

qspec_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return QSPEC_OK;
  QS_REQUIRE(ws != nullptr && have >= need, QSPEC_ERR_WORKSPACE,
             "workspace of %zu bytes needed (got %zu%s)", need, have, ws ? "" : ", NULL");
  QS_REQUIRE(aligned16(ws), QSPEC_ERR_ALIGN, "ws is not 16-byte aligned");
  return QSPEC_OK;
}

qspec_status check_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                          const float* draft_logits, const float* target_logits,
                          const float* u_accept, const float* u_sample, int32_t* n_accept,
                          int32_t* out_tok);

template <typename T>
qspec_status check_elem(const T* p, const char* name) {
  if (p == nullptr) return fail(QSPEC_ERR_NULL, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p) % alignof(T)) != 0)
    return fail(QSPEC_ERR_ALIGN, "%s is not aligned to its element size", name);
  return QSPEC_OK;
}

#define QS_EPTR(p) QS_TRY(check_elem((p), #p))

qspec_status check_heads(int n_heads, int n_kv) {
  QS_REQUIRE(n_heads >= 1 && n_kv >= 1 && n_heads % n_kv == 0 && n_heads <= 1024,
             QSPEC_ERR_SHAPE, "need n_heads a multiple of n_kv (got %d, %d)", n_heads, n_kv);
  return QSPEC_OK;
}

qspec_status check_cache(int64_t B, int64_t cap) {
  QS_REQUIRE(B >= 1 && B <= kMaxDim && cap >= 1 && cap <= QSPEC_MAX_CAP, QSPEC_ERR_SHAPE,
             "need B >= 1 and 1 <= cap <= %d (got %lld, %lld)", QSPEC_MAX_CAP, (long long)B,
             (long long)cap);
  return QSPEC_OK;
}

}  // namespace

extern "C" {

const char* qspec_status_str(qspec_status s) {
  switch (s) {
    case QSPEC_OK: return "ok";
    case QSPEC_ERR_NULL: return "null pointer";
    case QSPEC_ERR_SHAPE: return "bad shape";
    case QSPEC_ERR_UNSUPPORTED: return "unsupported argument";
    case QSPEC_ERR_ALIGN: return "misaligned pointer";
    case QSPEC_ERR_WORKSPACE: return "workspace too small";
    case QSPEC_ERR_DEVICE: return "unsupported device";
    case QSPEC_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* qspec_last_error(void) { return last_error(); }

const char* qspec_version(void) { return "qspec-gfx950 0.1"; }

qspec_status qspec_device_check(void) { return device_check(); }

size_t qspec_workspace_bytes(int op, int64_t a, int64_t b, int64_t c) {
  switch (op) {
    case QSPEC_OP_GEMM_W4A4:
    case QSPEC_OP_GEMM_W4A8:
      if (a < 1 || b < 1 || c < QSPEC_GROUP || c % QSPEC_GROUP) return 0;
      return w4a4_ws_bytes(a, b, c);
    case QSPEC_OP_GEMM_W4A16:
      if (a < 1 || b < 1 || c < QSPEC_GROUP || c % QSPEC_GROUP) return 0;
      return w4a16_ws_bytes(a, b, c);
    case QSPEC_OP_VERIFY:
      if (a < 1 || b < 1 || b > QSPEC_MAX_GAMMA || c < 1) return 0;
      return verify_ws_bytes(a, (int)b, c);
    default:
      return 0;
  }
}

int qspec_gemm_family(int op, int64_t M, int64_t N, int64_t K, int variant) {
  const bool w4a16 = op == QSPEC_OP_GEMM_W4A16;
  if (!w4a16 && op != QSPEC_OP_GEMM_W4A4 && op != QSPEC_OP_GEMM_W4A8) {
    set_error("op %d is not a GEMM op", op);
    return -1;
  }
  if (check_gemm(M, N, K, QSPEC_GROUP, variant, w4a16) != QSPEC_OK) return -1;
  if (op == QSPEC_OP_GEMM_W4A8) {
    if (variant == QSPEC_GEMM_TILED) {
      set_error("W4A8 runs the SKINNY or STREAM family (got variant %d)", variant);
      return -1;
    }
    return w4a8_pick(variant, M, N, K);
  }
  return w4a16 ? w4a16_pick(variant, M, N, K) : w4a4_pick(variant, M, N, K);
}

qspec_status qspec_pack_w4(const float* W, int64_t N, int64_t K, int group, uint8_t* Wq,
                           uint16_t* Ws, qspec_stream stream) {
  QS_REQUIRE(group == QSPEC_GROUP, QSPEC_ERR_UNSUPPORTED, "group must be 128 (got %d)", group);
  QS_REQUIRE(N >= 1 && N <= kMaxDim, QSPEC_ERR_SHAPE, "need N >= 1 (got %lld)", (long long)N);
  QS_TRY(check_k(K));
  QS_REQUIRE(N * (K / QSPEC_GROUP) <= ((int64_t)1 << 32), QSPEC_ERR_SHAPE, "size too large");
  QS_PTR(W);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_TRY(device_check());
  return hip_result(launch_pack_w4(W, N, K, Wq, Ws, (hipStream_t)stream), "pack_w4 launch");
}

qspec_status qspec_quant_act(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                             qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1 (got %lld)", (long long)M);
  QS_TRY(check_k(K));
  QS_PTR(X);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_TRY(device_check());
  return hip_result(launch_quant_act(X, M, K, Xq, Xs, (hipStream_t)stream), "quant_act launch");
}

qspec_status qspec_quant_act8(const uint16_t* X, int64_t M, int64_t K, int8_t* Xq, float* Xs,
                              qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1 (got %lld)", (long long)M);
  QS_TRY(check_k(K));
  QS_PTR(X);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_TRY(device_check());
  return hip_result(launch_quant_act8(X, M, K, Xq, Xs, (hipStream_t)stream), "quant_act8 launch");
}

qspec_status qspec_rotate_w(const float* W, int64_t N, int64_t K, float* Wr, qspec_stream stream) {
  QS_REQUIRE(N >= 1 && N <= kMaxDim, QSPEC_ERR_SHAPE, "need N >= 1 (got %lld)", (long long)N);
  QS_TRY(check_k(K));
  QS_REQUIRE(N * (K / QSPEC_GROUP) <= ((int64_t)1 << 34), QSPEC_ERR_SHAPE, "size too large");
  QS_PTR(W);
  QS_PTR(Wr);
  QS_TRY(device_check());
  return hip_result(launch_rotate(false, W, N, K, 0.125f, Wr, (hipStream_t)stream),
                    "rotate_w launch");
}

qspec_status qspec_rotate_x(const uint16_t* X, int64_t M, int64_t K, uint16_t* Xr,
                            qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1 (got %lld)", (long long)M);
  QS_TRY(check_k(K));
  QS_REQUIRE(M * (K / QSPEC_GROUP) <= ((int64_t)1 << 34), QSPEC_ERR_SHAPE, "size too large");
  QS_PTR(X);
  QS_PTR(Xr);
  QS_TRY(device_check());
  return hip_result(launch_rotate(true, X, M, K, 0.0625f, Xr, (hipStream_t)stream),
                    "rotate_x launch");
}

qspec_status qspec_quant_act_rot(const uint16_t* X, int64_t M, int64_t K, uint8_t* Xq, float* Xs,
                                 qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1 (got %lld)", (long long)M);
  QS_TRY(check_k(K));
  QS_PTR(X);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_TRY(device_check());
  return hip_result(launch_quant_act_rot(X, M, K, Xq, Xs, (hipStream_t)stream),
                    "quant_act_rot launch");
}

qspec_status qspec_gemm_w4a4(const uint8_t* Xq, const float* Xs, const uint8_t* Wq,
                             const uint16_t* Ws, int64_t M, int64_t N, int64_t K, int group,
                             int variant, float* Y, int32_t* P, void* ws, size_t ws_bytes,
                             qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, variant, false));
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(Y);
  if (P != nullptr) QS_PTR(P);
  QS_TRY(check_ws(ws, ws_bytes, w4a4_ws_bytes(M, N, K)));
  QS_TRY(device_check());
  return hip_result(launch_w4a4(Xq, Xs, Wq, Ws, M, N, K, variant, Y, nullptr, P, ws, ws_bytes,
                                (hipStream_t)stream),
                    "gemm_w4a4 launch");
}

qspec_status qspec_gemm_w4a4_bf16(const uint8_t* Xq, const float* Xs, const uint8_t* Wq,
                                  const uint16_t* Ws, int64_t M, int64_t N, int64_t K, int group,
                                  int variant, uint16_t* Y, void* ws, size_t ws_bytes,
                                  qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, variant, false));
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(Y);
  QS_TRY(check_ws(ws, ws_bytes, w4a4_ws_bytes(M, N, K)));
  QS_TRY(device_check());
  return hip_result(launch_w4a4(Xq, Xs, Wq, Ws, M, N, K, variant, nullptr, Y, nullptr, ws, ws_bytes,
                                (hipStream_t)stream),
                    "gemm_w4a4_bf16 launch");
}

qspec_status qspec_gemm_w4a8(const int8_t* Xq, const float* Xs, const uint8_t* Wq,
                             const uint16_t* Ws, int64_t M, int64_t N, int64_t K, int group,
                             int variant, float* Y, int32_t* P, void* ws, size_t ws_bytes,
                             qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, variant, false));
  QS_REQUIRE(variant == QSPEC_GEMM_AUTO || variant == QSPEC_GEMM_SKINNY ||
                 variant == QSPEC_GEMM_STREAM,
             QSPEC_ERR_UNSUPPORTED, "W4A8 runs the SKINNY or STREAM family (got variant %d)",
             variant);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(Y);
  if (P != nullptr) QS_PTR(P);
  QS_TRY(check_ws(ws, ws_bytes, w4a4_ws_bytes(M, N, K)));
  QS_TRY(device_check());
  return hip_result(launch_w4a8(Xq, Xs, Wq, Ws, M, N, K, variant, Y, P, ws, ws_bytes,
                                 (hipStream_t)stream),
                    "gemm_w4a8 launch");
}

qspec_status qspec_gemm_w4a16(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws, int64_t M,
                              int64_t N, int64_t K, int group, int variant, float* Y, void* ws,
                              size_t ws_bytes, qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, variant, true));
  QS_PTR(X);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(Y);
  QS_TRY(check_ws(ws, ws_bytes, w4a16_ws_bytes(M, N, K)));
  QS_TRY(device_check());
  return hip_result(launch_w4a16(X, Wq, Ws, M, N, K, variant, Y, ws, ws_bytes, (hipStream_t)stream),
                    "gemm_w4a16 launch");
}

qspec_status qspec_gemm_w4a16_swiglu(const uint16_t* X, const uint8_t* Wq, const uint16_t* Ws,
                                     int64_t M, int64_t N, int64_t K, int group, uint16_t* A,
                                     void* ws, size_t ws_bytes, qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, QSPEC_GEMM_SKINNY, true));
  QS_REQUIRE(N % 16 == 0, QSPEC_ERR_SHAPE,
             "N (gate|up rows) must be a multiple of 16 (got %lld)", (long long)N);
  QS_PTR(X);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(A);
  QS_TRY(check_ws(ws, ws_bytes, w4a16_ws_bytes(M, N, K)));
  QS_TRY(device_check());
  return hip_result(launch_w4a16_swiglu(X, Wq, Ws, M, N, K, A, ws, ws_bytes, (hipStream_t)stream),
                    "gemm_w4a16_swiglu launch");
}

qspec_status qspec_gemm_w4a4_swiglu(const uint8_t* Xq, const float* Xs, const uint8_t* Wq,
                                    const uint16_t* Ws, int64_t M, int64_t N, int64_t K, int group,
                                    uint16_t* A, qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, QSPEC_GEMM_STREAM, false));
  QS_REQUIRE(N % 16 == 0, QSPEC_ERR_SHAPE,
             "N (gate|up rows) must be a multiple of 16 (got %lld)", (long long)N);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(A);
  QS_TRY(device_check());
  return hip_result(launch_w4a4_swiglu(Xq, Xs, Wq, Ws, M, N, K, A, (hipStream_t)stream),
                    "gemm_w4a4_swiglu launch");
}

qspec_status qspec_gemm_w4a8_swiglu(const int8_t* Xq, const float* Xs, const uint8_t* Wq,
                                    const uint16_t* Ws, int64_t M, int64_t N, int64_t K, int group,
                                    uint16_t* A, qspec_stream stream) {
  QS_TRY(check_gemm(M, N, K, group, QSPEC_GEMM_STREAM, false));
  QS_REQUIRE(N % 16 == 0, QSPEC_ERR_SHAPE,
             "N (gate|up rows) must be a multiple of 16 (got %lld)", (long long)N);
  QS_PTR(Xq);
  QS_PTR(Xs);
  QS_PTR(Wq);
  QS_PTR(Ws);
  QS_PTR(A);
  QS_TRY(device_check());
  return hip_result(launch_w4a8_swiglu(Xq, Xs, Wq, Ws, M, N, K, A, (hipStream_t)stream),
                    "gemm_w4a8_swiglu launch");
}

qspec_status qspec_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                          const float* draft_logits, const float* target_logits,
                          const float* u_accept, const float* u_sample, int32_t* n_accept,
                          int32_t* out_tok, void* ws, size_t ws_bytes, qspec_stream stream) {
  QS_TRY(check_verify(mode, B, gamma, V, draft_tok, draft_logits, target_logits, u_accept,
                      u_sample, n_accept, out_tok));
  QS_TRY(check_ws(ws, ws_bytes, verify_ws_bytes(B, gamma, V)));
  QS_TRY(device_check());
  return hip_result(launch_verify(mode, B, gamma, V, draft_tok, draft_logits, target_logits,
                                  u_accept, u_sample, n_accept, out_tok, ws, (hipStream_t)stream),
                    "verify launch");
}

qspec_status qspec_verify_noalloc(int mode, int64_t B, int gamma, int64_t V,
                                  const int32_t* draft_tok, const float* draft_logits,
                                  const float* target_logits, const float* u_accept,
                                  const float* u_sample, int32_t* n_accept, int32_t* out_tok,
                                  qspec_stream stream) {
  QS_TRY(check_verify(mode, B, gamma, V, draft_tok, draft_logits, target_logits, u_accept,
                      u_sample, n_accept, out_tok));
  const size_t need = verify_ws_bytes(B, gamma, V);
  QS_REQUIRE(need <= kVerifyScratchBytes, QSPEC_ERR_WORKSPACE,
             "these sizes need %zu bytes of scratch; the fixed scratch of "
             "qspec_verify_noalloc holds %zu (call qspec_verify with a workspace)",
             need, kVerifyScratchBytes);
  QS_TRY(device_check());
  return hip_result(launch_verify_noalloc(mode, B, gamma, V, draft_tok, draft_logits,
                                          target_logits, u_accept, u_sample, n_accept, out_tok,
                                          (hipStream_t)stream),
                    "verify_noalloc launch");
}

}  // extern "C"

namespace {
qspec_status check_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                          const float* draft_logits, const float* target_logits,
                          const float* u_accept, const float* u_sample, int32_t* n_accept,
                          int32_t* out_tok) {
  QS_REQUIRE(mode == QSPEC_VERIFY_GREEDY || mode == QSPEC_VERIFY_SAMPLE, QSPEC_ERR_UNSUPPORTED,
             "unknown verify mode %d", mode);
  QS_REQUIRE(gamma >= 1 && gamma <= QSPEC_MAX_GAMMA, QSPEC_ERR_SHAPE,
             "gamma must be in [1, %d] (got %d)", QSPEC_MAX_GAMMA, gamma);
  QS_REQUIRE(B >= 1 && V >= 1 && V <= ((int64_t)1 << 23), QSPEC_ERR_SHAPE,
             "need B >= 1 and 1 <= V <= 2^23");
  QS_REQUIRE(B * (2 * gamma + 1) <= 65535, QSPEC_ERR_SHAPE,
             "B * (2 gamma + 1) must be at most 65535");
  QS_PTR(draft_tok);
  QS_PTR(target_logits);
  QS_PTR(n_accept);
  QS_PTR(out_tok);
  if (mode == QSPEC_VERIFY_SAMPLE) {
    QS_PTR(draft_logits);
    QS_PTR(u_accept);
    QS_PTR(u_sample);
  } else {
    QS_REQUIRE(draft_logits == nullptr && u_accept == nullptr && u_sample == nullptr,
               QSPEC_ERR_UNSUPPORTED, "greedy mode takes no draft logits or uniforms");
  }
  return QSPEC_OK;
}
}  // namespace

extern "C" {

// ---------------------------------------------------------------- decoder kernels
qspec_status qspec_embed(const uint16_t* emb, int64_t V, int64_t d, const int32_t* tok, int64_t M,
                         float* x, qspec_stream stream) {
  QS_REQUIRE(V >= 1 && d >= 8 && d % 8 == 0 && d <= kMaxDim && M >= 1 && M <= kMaxDim,
             QSPEC_ERR_SHAPE, "need V >= 1, d a positive multiple of 8, M >= 1");
  QS_PTR(emb);
  QS_EPTR(tok);
  QS_EPTR(x);
  QS_TRY(device_check());
  return hip_result(launch_embed(emb, V, d, tok, M, x, (hipStream_t)stream), "embed launch");
}

qspec_status qspec_add_rmsnorm(float* x, int64_t x_stride, const float* add, int64_t add_stride,
                               int64_t M, int64_t d, double eps, uint16_t* y,
                               qspec_stream stream) {
  QS_REQUIRE(d >= 1 && d <= QSPEC_MAX_D && x_stride >= d && M >= 1 && M <= kMaxDim,
             QSPEC_ERR_SHAPE, "need 1 <= d <= %d, x_stride >= d, M >= 1", QSPEC_MAX_D);
  QS_REQUIRE(add == nullptr || add_stride >= d, QSPEC_ERR_SHAPE, "need add_stride >= d");
  QS_REQUIRE(eps >= 0.0, QSPEC_ERR_SHAPE, "eps must be >= 0");
  QS_EPTR(x);
  if (add != nullptr) QS_EPTR(add);
  QS_EPTR(y);
  QS_TRY(device_check());
  return hip_result(launch_add_rmsnorm(x, x_stride, add, add_stride, M, d, eps, y,
                                       (hipStream_t)stream),
                    "add_rmsnorm launch");
}

qspec_status qspec_add_rmsnorm_quant(float* x, int64_t x_stride, const float* add,
                                     int64_t add_stride, int64_t M, int64_t d, double eps,
                                     uint16_t* y, uint8_t* yq, float* ys, qspec_stream stream) {
  QS_REQUIRE(d >= 1 && d <= QSPEC_MAX_D && x_stride >= d && M >= 1 && M <= kMaxDim,
             QSPEC_ERR_SHAPE, "need 1 <= d <= %d, x_stride >= d, M >= 1", QSPEC_MAX_D);
  QS_TRY(check_k(d));
  QS_REQUIRE(add == nullptr || add_stride >= d, QSPEC_ERR_SHAPE, "need add_stride >= d");
  QS_REQUIRE(eps >= 0.0, QSPEC_ERR_SHAPE, "eps must be >= 0");
  QS_EPTR(x);
  if (add != nullptr) QS_EPTR(add);
  QS_EPTR(y);
  QS_PTR(yq);
  QS_PTR(ys);
  QS_TRY(device_check());
  return hip_result(launch_add_rmsnorm_quant(x, x_stride, add, add_stride, M, d, eps, y, yq, ys,
                                             (hipStream_t)stream),
                    "add_rmsnorm_quant launch");
}

qspec_status qspec_add_rmsnorm_quant8(float* x, int64_t x_stride, const float* add,
                                      int64_t add_stride, int64_t M, int64_t d, double eps,
                                      uint16_t* y, int8_t* yq, float* ys, qspec_stream stream) {
  QS_REQUIRE(d >= 1 && d <= QSPEC_MAX_D && x_stride >= d && M >= 1 && M <= kMaxDim,
             QSPEC_ERR_SHAPE, "need 1 <= d <= %d, x_stride >= d, M >= 1", QSPEC_MAX_D);
  QS_TRY(check_k(d));
  QS_REQUIRE(add == nullptr || add_stride >= d, QSPEC_ERR_SHAPE, "need add_stride >= d");
  QS_REQUIRE(eps >= 0.0, QSPEC_ERR_SHAPE, "eps must be >= 0");
  QS_EPTR(x);
  if (add != nullptr) QS_EPTR(add);
  QS_EPTR(y);
  QS_PTR(yq);
  QS_PTR(ys);
  QS_TRY(device_check());
  return hip_result(launch_add_rmsnorm_quant8(x, x_stride, add, add_stride, M, d, eps, y, yq, ys,
                                              (hipStream_t)stream),
                    "add_rmsnorm_quant8 launch");
}

qspec_status qspec_rope_kv(const float* qkv, int64_t M, int n_heads, int n_kv, const int32_t* seq,
                           const int32_t* pos, double rope_base, float* q_out, uint16_t* kcache,
                           uint16_t* vcache, int64_t B, int64_t cap, qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1");
  QS_TRY(check_heads(n_heads, n_kv));
  QS_TRY(check_cache(B, cap));
  QS_REQUIRE(rope_base > 0.0, QSPEC_ERR_SHAPE, "rope_base must be > 0");
  QS_EPTR(qkv);
  QS_EPTR(seq);
  QS_EPTR(pos);
  QS_EPTR(q_out);
  QS_EPTR(kcache);
  QS_EPTR(vcache);
  QS_TRY(device_check());
  return hip_result(launch_rope_kv(qkv, M, n_heads, n_kv, QSPEC_HEAD_DIM, seq, pos, rope_base,
                                   q_out, kcache, vcache, B, cap, (hipStream_t)stream),
                    "rope_kv launch");
}

qspec_status qspec_attention(const float* q, const uint16_t* kcache, const uint16_t* vcache,
                             int64_t M, int n_heads, int n_kv, const int32_t* seq,
                             const int32_t* pos, int64_t B, int64_t cap, uint16_t* out,
                             qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1");
  QS_TRY(check_heads(n_heads, n_kv));
  QS_REQUIRE(n_kv <= 65535, QSPEC_ERR_SHAPE, "n_kv too large");
  QS_TRY(check_cache(B, cap));
  QS_EPTR(q);
  QS_EPTR(kcache);
  QS_EPTR(vcache);
  QS_EPTR(seq);
  QS_EPTR(pos);
  QS_EPTR(out);
  QS_TRY(device_check());
  return hip_result(launch_attention(q, kcache, vcache, M, n_heads, n_kv, seq, pos, B, cap, out,
                                     (hipStream_t)stream),
                    "attention launch");
}

qspec_status qspec_rope_attention(const float* qkv, int64_t M, int n_heads, int n_kv,
                                  const int32_t* seq, const int32_t* pos, double rope_base,
                                  float* q_out, uint16_t* kcache, uint16_t* vcache, int64_t B,
                                  int64_t cap, uint16_t* out, qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim, QSPEC_ERR_SHAPE, "need M >= 1");
  QS_TRY(check_heads(n_heads, n_kv));
  QS_REQUIRE(n_kv <= 65535, QSPEC_ERR_SHAPE, "n_kv too large");
  QS_TRY(check_cache(B, cap));
  QS_REQUIRE(rope_base > 0.0, QSPEC_ERR_SHAPE, "rope_base must be > 0");
  QS_EPTR(qkv);
  QS_EPTR(seq);
  QS_EPTR(pos);
  QS_EPTR(q_out);
  QS_EPTR(kcache);
  QS_EPTR(vcache);
  QS_EPTR(out);
  QS_TRY(device_check());
  return hip_result(launch_rope_attention(qkv, M, n_heads, n_kv, seq, pos, rope_base, q_out,
                                          kcache, vcache, B, cap, out, (hipStream_t)stream),
                    "rope_attention launch");
}

qspec_status qspec_silu_mul(const float* gu, int64_t M, int64_t ffn, uint16_t* a,
                            qspec_stream stream) {
  QS_REQUIRE(M >= 1 && ffn >= 1 && M * ffn <= ((int64_t)1 << 40), QSPEC_ERR_SHAPE,
             "need M >= 1 and ffn >= 1");
  QS_EPTR(gu);
  QS_EPTR(a);
  QS_TRY(device_check());
  return hip_result(launch_silu_mul(gu, M, ffn, a, (hipStream_t)stream), "silu_mul launch");
}

qspec_status qspec_silu_mul_pairs(const float* gu, int64_t M, int64_t ffn, uint16_t* a,
                                  qspec_stream stream) {
  QS_REQUIRE(M >= 1 && ffn >= 8 && ffn % 8 == 0 && M * ffn <= ((int64_t)1 << 40), QSPEC_ERR_SHAPE,
             "need M >= 1 and ffn a positive multiple of 8");
  QS_EPTR(gu);
  QS_EPTR(a);
  QS_TRY(device_check());
  return hip_result(launch_silu_mul_pairs(gu, M, ffn, a, (hipStream_t)stream),
                    "silu_mul_pairs launch");
}

qspec_status qspec_argmax(const float* x, int64_t M, int64_t V, int32_t* out, int64_t out_stride,
                          qspec_stream stream) {
  QS_REQUIRE(M >= 1 && M <= kMaxDim && V >= 1 && V <= kMaxDim && out_stride >= 1,
             QSPEC_ERR_SHAPE, "need M >= 1, 1 <= V < 2^31, out_stride >= 1");
  QS_EPTR(x);
  QS_EPTR(out);
  QS_TRY(device_check());
  return hip_result(launch_argmax(x, M, V, out, out_stride, (hipStream_t)stream),
                    "argmax launch");
}

qspec_status qspec_spec_prepare(int phase, int64_t B, int gamma, int j, const int32_t* len,
                                const int32_t* vtok, int32_t* drafts, int32_t* seq, int32_t* pos,
                                int32_t* tok, qspec_stream stream) {
  QS_REQUIRE(phase == 0 || phase == 1, QSPEC_ERR_UNSUPPORTED, "phase must be 0 or 1");
  QS_REQUIRE(B >= 1 && B <= ((int64_t)1 << 24) && gamma >= 0 && gamma <= QSPEC_MAX_GAMMA,
             QSPEC_ERR_SHAPE, "need 1 <= B <= 2^24 and 0 <= gamma <= %d", QSPEC_MAX_GAMMA);
  if (phase == 0)
    QS_REQUIRE(j >= 0 && j <= gamma, QSPEC_ERR_SHAPE, "draft step j must be in [0, gamma]");
  else
    QS_REQUIRE(gamma >= 1, QSPEC_ERR_SHAPE, "verify needs gamma >= 1");
  QS_EPTR(len);
  QS_EPTR(vtok);
  if (phase == 1) QS_EPTR(drafts);
  QS_EPTR(seq);
  QS_EPTR(pos);
  QS_EPTR(tok);
  QS_TRY(device_check());
  return hip_result(launch_spec_prepare(phase, B, gamma, j, len, vtok, drafts, seq, pos, tok,
                                        (hipStream_t)stream),
                    "spec_prepare launch");
}

qspec_status qspec_spec_commit(int64_t B, int gamma, const int32_t* n_accept,
                               const int32_t* out_tok, int32_t* len, int32_t* vtok,
                               int64_t vtok_stride, int32_t* gen, int64_t gen_cap, int32_t* n_gen,
                               int max_gen, int64_t* stats, qspec_stream stream) {
  QS_REQUIRE(B >= 1 && B <= 65536 && gamma >= 0 && gamma <= QSPEC_MAX_GAMMA, QSPEC_ERR_SHAPE,
             "need 1 <= B <= 65536 and 0 <= gamma <= %d", QSPEC_MAX_GAMMA);
  QS_REQUIRE(vtok_stride >= 1 && gen_cap >= 1 && max_gen >= 1, QSPEC_ERR_SHAPE,
             "need vtok_stride, gen_cap and max_gen >= 1");
  if (n_accept != nullptr) QS_EPTR(n_accept);
  QS_EPTR(out_tok);
  QS_EPTR(len);
  QS_EPTR(vtok);
  QS_EPTR(gen);
  QS_EPTR(n_gen);
  QS_EPTR(stats);
  QS_TRY(device_check());
  return hip_result(launch_spec_commit(B, gamma, n_accept, out_tok, len, vtok, vtok_stride, gen,
                                       gen_cap, n_gen, max_gen, stats, (hipStream_t)stream),
                    "spec_commit launch");
}

// ---------------------------------------------------------------- ceiling probes
qspec_status qspec_probe_read(const void* buf, int64_t bytes, int blocks, int unroll,
                              uint32_t* sink, qspec_stream stream) {
  QS_REQUIRE(bytes >= 16 && bytes % 16 == 0, QSPEC_ERR_SHAPE,
             "bytes must be a positive multiple of 16");
  QS_REQUIRE(blocks >= 1 && blocks <= (1 << 20), QSPEC_ERR_SHAPE, "need 1 <= blocks <= 2^20");
  QS_REQUIRE(unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8 || unroll == 16,
             QSPEC_ERR_UNSUPPORTED, "unroll must be 1, 2, 4, 8 or 16");
  QS_PTR(buf);
  QS_EPTR(sink);
  QS_TRY(device_check());
  return hip_result(launch_probe_read(buf, bytes, blocks, unroll, sink, (hipStream_t)stream),
                    "probe_read launch");
}

qspec_status qspec_probe_mfma(int kind, int blocks, int iters, float* sink, qspec_stream stream) {
  QS_REQUIRE(kind == 0 || kind == 1, QSPEC_ERR_UNSUPPORTED, "kind must be 0 or 1");
  QS_REQUIRE(blocks >= 1 && blocks <= (1 << 20) && iters >= 1, QSPEC_ERR_SHAPE,
             "need 1 <= blocks <= 2^20 and iters >= 1");
  QS_EPTR(sink);
  QS_TRY(device_check());
  return hip_result(launch_probe_mfma(kind, blocks, iters, sink, (hipStream_t)stream),
                    "probe_mfma launch");
}

qspec_status qspec_probe_empty(qspec_stream stream) {
  QS_TRY(device_check());
  return hip_result(launch_probe_empty((hipStream_t)stream), "probe_empty launch");
}

}  // extern "C"
