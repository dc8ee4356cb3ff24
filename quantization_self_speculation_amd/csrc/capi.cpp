// C-ABI layer of libqspec.so: argument validation, the device check, status
// codes and dispatch to the HIP launchers.  Nothing here allocates device
// memory; validation finishes before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "launch.h"

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
  QS_REQUIRE(K >= QSPEC_GROUP && K % QSPEC_GROUP == 0 && K <= ((int64_t)1 << 26), QSPEC_ERR_SHAPE,
             "K must be a multiple of 128 in [128, 2^26] (got %lld)", (long long)K);
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
                  variant == QSPEC_GEMM_TILED || (w4a16 && variant == QSPEC_GEMM_GEMV);
  QS_REQUIRE(ok, QSPEC_ERR_UNSUPPORTED, "unknown variant %d", variant);
  return QSPEC_OK;
}

qspec_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return QSPEC_OK;
  QS_REQUIRE(ws != nullptr && have >= need, QSPEC_ERR_WORKSPACE,
             "workspace of %zu bytes needed (got %zu%s)", need, have, ws ? "" : ", NULL");
  QS_REQUIRE(aligned16(ws), QSPEC_ERR_ALIGN, "ws is not 16-byte aligned");
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
  return hip_result(launch_w4a4(Xq, Xs, Wq, Ws, M, N, K, variant, Y, P, ws, (hipStream_t)stream),
                    "gemm_w4a4 launch");
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
  return hip_result(launch_w4a16(X, Wq, Ws, M, N, K, variant, Y, ws, (hipStream_t)stream),
                    "gemm_w4a16 launch");
}

qspec_status qspec_verify(int mode, int64_t B, int gamma, int64_t V, const int32_t* draft_tok,
                          const float* draft_logits, const float* target_logits,
                          const float* u_accept, const float* u_sample, int32_t* n_accept,
                          int32_t* out_tok, void* ws, size_t ws_bytes, qspec_stream stream) {
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
  QS_TRY(check_ws(ws, ws_bytes, verify_ws_bytes(B, gamma, V)));
  QS_TRY(device_check());
  return hip_result(launch_verify(mode, B, gamma, V, draft_tok, draft_logits, target_logits,
                                  u_accept, u_sample, n_accept, out_tok, ws, (hipStream_t)stream),
                    "verify launch");
}

}  // extern "C"
