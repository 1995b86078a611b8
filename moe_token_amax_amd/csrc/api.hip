// C ABI of the W8A8_DYNAMIC library: argument checks, workspace sizing and the
// MoE chain. Declarations and contracts are in include/w8a8.h.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/w8a8.h"
#include "launch.hpp"
#include "mx.hpp"
#include "w4.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return W8A8_OK;
}

int launched(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(W8A8_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(err));
  return ok();
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// W8A8_CHECK set to anything but "" or "0" in the environment (read at every
// call): the grouped calls copy group_list to the host, synchronizing the
// call's stream, and reject a negative count or counts summing past R before
// anything is launched. A debugging aid, off by default: it synchronizes, so
// it cannot be used under graph capture. Without it the kernels still stay
// in bounds (a negative count owns no rows, rows past R are never touched),
// but the results of such a list are not meaningful.
bool debug_checks() {
  const char* v = std::getenv("W8A8_CHECK");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

int check_group_list(const char* who, const int64_t* group_list, int64_t E, int64_t R, void* stream) {
  if (!debug_checks()) return W8A8_OK;
  std::vector<int64_t> h((size_t)E);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t err = hipMemcpyAsync(h.data(), group_list, (size_t)E * sizeof(int64_t), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess)
    return fail(W8A8_ERR_LAUNCH, "%s: W8A8_CHECK copy of group_list: %s", who, hipGetErrorString(err));
  int64_t sum = 0;
  for (int64_t e = 0; e < E; ++e) {
    if (h[(size_t)e] < 0)
      return fail(W8A8_ERR_SHAPE, "%s: group_list[%lld] = %lld is negative", who, (long long)e,
                  (long long)h[(size_t)e]);
    sum += h[(size_t)e];
    if (sum > R)
      return fail(W8A8_ERR_SHAPE, "%s: group_list counts pass R = %lld rows at expert %lld", who, (long long)R,
                  (long long)e);
  }
  return W8A8_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows / columns limit of the grids
constexpr int64_t kMaxExperts = 1024;           // LDS tile table of the grouped kernel

int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

struct MoeWs {
  int64_t q1, s1, h, q2, s2, inner, total;
};

MoeWs moe_layout(int64_t R, int64_t E, int64_t H, int64_t I) {
  MoeWs w{};
  int64_t o = 0;
  w.q1 = o; o += align256(R * H);                // int8 [R, H] (BF16 input only)
  w.s1 = o; o += align256(R * 4);                // f32 [R]
  w.h = o;  o += align256(R * 2 * I * 2);        // BF16 [R, 2I]
  w.q2 = o; o += align256(R * I);                // int8 [R, I]
  w.s2 = o; o += align256(R * 4);                // f32 [R]
  w.inner = o;
  o += align256(std::max(w8a8::grouped_ws_bytes(R, E, 2 * I, H), w8a8::grouped_ws_bytes(R, E, H, I)));
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

const char* w8a8_status_str(int s) {
  switch (s) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL: return "null pointer";
    case W8A8_ERR_SHAPE: return "invalid shape";
    case W8A8_ERR_ALIGN: return "misaligned buffer";
    case W8A8_ERR_UNSUPPORTED: return "unsupported";
    case W8A8_ERR_WORKSPACE: return "workspace too small";
    case W8A8_ERR_LAUNCH: return "launch failed";
    default: return "unknown status";
  }
}

const char* w8a8_last_error(void) { return g_last_error.c_str(); }

int w8a8_abi_version(void) { return 1; }

int w8a8_dynamic_quant_ld(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                          float* x_scale, void* stream) {
  if (M < 0 || K < 1 || M >= kMaxDim * 4 || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "dynamic_quant: need M >= 0 and 1 <= K <= %d (M=%lld K=%lld)",
                W8A8_MAX_K, (long long)M, (long long)K);
  if (ldx < K || ldq < K)
    return fail(W8A8_ERR_SHAPE, "dynamic_quant: need ldx >= K and ldq >= K (ldx=%lld ldq=%lld K=%lld)",
                (long long)ldx, (long long)ldq, (long long)K);
  if (M == 0) return ok();
  if (!x || !q || !x_scale) return fail(W8A8_ERR_NULL, "dynamic_quant: null pointer");
  if (!aligned(x, 2) || !aligned(x_scale, 4))
    return fail(W8A8_ERR_ALIGN, "dynamic_quant: x must be 2-byte and x_scale 4-byte aligned");
  return launched(w8a8::launch_dynamic_quant(x, M, K, q, x_scale, false, (hipStream_t)stream, ldx, ldq),
                  "dynamic_quant");
}

int w8a8_dynamic_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* x_scale,
                       void* stream) {
  return w8a8_dynamic_quant_ld(x, M, K, K, q, K, x_scale, stream);
}

int w8a8_dynamic_quant_packed(const uint16_t* x, int64_t M, int64_t K, void* q_packed,
                              float* x_scale, void* stream) {
  if (M < 0 || K < 1 || M >= kMaxDim * 4 || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "dynamic_quant_packed: need M >= 0 and 1 <= K <= %d", W8A8_MAX_K);
  if (K % 8)
    return fail(W8A8_ERR_UNSUPPORTED, "dynamic_quant_packed: needs K %% 8 == 0 (K=%lld)", (long long)K);
  if (M == 0) return ok();
  if (!x || !q_packed || !x_scale) return fail(W8A8_ERR_NULL, "dynamic_quant_packed: null pointer");
  if (!aligned(x, 16) || !aligned(q_packed, 16) || !aligned(x_scale, 4))
    return fail(W8A8_ERR_ALIGN, "dynamic_quant_packed: x and q_packed need 16-byte alignment");
  return launched(w8a8::launch_dynamic_quant(x, M, K, reinterpret_cast<int8_t*>(q_packed), x_scale,
                                             true, (hipStream_t)stream),
                  "dynamic_quant_packed");
}

int64_t w8a8_packed_weight_bytes(int64_t E, int64_t N, int64_t K) {
  if (E < 0 || N < 0 || K < 0) return -1;
  return E * w8a8::round_up(N, 16) * w8a8::round_up(K, 64);
}

int w8a8_prepack_weight(const int8_t* w, int64_t E, int64_t N, int64_t K, void* w_packed,
                        void* stream) {
  if (E < 1 || N < 1 || K < 1 || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "prepack_weight: need E, N >= 1 and 1 <= K <= %d", W8A8_MAX_K);
  if (!w || !w_packed) return fail(W8A8_ERR_NULL, "prepack_weight: null pointer");
  if (!aligned(w_packed, 16)) return fail(W8A8_ERR_ALIGN, "prepack_weight: w_packed not 16-byte aligned");
  return launched(w8a8::launch_prepack(w, E, N, K, w_packed, (hipStream_t)stream), "prepack_weight");
}

// BF16-input branch of w8a8_linear: codes (packed-size bound) + scales
static int64_t bf16_codes_bytes(int64_t M, int64_t K) {
  return align256(w8a8::round_up(M, 16) * w8a8::round_up(K, 64));
}

int64_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return w8a8::plan_dense(M, N, K).ws_bytes + bf16_codes_bytes(M, K) + align256(4 * M);
}

int w8a8_linear(const int8_t* q, const float* x_scale, int64_t M, int64_t K, const void* w_packed,
                const float* w_scale, int64_t N, const uint16_t* bias, void* y, int out,
                void* workspace, int64_t ws_bytes, void* stream) {
  if (M < 0 || K < 1 || N < 1 || M >= kMaxDim || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "linear: need M >= 0, N >= 1, 1 <= K <= %d", W8A8_MAX_K);
  const bool packed = (out & W8A8_A_PACKED) != 0;
  out &= ~W8A8_A_PACKED;
  if (out != W8A8_OUT_BF16 && out != W8A8_OUT_I32)
    return fail(W8A8_ERR_UNSUPPORTED, "linear: unknown output kind %d", out);
  if (packed && w8a8::round_up(M, 16) * w8a8::round_up(K, 64) >= ((int64_t)1 << 32))
    return fail(W8A8_ERR_UNSUPPORTED, "linear: packed activations past 4 GB");
  if (M == 0) return ok();
  if (!x_scale) {
    // BF16 activation: quantize inside (w8a8_dynamic_quant's numerics), then multiply
    if (packed) return fail(W8A8_ERR_UNSUPPORTED, "linear: W8A8_A_PACKED needs INT8 codes and x_scale");
    if (!q || !w_packed || !w_scale || !y) return fail(W8A8_ERR_NULL, "linear: null pointer");
    if (!aligned(q, 2) || !aligned(w_packed, 16) || !aligned(w_scale, 4) || !aligned(y, 4) ||
        (bias && !aligned(bias, 2)))
      return fail(W8A8_ERR_ALIGN, "linear: x 2-byte, w_packed 16-byte, w_scale and y 4-byte alignment");
    const uint16_t* x = reinterpret_cast<const uint16_t*>(q);
    hipStream_t s = (hipStream_t)stream;
    if (w8a8::decode_fused_ok(M, K, x))
      return launched(w8a8::launch_decode_fused(x, M, K, w_packed, w_scale, N, bias, y, out, s),
                      "linear (fused quant)");
    const int64_t need = w8a8_linear_workspace_bytes(M, N, K);
    if (!workspace || ws_bytes < need || !aligned(workspace, 256))
      return fail(W8A8_ERR_WORKSPACE, "linear: BF16 input needs %lld workspace bytes (256-byte aligned), got %lld",
                  (long long)need, (long long)ws_bytes);
    int8_t* codes = reinterpret_cast<int8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + bf16_codes_bytes(M, K));
    // packed codes from 16 rows up (whole 1 KB blocks per 16 rows), row-major below
    const bool pk = M >= 16 && K % 8 == 0 && aligned(x, 16);
    hipError_t e = w8a8::launch_dynamic_quant(x, M, K, codes, scales, pk, s);
    if (e != hipSuccess) return launched(e, "linear: quant");
    const w8a8::DensePlan plan = w8a8::plan_dense(M, N, K);
    return launched(w8a8::launch_dense_gemm(plan, codes, scales, M, K, w_packed, w_scale, N, bias, y, out,
                                            pk, nullptr, s),
                    "linear");
  }
  if (!q || !w_packed || !w_scale || !y) return fail(W8A8_ERR_NULL, "linear: null pointer");
  if (!aligned(w_packed, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      (bias && !aligned(bias, 2)) || (packed && !aligned(q, 16)))
    return fail(W8A8_ERR_ALIGN,
                "linear: w_packed (and packed q) need 16-byte, scales and y 4-byte alignment");
  const w8a8::DensePlan plan = w8a8::plan_dense(M, N, K);
  if (plan.ws_bytes > 0 && (!workspace || ws_bytes < plan.ws_bytes || !aligned(workspace, 16)))
    return fail(W8A8_ERR_WORKSPACE, "linear: needs %lld workspace bytes (16-byte aligned), got %lld",
                (long long)plan.ws_bytes, (long long)ws_bytes);
  return launched(w8a8::launch_dense_gemm(plan, q, x_scale, M, K, w_packed, w_scale, N, bias, y, out,
                                          packed, workspace, (hipStream_t)stream),
                  "linear");
}

int w8a8_linear_ld(const int8_t* q, int64_t ldq, const float* x_scale, int64_t M, int64_t K,
                   const void* w_packed, const float* w_scale, int64_t N, const uint16_t* bias, void* y,
                   int64_t ldy, int out, void* workspace, int64_t ws_bytes, void* stream) {
  if (M < 0 || K < 1 || N < 1 || M >= kMaxDim || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "linear_ld: need M >= 0, N >= 1, 1 <= K <= %d", W8A8_MAX_K);
  if (ldq < K || ldy < N)
    return fail(W8A8_ERR_SHAPE, "linear_ld: need ldq >= K and ldy >= N (ldq=%lld ldy=%lld)", (long long)ldq,
                (long long)ldy);
  if (out != W8A8_OUT_BF16 && out != W8A8_OUT_I32)
    return fail(W8A8_ERR_UNSUPPORTED, "linear_ld: row-major INT8 codes only; unknown output kind %d", out);
  if (M == 0) return ok();
  if (!q || !x_scale || !w_packed || !w_scale || !y) return fail(W8A8_ERR_NULL, "linear_ld: null pointer");
  if (!aligned(w_packed, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      (bias && !aligned(bias, 2)))
    return fail(W8A8_ERR_ALIGN, "linear_ld: w_packed 16-byte, scales and y 4-byte alignment");
  const w8a8::DensePlan plan = w8a8::plan_dense(M, N, K);
  if (plan.ws_bytes > 0 && (!workspace || ws_bytes < plan.ws_bytes || !aligned(workspace, 16)))
    return fail(W8A8_ERR_WORKSPACE, "linear_ld: needs %lld workspace bytes (16-byte aligned), got %lld",
                (long long)plan.ws_bytes, (long long)ws_bytes);
  return launched(w8a8::launch_dense_gemm(plan, q, x_scale, M, K, w_packed, w_scale, N, bias, y, out, false,
                                          workspace, (hipStream_t)stream, nullptr, ldq, ldy),
                  "linear_ld");
}

int64_t w8a8_grouped_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K) {
  return w8a8::grouped_ws_bytes(R, E, N, K);
}

static int check_grouped(const char* who, int64_t R, int64_t E, int64_t N, int64_t K) {
  if (R < 0 || E < 1 || N < 1 || K < 1 || R >= kMaxDim || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "%s: need R >= 0, E >= 1, N >= 1, 1 <= K <= %d", who, W8A8_MAX_K);
  if (E > kMaxExperts)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: at most %lld experts", who, (long long)kMaxExperts);
  return W8A8_OK;
}

static int check_grouped_call(const char* who, const int8_t* a, const float* a_scale,
                              const int64_t* group_list, int64_t R, int64_t E, int64_t N, int64_t K,
                              const void* w_packed, const float* w_scale, void* y, int out) {
  int st = check_grouped(who, R, E, N, K);
  if (st) return st;
  if (out != W8A8_OUT_BF16 && out != W8A8_OUT_I32)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: unknown output kind %d", who, out);
  if (R == 0) return W8A8_OK;
  if (!a || !a_scale || !group_list || !w_packed || !w_scale || !y)
    return fail(W8A8_ERR_NULL, "%s: null pointer", who);
  if (!aligned(w_packed, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      !aligned(group_list, 8))
    return fail(W8A8_ERR_ALIGN, "%s: misaligned buffer", who);
  return W8A8_OK;
}

int w8a8_grouped_gemm(const int8_t* a, const float* a_scale, const int64_t* group_list, int64_t R,
                      int64_t E, int64_t N, int64_t K, const void* w_packed, const float* w_scale,
                      void* y, int out, void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_grouped_call("grouped_gemm", a, a_scale, group_list, R, E, N, K, w_packed, w_scale, y, out);
  if (st) return st;
  if (R == 0) return ok();
  const int64_t need = w8a8::grouped_ws_bytes(R, E, N, K);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
    return fail(W8A8_ERR_WORKSPACE, "grouped_gemm: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  st = check_group_list("grouped_gemm", group_list, E, R, stream);
  if (st) return st;
  return launched(w8a8::launch_grouped_gemm(a, a_scale, group_list, R, E, N, K, w_packed, w_scale, y,
                                            out, workspace, (hipStream_t)stream),
                  "grouped_gemm");
}

int w8a8_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int8_t* q, float* scale,
                      void* stream) {
  if (R < 0 || I < 1 || R >= kMaxDim * 4 || I > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "swiglu_quant: need R >= 0 and 1 <= I <= %d", W8A8_MAX_K);
  if (R == 0) return ok();
  if (!h || !q || !scale) return fail(W8A8_ERR_NULL, "swiglu_quant: null pointer");
  if (!aligned(h, 2) || !aligned(scale, 4)) return fail(W8A8_ERR_ALIGN, "swiglu_quant: misaligned buffer");
  return launched(w8a8::launch_swiglu_quant(h, R, I, q, scale, (hipStream_t)stream), "swiglu_quant");
}

int64_t w8a8_moe_workspace_bytes(int64_t R, int64_t E, int64_t H, int64_t I) {
  if (R <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return moe_layout(R, E, H, I).total;
}

int w8a8_moe_grouped(const void* x_rows, const float* x_scale, const int64_t* group_list, int64_t R,
                     int64_t E, int64_t H, int64_t I, const void* w13_packed,
                     const float* w13_scale, const void* w2_packed, const float* w2_scale,
                     uint16_t* y, void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_grouped("moe_grouped", R, E, 2 * I, H);
  if (st) return st;
  st = check_grouped("moe_grouped", R, E, H, I);
  if (st) return st;
  if (R == 0) return ok();
  if (!x_rows || !group_list || !w13_packed || !w13_scale || !w2_packed || !w2_scale || !y)
    return fail(W8A8_ERR_NULL, "moe_grouped: null pointer");
  if (!aligned(w13_packed, 16) || !aligned(w2_packed, 16) || !aligned(group_list, 8) ||
      !aligned(w13_scale, 4) || !aligned(w2_scale, 4) || !aligned(y, 4) ||
      (x_scale && !aligned(x_scale, 4)) || !aligned(x_rows, 2))
    return fail(W8A8_ERR_ALIGN, "moe_grouped: misaligned buffer");
  const MoeWs L = moe_layout(R, E, H, I);
  if (!workspace || ws_bytes < L.total || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "moe_grouped: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)L.total, (long long)ws_bytes);
  st = check_group_list("moe_grouped", group_list, E, R, stream);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  const int8_t* q1 = reinterpret_cast<const int8_t*>(x_rows);
  const float* s1 = x_scale;
  hipError_t err;
  if (!x_scale) {
    // rows arrived as BF16 without a per-token scale: quantize them first
    err = w8a8::launch_dynamic_quant(reinterpret_cast<const uint16_t*>(x_rows), R, H,
                                     reinterpret_cast<int8_t*>(ws + L.q1),
                                     reinterpret_cast<float*>(ws + L.s1), false, s);
    if (err != hipSuccess) return launched(err, "moe_grouped: dynamic_quant");
    q1 = reinterpret_cast<const int8_t*>(ws + L.q1);
    s1 = reinterpret_cast<const float*>(ws + L.s1);
  }
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  int8_t* q2 = reinterpret_cast<int8_t*>(ws + L.q2);
  float* s2 = reinterpret_cast<float*>(ws + L.s2);
  err = w8a8::launch_grouped_gemm(q1, s1, group_list, R, E, 2 * I, H, w13_packed, w13_scale, h,
                                  w8a8::kOutBf16, ws + L.inner, s);
  if (err != hipSuccess) return launched(err, "moe_grouped: W13");
  err = w8a8::launch_swiglu_quant(h, R, I, q2, s2, s);
  if (err != hipSuccess) return launched(err, "moe_grouped: swiglu_quant");
  err = w8a8::launch_grouped_gemm(q2, s2, group_list, R, E, H, I, w2_packed, w2_scale, y,
                                  w8a8::kOutBf16, ws + L.inner, s);
  return launched(err, "moe_grouped: W2");
}

// ---------------------------------------------------------------------------
// Around the MoE chain: route, INT8 gather, weighted combine, whole layer
// ---------------------------------------------------------------------------
static int check_route(const char* who, int64_t T, int64_t top_k, int64_t E) {
  if (T < 0 || top_k < 1 || E < 1 || T * top_k >= kMaxDim)
    return fail(W8A8_ERR_SHAPE, "%s: need T >= 0, top_k >= 1, E >= 1 and T * top_k < 2^31", who);
  if (E > kMaxExperts)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: at most %lld experts", who, (long long)kMaxExperts);
  return W8A8_OK;
}

int w8a8_moe_route(const int32_t* topk_ids, int64_t T, int64_t top_k, int64_t E,
                   int64_t* group_list, int32_t* row_token, int32_t* pair_row, void* stream) {
  int st = check_route("moe_route", T, top_k, E);
  if (st) return st;
  if (!group_list || (T > 0 && (!topk_ids || !row_token || !pair_row)))
    return fail(W8A8_ERR_NULL, "moe_route: null pointer");
  if (!aligned(group_list, 8) || !aligned(topk_ids, 4) || !aligned(row_token, 4) ||
      !aligned(pair_row, 4))
    return fail(W8A8_ERR_ALIGN, "moe_route: misaligned buffer");
  return launched(w8a8::launch_route(topk_ids, T, top_k, E, group_list, row_token, pair_row,
                                     (hipStream_t)stream),
                  "moe_route");
}

int w8a8_moe_gather(const int8_t* q, const float* scale, int64_t T, int64_t H,
                    const int32_t* row_token, int64_t R, int8_t* q_rows, float* s_rows,
                    void* stream) {
  if (T < 0 || R < 0 || H < 1 || T >= kMaxDim || R >= kMaxDim || H > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "moe_gather: need T >= 0, R >= 0 and 1 <= H <= %d", W8A8_MAX_K);
  if (R == 0) return ok();
  if (!q || !scale || !row_token || !q_rows || !s_rows)
    return fail(W8A8_ERR_NULL, "moe_gather: null pointer");
  if (!aligned(scale, 4) || !aligned(row_token, 4) || !aligned(s_rows, 4))
    return fail(W8A8_ERR_ALIGN, "moe_gather: misaligned buffer");
  return launched(w8a8::launch_gather_rows(q, scale, row_token, T, R, H, q_rows, s_rows,
                                           (hipStream_t)stream),
                  "moe_gather");
}

int w8a8_moe_combine(const uint16_t* y_rows, int64_t R, int64_t H, const int32_t* pair_row,
                     const float* topk_weights, int64_t T, int64_t top_k, uint16_t* out,
                     void* stream) {
  if (T < 0 || R < 0 || H < 1 || top_k < 1 || T * top_k >= kMaxDim || R >= kMaxDim ||
      H >= kMaxDim)
    return fail(W8A8_ERR_SHAPE, "moe_combine: need T >= 0, R >= 0, H >= 1, top_k >= 1");
  if (T == 0) return ok();
  if (!pair_row || !topk_weights || !out || (R > 0 && !y_rows))
    return fail(W8A8_ERR_NULL, "moe_combine: null pointer");
  if (!aligned(y_rows, 2) || !aligned(pair_row, 4) || !aligned(topk_weights, 4) ||
      !aligned(out, 2))
    return fail(W8A8_ERR_ALIGN, "moe_combine: misaligned buffer");
  return launched(w8a8::launch_combine(y_rows, pair_row, topk_weights, T, top_k, R, H, out,
                                       (hipStream_t)stream),
                  "moe_combine");
}

namespace {

struct LayerWs {
  int64_t q, s, gl, rt, pr, qr, sr, y, chain, total;
};

LayerWs layer_layout(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I) {
  const int64_t P = T * k;
  LayerWs w{};
  int64_t o = 0;
  w.q = o;  o += align256(T * H);          // int8 [T, H]: the tokens, quantized once
  w.s = o;  o += align256(T * 4);          // f32 [T]
  w.gl = o; o += align256(E * 8);          // int64 [E]
  w.rt = o; o += align256(P * 4);          // int32 [P]
  w.pr = o; o += align256(P * 4);          // int32 [T, k]
  w.qr = o; o += align256(P * H);          // int8 [P, H]
  w.sr = o; o += align256(P * 4);          // f32 [P]
  w.y = o;  o += align256(P * H * 2);      // BF16 [P, H]
  w.chain = o;
  o += moe_layout(P, E, H, I).total;
  w.total = o;
  return w;
}

}  // namespace

int64_t w8a8_moe_layer_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t H, int64_t I) {
  if (T <= 0 || top_k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return layer_layout(T, top_k, E, H, I).total;
}

int w8a8_moe_layer(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                   const float* topk_weights, int64_t top_k, int64_t E, int64_t I,
                   const void* w13_packed, const float* w13_scale, const void* w2_packed,
                   const float* w2_scale, uint16_t* out, void* workspace, int64_t ws_bytes,
                   void* stream) {
  int st = check_route("moe_layer", T, top_k, E);
  if (st) return st;
  const int64_t P = T * top_k;
  st = check_grouped("moe_layer", P, E, 2 * I, H);
  if (st) return st;
  st = check_grouped("moe_layer", P, E, H, I);
  if (st) return st;
  if (T == 0) return ok();
  if (!x || !topk_ids || !topk_weights || !w13_packed || !w13_scale || !w2_packed || !w2_scale ||
      !out)
    return fail(W8A8_ERR_NULL, "moe_layer: null pointer");
  if (!aligned(x, 2) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(w13_packed, 16) || !aligned(w2_packed, 16) || !aligned(w13_scale, 4) ||
      !aligned(w2_scale, 4) || !aligned(out, 2))
    return fail(W8A8_ERR_ALIGN, "moe_layer: misaligned buffer");
  const LayerWs L = layer_layout(T, top_k, E, H, I);
  if (!workspace || ws_bytes < L.total || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "moe_layer: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)L.total, (long long)ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  int8_t* q = reinterpret_cast<int8_t*>(ws + L.q);
  float* sc = reinterpret_cast<float*>(ws + L.s);
  int64_t* gl = reinterpret_cast<int64_t*>(ws + L.gl);
  int32_t* rt = reinterpret_cast<int32_t*>(ws + L.rt);
  int32_t* pr = reinterpret_cast<int32_t*>(ws + L.pr);
  int8_t* qr = reinterpret_cast<int8_t*>(ws + L.qr);
  float* sr = reinterpret_cast<float*>(ws + L.sr);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
  hipError_t err = w8a8::launch_dynamic_quant(x, T, H, q, sc, false, s);
  if (err != hipSuccess) return launched(err, "moe_layer: dynamic_quant");
  err = w8a8::launch_route(topk_ids, T, top_k, E, gl, rt, pr, s);
  if (err != hipSuccess) return launched(err, "moe_layer: route");
  err = w8a8::launch_gather_rows(q, sc, rt, T, P, H, qr, sr, s);
  if (err != hipSuccess) return launched(err, "moe_layer: gather");
  st = w8a8_moe_grouped(qr, sr, gl, P, E, H, I, w13_packed, w13_scale, w2_packed, w2_scale, y,
                        ws + L.chain, L.total - L.chain, stream);
  if (st) return st;
  return launched(w8a8::launch_combine(y, pr, topk_weights, T, top_k, P, H, out, s),
                  "moe_layer: combine");
}

// ---------------------------------------------------------------------------
// MXFP8 variant
// ---------------------------------------------------------------------------
static int64_t mx_payload_bytes(int64_t N, int64_t K) {
  return align256(w8a8::round_up(N, 16) * w8a8::round_up(K, 64));
}

static int check_mx_k(const char* who, int64_t K) {
  if (K < 32 || K > W8A8_MAX_K) return fail(W8A8_ERR_SHAPE, "%s: need 32 <= K <= %d", who, W8A8_MAX_K);
  if (K % 32)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: K = %lld is not a multiple of the MX group size 32", who,
                (long long)K);
  return W8A8_OK;
}

int w8a8_mx_quant(const uint16_t* x, int64_t M, int64_t K, uint8_t* e4m3, uint8_t* e8m0,
                  int scale_alg, void* stream) {
  int st = check_mx_k("mx_quant", K);
  if (st) return st;
  if (M < 0 || M >= kMaxDim) return fail(W8A8_ERR_SHAPE, "mx_quant: bad M");
  if (scale_alg != 0 && scale_alg != 1) return fail(W8A8_ERR_UNSUPPORTED, "mx_quant: scale_alg must be 0 or 1");
  if (M == 0) return ok();
  if (!x || !e4m3 || !e8m0) return fail(W8A8_ERR_NULL, "mx_quant: null pointer");
  if (!aligned(x, 16) || !aligned(e4m3, 8)) return fail(W8A8_ERR_ALIGN, "mx_quant: x needs 16-byte, e4m3 8-byte alignment");
  return launched(w8a8::launch_mx_quant(x, M, K, scale_alg, e4m3, false, e8m0, nullptr, 0,
                                        (hipStream_t)stream),
                  "mx_quant");
}

int w8a8_mx_resolve_block_fp8(const uint8_t* w_e4m3, const float* scale_inv, int64_t N, int64_t K,
                              int64_t BN, int64_t BK, uint16_t* w_bf16, void* stream) {
  if (N < 1 || K < 1 || BN < 1 || BK < 1 || N >= kMaxDim || K >= kMaxDim)
    return fail(W8A8_ERR_SHAPE, "mx_resolve: need N, K, BN, BK >= 1");
  if (!w_e4m3 || !scale_inv || !w_bf16) return fail(W8A8_ERR_NULL, "mx_resolve: null pointer");
  if (!aligned(scale_inv, 4) || !aligned(w_bf16, 2)) return fail(W8A8_ERR_ALIGN, "mx_resolve: misaligned buffer");
  return launched(w8a8::launch_mx_resolve(w_e4m3, scale_inv, N, K, BN, BK, w_bf16, (hipStream_t)stream),
                  "mx_resolve");
}

int64_t w8a8_mx_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return mx_payload_bytes(N, K) + align256(w8a8::mx_scale_kb_bytes(w8a8::round_up(N, 16), K));
}

int w8a8_mx_prepack_weight(const uint8_t* w_e4m3, const uint8_t* w_e8m0, int64_t N, int64_t K,
                           void* packed, void* stream) {
  int st = check_mx_k("mx_prepack_weight", K);
  if (st) return st;
  if (N < 1 || N >= kMaxDim) return fail(W8A8_ERR_SHAPE, "mx_prepack_weight: bad N");
  if (!w_e4m3 || !w_e8m0 || !packed) return fail(W8A8_ERR_NULL, "mx_prepack_weight: null pointer");
  if (!aligned(packed, 256)) return fail(W8A8_ERR_ALIGN, "mx_prepack_weight: packed needs 256-byte alignment");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = w8a8::launch_prepack(reinterpret_cast<const int8_t*>(w_e4m3), 1, N, K, packed, s);
  if (e != hipSuccess) return launched(e, "mx_prepack_weight: payload");
  e = w8a8::launch_mx_scale_relayout(w_e8m0, N, K, w8a8::round_up(N, 16),
                                     reinterpret_cast<uint8_t*>(packed) + mx_payload_bytes(N, K), s);
  return launched(e, "mx_prepack_weight: scales");
}

int64_t w8a8_mx_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return mx_payload_bytes(M, K) + align256(w8a8::mx_scale_kb_bytes(w8a8::round_up(M, 2), K));
}

int w8a8_mx_linear(const void* x, const uint8_t* x_e8m0, int64_t M, int64_t K, const void* w_packed,
                   int64_t N, uint16_t* y, int scale_alg, void* workspace, int64_t ws_bytes,
                   void* stream) {
  int st = check_mx_k("mx_linear", K);
  if (st) return st;
  if (M < 0 || N < 1 || M >= kMaxDim || N >= kMaxDim) return fail(W8A8_ERR_SHAPE, "mx_linear: bad M or N");
  if (scale_alg != 0 && scale_alg != 1) return fail(W8A8_ERR_UNSUPPORTED, "mx_linear: scale_alg must be 0 or 1");
  if (M == 0) return ok();
  if (!x || !w_packed || !y) return fail(W8A8_ERR_NULL, "mx_linear: null pointer");
  if (!aligned(w_packed, 256) || !aligned(y, 4) || !aligned(x, 16))
    return fail(W8A8_ERR_ALIGN, "mx_linear: x needs 16-byte, w_packed 256-byte, y 4-byte alignment");
  const int64_t need = w8a8_mx_linear_workspace_bytes(M, K);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "mx_linear: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  // workspace: the activation payload in P16x64 blocks, then its k-block-major scales
  uint8_t* a_payload = ws;
  uint8_t* a_scale_kb = ws + mx_payload_bytes(M, K);
  const int64_t Mp = w8a8::round_up(M, 2);  // even row count: dword-aligned scale pairs
  hipError_t e;
  if (!x_e8m0) {
    // BF16 activation: dynamic MX quantization, written straight into blocks
    e = w8a8::launch_mx_quant(reinterpret_cast<const uint16_t*>(x), M, K, scale_alg, a_payload, true,
                              nullptr, a_scale_kb, Mp, s);
    if (e != hipSuccess) return launched(e, "mx_linear: quant");
  } else {
    // pre-quantized activation: E4M3 [M, K] with its row-major E8M0 [M, K/32]
    e = w8a8::launch_prepack(reinterpret_cast<const int8_t*>(x), 1, M, K, a_payload, s);
    if (e != hipSuccess) return launched(e, "mx_linear: payload");
    e = w8a8::launch_mx_scale_relayout(x_e8m0, M, K, Mp, a_scale_kb, s);
    if (e != hipSuccess) return launched(e, "mx_linear: scales");
  }
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(w_packed);
  e = w8a8::launch_mx_gemm(a_payload, a_scale_kb, Mp, M, K, wp, wp + mx_payload_bytes(N, K), N, y, s);
  return launched(e, "mx_linear: gemm");
}

int w8a8_mx_gemm(const uint8_t* a_e4m3, const uint8_t* a_scale_kb, int64_t M, int64_t K,
                 const void* w_packed, int64_t N, uint16_t* y, void* stream) {
  int st = check_mx_k("mx_gemm", K);
  if (st) return st;
  if (M < 0 || N < 1 || M >= kMaxDim || N >= kMaxDim) return fail(W8A8_ERR_SHAPE, "mx_gemm: bad M or N");
  if (M == 0) return ok();
  if (!a_e4m3 || !a_scale_kb || !w_packed || !y) return fail(W8A8_ERR_NULL, "mx_gemm: null pointer");
  if (!aligned(a_e4m3, 256) || !aligned(a_scale_kb, 4) || !aligned(w_packed, 256) || !aligned(y, 2))
    return fail(W8A8_ERR_ALIGN, "mx_gemm: a needs 256-byte, scales 4-byte, w_packed 256-byte alignment");
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(w_packed);
  return launched(w8a8::launch_mx_gemm(a_e4m3, a_scale_kb, w8a8::round_up(M, 2), M, K, wp,
                                       wp + mx_payload_bytes(N, K), N, y, (hipStream_t)stream),
                  "mx_gemm");
}

// ---------------------------------------------------------------------------
// MXFP8 MoE: one-expert-at-a-time weight preparation and the grouped chain
// ---------------------------------------------------------------------------
int64_t w8a8_mx_moe_staging_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return N * K * 2;
}

int w8a8_mx_moe_prepare(uint8_t* w_e4m3, const float* scale_inv, int64_t E, int64_t N, int64_t K,
                        int64_t BN, int64_t BK, int scale_alg, uint8_t* w_e8m0, void* packed,
                        void* staging, int64_t staging_bytes, void* stream) {
  int st = check_mx_k("mx_moe_prepare", K);
  if (st) return st;
  if (E < 1 || N < 1 || BN < 1 || BK < 1 || N >= kMaxDim || E >= kMaxDim)
    return fail(W8A8_ERR_SHAPE, "mx_moe_prepare: need E, N, BN, BK >= 1");
  if (scale_alg != 0 && scale_alg != 1)
    return fail(W8A8_ERR_UNSUPPORTED, "mx_moe_prepare: scale_alg must be 0 or 1");
  if (!w_e4m3 || !scale_inv || !w_e8m0 || !staging)
    return fail(W8A8_ERR_NULL, "mx_moe_prepare: null pointer");
  if (!aligned(w_e4m3, 8) || (N * K) % 8 || !aligned(scale_inv, 4) || !aligned(staging, 16) ||
      (packed && !aligned(packed, 256)))
    return fail(W8A8_ERR_ALIGN, "mx_moe_prepare: misaligned buffer");
  if (staging_bytes < w8a8_mx_moe_staging_bytes(N, K))
    return fail(W8A8_ERR_WORKSPACE, "mx_moe_prepare: needs %lld staging bytes, got %lld",
                (long long)w8a8_mx_moe_staging_bytes(N, K), (long long)staging_bytes);
  hipStream_t s = (hipStream_t)stream;
  uint16_t* bf16 = reinterpret_cast<uint16_t*>(staging);
  const int64_t sn = (N + BN - 1) / BN, sk = (K + BK - 1) / BK;
  const int64_t stride = w8a8_mx_packed_bytes(N, K);
  for (int64_t e = 0; e < E; ++e) {
    // resolve one expert into the staging buffer, then write its MX payload
    // over its own FP8 source bytes and its scales into the scale buffer
    uint8_t* we = w_e4m3 + e * N * K;
    uint8_t* se = w_e8m0 + e * N * (K / 32);
    hipError_t err = w8a8::launch_mx_resolve(we, scale_inv + e * sn * sk, N, K, BN, BK, bf16, s);
    if (err != hipSuccess) return launched(err, "mx_moe_prepare: resolve");
    err = w8a8::launch_mx_quant(bf16, N, K, scale_alg, we, false, se, nullptr, 0, s);
    if (err != hipSuccess) return launched(err, "mx_moe_prepare: quant");
    if (packed) {
      uint8_t* pe = reinterpret_cast<uint8_t*>(packed) + e * stride;
      err = w8a8::launch_prepack(reinterpret_cast<const int8_t*>(we), 1, N, K, pe, s);
      if (err != hipSuccess) return launched(err, "mx_moe_prepare: prepack");
      err = w8a8::launch_mx_scale_relayout(se, N, K, w8a8::round_up(N, 16), pe + mx_payload_bytes(N, K), s);
      if (err != hipSuccess) return launched(err, "mx_moe_prepare: scales");
    }
  }
  return ok();
}

int w8a8_mx_swiglu_quant(const uint16_t* h, int64_t R, int64_t I, int scale_alg, uint8_t* e4m3,
                         uint8_t* e8m0, void* stream) {
  int st = check_mx_k("mx_swiglu_quant", I);
  if (st) return st;
  if (R < 0 || R >= kMaxDim) return fail(W8A8_ERR_SHAPE, "mx_swiglu_quant: bad R");
  if (scale_alg != 0 && scale_alg != 1)
    return fail(W8A8_ERR_UNSUPPORTED, "mx_swiglu_quant: scale_alg must be 0 or 1");
  if (R == 0) return ok();
  if (!h || !e4m3 || !e8m0) return fail(W8A8_ERR_NULL, "mx_swiglu_quant: null pointer");
  if (!aligned(h, 16) || !aligned(e4m3, 8))
    return fail(W8A8_ERR_ALIGN, "mx_swiglu_quant: h needs 16-byte, e4m3 8-byte alignment");
  return launched(w8a8::launch_mx_swiglu_quant(h, R, I, scale_alg, e4m3, e8m0, (hipStream_t)stream),
                  "mx_swiglu_quant");
}

namespace {

struct MxGroupWs {
  int64_t tiles, count, payload, scales, total;
};

MxGroupWs mx_group_layout(int64_t R, int64_t E, int64_t K) {
  const int64_t Rs = w8a8::mx_padded_rows(R, E);
  MxGroupWs w{};
  int64_t o = 0;
  w.tiles = o;   o += align256(w8a8::mx_max_tiles(R, E) * 16);   // int4 tile records
  w.count = o;   o += 256;                                        // int: records written
  w.payload = o; o += align256(Rs * w8a8::round_up(K, 64));       // P16x64 blocks, padded rows
  w.scales = o;  o += align256(w8a8::mx_scale_kb_bytes(Rs, K));   // [KB][Rs][2]
  w.total = o;
  return w;
}

int check_mx_grouped(const char* who, int64_t R, int64_t E, int64_t N, int64_t K, int scale_alg) {
  int st = check_mx_k(who, K);
  if (st) return st;
  if (R < 0 || E < 1 || N < 1 || R >= kMaxDim / 2 || N >= kMaxDim)
    return fail(W8A8_ERR_SHAPE, "%s: need R >= 0, E >= 1, N >= 1", who);
  if (E > kMaxExperts) return fail(W8A8_ERR_UNSUPPORTED, "%s: at most %lld experts", who, (long long)kMaxExperts);
  if (scale_alg != 0 && scale_alg != 1) return fail(W8A8_ERR_UNSUPPORTED, "%s: scale_alg must be 0 or 1", who);
  return W8A8_OK;
}

}  // namespace

int64_t w8a8_mx_moe_packed_bytes(int64_t E, int64_t N, int64_t K) {
  if (E < 1) return 0;
  return E * w8a8_mx_packed_bytes(N, K);
}

int64_t w8a8_mx_grouped_workspace_bytes(int64_t R, int64_t E, int64_t K) {
  if (R < 1 || E < 1 || K < 1) return 0;
  return mx_group_layout(R, E, K).total;
}

int w8a8_mx_grouped_gemm(const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E, int64_t N,
                         int64_t K, int act, const void* w_packed, int scale_alg, uint16_t* y,
                         void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_mx_grouped("mx_grouped_gemm", R, E, N, K, scale_alg);
  if (st) return st;
  if (act != W8A8_ACT_NONE && act != W8A8_ACT_SWIGLU)
    return fail(W8A8_ERR_UNSUPPORTED, "mx_grouped_gemm: unknown act %d", act);
  if (R == 0) return ok();
  if (!x || !group_list || !w_packed || !y) return fail(W8A8_ERR_NULL, "mx_grouped_gemm: null pointer");
  if (!aligned(x, 16) || !aligned(group_list, 8) || !aligned(w_packed, 256) || !aligned(y, 2))
    return fail(W8A8_ERR_ALIGN, "mx_grouped_gemm: misaligned buffer");
  const MxGroupWs L = mx_group_layout(R, E, K);
  if (!workspace || ws_bytes < L.total || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "mx_grouped_gemm: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)L.total, (long long)ws_bytes);
  st = check_group_list("mx_grouped_gemm", group_list, E, R, stream);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
  int* count = reinterpret_cast<int*>(ws + L.count);
  uint8_t* pay = reinterpret_cast<uint8_t*>(ws + L.payload);
  uint8_t* sc = reinterpret_cast<uint8_t*>(ws + L.scales);
  hipError_t err = w8a8::launch_mx_group_schedule(group_list, E, R, tiles, count, s);
  if (err != hipSuccess) return launched(err, "mx_grouped_gemm: schedule");
  const int64_t ldx = act == W8A8_ACT_SWIGLU ? 2 * K : K;
  err = w8a8::launch_mx_quant_tiles(x, ldx, K, act, tiles, count, R, E, scale_alg, pay, sc, s);
  if (err != hipSuccess) return launched(err, "mx_grouped_gemm: quant");
  const uint8_t* wp = reinterpret_cast<const uint8_t*>(w_packed);
  return launched(w8a8::launch_mx_grouped_gemm(pay, sc, R, E, K, tiles, count, wp,
                                               w8a8_mx_packed_bytes(N, K), mx_payload_bytes(N, K), N,
                                               y, s),
                  "mx_grouped_gemm: gemm");
}

int64_t w8a8_mx_moe_workspace_bytes(int64_t R, int64_t E, int64_t H, int64_t I) {
  if (R < 1 || E < 1 || H < 1 || I < 1) return 0;
  const MxGroupWs a = mx_group_layout(R, E, H), b = mx_group_layout(R, E, I);
  return std::max(a.total, b.total) + align256(R * 2 * I * 2);
}

int w8a8_mx_moe_grouped(const uint16_t* x_rows, const int64_t* group_list, int64_t R, int64_t E,
                        int64_t H, int64_t I, const void* w13_packed, const void* w2_packed,
                        int scale_alg, uint16_t* y, void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_mx_grouped("mx_moe_grouped", R, E, 2 * I, H, scale_alg);
  if (st) return st;
  st = check_mx_grouped("mx_moe_grouped", R, E, H, I, scale_alg);
  if (st) return st;
  if (R == 0) return ok();
  if (!x_rows || !group_list || !w13_packed || !w2_packed || !y)
    return fail(W8A8_ERR_NULL, "mx_moe_grouped: null pointer");
  if (!aligned(x_rows, 16) || !aligned(group_list, 8) || !aligned(w13_packed, 256) ||
      !aligned(w2_packed, 256) || !aligned(y, 2))
    return fail(W8A8_ERR_ALIGN, "mx_moe_grouped: misaligned buffer");
  const int64_t need = w8a8_mx_moe_workspace_bytes(R, E, H, I);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "mx_moe_grouped: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  st = check_group_list("mx_moe_grouped", group_list, E, R, stream);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  // the two stages share the schedule and the activation region (W13's MX
  // input is dead once W13 has run); h [R, 2I] BF16 sits after it
  const MxGroupWs L = mx_group_layout(R, E, std::max(H, I));
  int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
  int* count = reinterpret_cast<int*>(ws + L.count);
  uint8_t* pay = reinterpret_cast<uint8_t*>(ws + L.payload);
  const int64_t Rs = w8a8::mx_padded_rows(R, E);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + need - align256(R * 2 * I * 2));
  const uint8_t* w13 = reinterpret_cast<const uint8_t*>(w13_packed);
  const uint8_t* w2 = reinterpret_cast<const uint8_t*>(w2_packed);
  hipError_t err = w8a8::launch_mx_group_schedule(group_list, E, R, tiles, count, s);
  if (err != hipSuccess) return launched(err, "mx_moe_grouped: schedule");
  // W13: MX quant of the rows, grouped block-scaled matmul -> h
  uint8_t* sc1 = pay + align256(Rs * w8a8::round_up(H, 64));
  err = w8a8::launch_mx_quant_tiles(x_rows, H, H, 0, tiles, count, R, E, scale_alg, pay, sc1, s);
  if (err != hipSuccess) return launched(err, "mx_moe_grouped: quant");
  err = w8a8::launch_mx_grouped_gemm(pay, sc1, R, E, H, tiles, count, w13, w8a8_mx_packed_bytes(2 * I, H),
                                     mx_payload_bytes(2 * I, H), 2 * I, h, s);
  if (err != hipSuccess) return launched(err, "mx_moe_grouped: W13");
  // SwiGLU -> BF16 -> MX quant, grouped block-scaled matmul -> y
  uint8_t* sc2 = pay + align256(Rs * w8a8::round_up(I, 64));
  err = w8a8::launch_mx_quant_tiles(h, 2 * I, I, 1, tiles, count, R, E, scale_alg, pay, sc2, s);
  if (err != hipSuccess) return launched(err, "mx_moe_grouped: swiglu quant");
  return launched(w8a8::launch_mx_grouped_gemm(pay, sc2, R, E, I, tiles, count, w2,
                                               w8a8_mx_packed_bytes(H, I), mx_payload_bytes(H, I), H, y, s),
                  "mx_moe_grouped: W2");
}


// ---------------------------------------------------------------------------
// W4A16 weight variant
// ---------------------------------------------------------------------------
// rows of one W4A16 / FP4 linear: row groups of 16 (FP4) or 32 (INT4) rows
// along the grid's y, which holds at most 65535
constexpr int64_t kW4MaxRows = (int64_t)16 * 65535;

static int check_w4(const char* who, int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "%s: need N >= 1 and 1 <= K <= %d", who, W8A8_MAX_K);
  if (K % 32)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: K = %lld is not a multiple of the group size 32", who,
                (long long)K);
  return W8A8_OK;
}

int64_t w8a8_w4a16_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return w8a8::w4_packed_bytes(N, K);
}

int64_t w8a8_w4a16_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return w8a8::w4_linear_ws_bytes(M, K);
}

int w8a8_w4a16_quant_weight(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* scale,
                            void* packed, void* stream) {
  int st = check_w4("w4a16_quant_weight", N, K);
  if (st) return st;
  if (!w || (!q && !scale && !packed)) return fail(W8A8_ERR_NULL, "w4a16_quant_weight: null pointer");
  if (!aligned(w, 2) || (scale && !aligned(scale, 2)) || (packed && !aligned(packed, 16)))
    return fail(W8A8_ERR_ALIGN, "w4a16_quant_weight: misaligned buffer");
  return launched(w8a8::launch_w4_quant_pack(w, N, K, q, scale, reinterpret_cast<uint8_t*>(packed),
                                             (hipStream_t)stream),
                  "w4a16_quant_weight");
}

int w8a8_w4a16_pack(const int8_t* q, const uint16_t* scale, int64_t N, int64_t K, void* packed,
                    void* stream) {
  int st = check_w4("w4a16_pack", N, K);
  if (st) return st;
  if (!q || !scale || !packed) return fail(W8A8_ERR_NULL, "w4a16_pack: null pointer");
  if (!aligned(scale, 2) || !aligned(packed, 16)) return fail(W8A8_ERR_ALIGN, "w4a16_pack: misaligned buffer");
  return launched(w8a8::launch_w4_pack(q, scale, N, K, reinterpret_cast<uint8_t*>(packed),
                                       (hipStream_t)stream),
                  "w4a16_pack");
}

int64_t w8a8_fp4_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return w8a8::fp4_packed_bytes(N, K);
}

int w8a8_fp4_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                          void* packed, void* stream) {
  int st = check_w4("fp4_quant_weight", N, K);
  if (st) return st;
  if (!w || (!codes && !scales && !packed)) return fail(W8A8_ERR_NULL, "fp4_quant_weight: null pointer");
  if (!aligned(w, 2) || (packed && !aligned(packed, 16)))
    return fail(W8A8_ERR_ALIGN, "fp4_quant_weight: misaligned buffer");
  return launched(w8a8::launch_fp4_quant_pack(w, N, K, codes, scales, reinterpret_cast<uint8_t*>(packed),
                                              (hipStream_t)stream),
                  "fp4_quant_weight");
}

int w8a8_fp4_linear(const uint16_t* x, int64_t M, int64_t K, const void* w_packed, int64_t N,
                    uint16_t* y, void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_w4("fp4_linear", N, K);
  if (st) return st;
  if (M < 0 || M > kW4MaxRows)
    return fail(W8A8_ERR_SHAPE, "fp4_linear: need 0 <= M <= %lld (rows of one launch)", (long long)kW4MaxRows);
  if (M == 0) return ok();
  if (!x || !w_packed || !y) return fail(W8A8_ERR_NULL, "fp4_linear: null pointer");
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 2))
    return fail(W8A8_ERR_ALIGN, "fp4_linear: x and w_packed need 16-byte alignment");
  const int64_t need = w8a8::w4_linear_ws_bytes(M, K);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
    return fail(W8A8_ERR_WORKSPACE, "fp4_linear: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  return launched(w8a8::launch_fp4_linear(x, M, K, reinterpret_cast<const uint8_t*>(w_packed), N, y, workspace,
                                          (hipStream_t)stream),
                  "fp4_linear");
}

// ---------------------------------------------------------------------------
// grouped form (low-bit expert weights)
// ---------------------------------------------------------------------------
static int check_lowbit_grouped(const char* who, int fmt, int64_t R, int64_t E, int64_t N, int64_t K) {
  if (fmt != W8A8_LOWBIT_INT4 && fmt != W8A8_LOWBIT_FP4)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: unknown weight format %d", who, fmt);
  int st = check_w4(who, N, K);
  if (st) return st;
  if (R < 0 || R >= kMaxDim || E < 1)
    return fail(W8A8_ERR_SHAPE, "%s: need 0 <= R < 2^31 and E >= 1", who);
  if (E > kMaxExperts) return fail(W8A8_ERR_UNSUPPORTED, "%s: at most %lld experts", who, (long long)kMaxExperts);
  if (N % 16)
    return fail(W8A8_ERR_UNSUPPORTED, "%s: N = %lld is not a multiple of 16 (one packed column block)", who,
                (long long)N);
  return W8A8_OK;
}

int w8a8_w4a16_grouped_gemm(int fmt, const uint16_t* x, const int64_t* group_list, int64_t R, int64_t E,
                            int64_t N, int64_t K, const void* w_packed, uint16_t* y, void* stream) {
  int st = check_lowbit_grouped("w4a16_grouped_gemm", fmt, R, E, N, K);
  if (st) return st;
  if (R == 0) return ok();
  if (!x || !group_list || !w_packed || !y) return fail(W8A8_ERR_NULL, "w4a16_grouped_gemm: null pointer");
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 8) || !aligned(group_list, 8))
    return fail(W8A8_ERR_ALIGN, "w4a16_grouped_gemm: x and w_packed need 16-byte, y 8-byte alignment");
  st = check_group_list("w4a16_grouped_gemm", group_list, E, R, stream);
  if (st) return st;
  return launched(w8a8::launch_lowbit_grouped(fmt, x, group_list, R, E, N, K,
                                              reinterpret_cast<const uint8_t*>(w_packed), y, (hipStream_t)stream),
                  "w4a16_grouped_gemm");
}

int w8a8_w4a16_swiglu(const uint16_t* h, int64_t R, int64_t I, uint16_t* a, void* stream) {
  if (R < 0 || I < 1 || R >= kMaxDim || I >= kMaxDim / 2)
    return fail(W8A8_ERR_SHAPE, "w4a16_swiglu: need R >= 0 and I >= 1");
  if (R == 0) return ok();
  if (!h || !a) return fail(W8A8_ERR_NULL, "w4a16_swiglu: null pointer");
  if (!aligned(h, 2) || !aligned(a, 2)) return fail(W8A8_ERR_ALIGN, "w4a16_swiglu: misaligned buffer");
  return launched(w8a8::launch_lowbit_swiglu(h, R, I, a, (hipStream_t)stream), "w4a16_swiglu");
}

int64_t w8a8_w4a16_moe_workspace_bytes(int64_t R, int64_t H, int64_t I) {
  if (R < 1 || H < 1 || I < 1) return 0;
  return align256(R * 2 * I * 2) + align256(R * I * 2);
}

int w8a8_w4a16_moe_grouped(int fmt, const uint16_t* x_rows, const int64_t* group_list, int64_t R, int64_t E,
                           int64_t H, int64_t I, const void* w13_packed, const void* w2_packed, uint16_t* y,
                           void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_lowbit_grouped("w4a16_moe_grouped", fmt, R, E, 2 * I, H);
  if (st) return st;
  st = check_lowbit_grouped("w4a16_moe_grouped", fmt, R, E, H, I);
  if (st) return st;
  if (R == 0) return ok();
  if (!x_rows || !group_list || !w13_packed || !w2_packed || !y)
    return fail(W8A8_ERR_NULL, "w4a16_moe_grouped: null pointer");
  if (!aligned(x_rows, 16) || !aligned(w13_packed, 16) || !aligned(w2_packed, 16) || !aligned(y, 8) ||
      !aligned(group_list, 8))
    return fail(W8A8_ERR_ALIGN, "w4a16_moe_grouped: misaligned buffer");
  const int64_t need = w8a8_w4a16_moe_workspace_bytes(R, H, I);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256))
    return fail(W8A8_ERR_WORKSPACE, "w4a16_moe_grouped: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  st = check_group_list("w4a16_moe_grouped", group_list, E, R, stream);
  if (st) return st;
  uint16_t* h = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* a = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(workspace) + align256(R * 2 * I * 2));
  const hipStream_t s = (hipStream_t)stream;
  hipError_t err = w8a8::launch_lowbit_grouped(fmt, x_rows, group_list, R, E, 2 * I, H,
                                               reinterpret_cast<const uint8_t*>(w13_packed), h, s);
  if (err != hipSuccess) return launched(err, "w4a16_moe_grouped: W13");
  err = w8a8::launch_lowbit_swiglu(h, R, I, a, s);
  if (err != hipSuccess) return launched(err, "w4a16_moe_grouped: swiglu");
  return launched(w8a8::launch_lowbit_grouped(fmt, a, group_list, R, E, H, I,
                                              reinterpret_cast<const uint8_t*>(w2_packed), y, s),
                  "w4a16_moe_grouped: W2");
}

int w8a8_w4a16_linear(const uint16_t* x, int64_t M, int64_t K, const void* w_packed, int64_t N,
                      uint16_t* y, void* workspace, int64_t ws_bytes, void* stream) {
  int st = check_w4("w4a16_linear", N, K);
  if (st) return st;
  if (M < 0 || M > kW4MaxRows)
    return fail(W8A8_ERR_SHAPE, "w4a16_linear: need 0 <= M <= %lld (rows of one launch)", (long long)kW4MaxRows);
  if (M == 0) return ok();
  if (!x || !w_packed || !y) return fail(W8A8_ERR_NULL, "w4a16_linear: null pointer");
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 2))
    return fail(W8A8_ERR_ALIGN, "w4a16_linear: x and w_packed need 16-byte alignment");
  const int64_t need = w8a8::w4_linear_ws_bytes(M, K);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256)))
    return fail(W8A8_ERR_WORKSPACE, "w4a16_linear: needs %lld workspace bytes (256-byte aligned), got %lld",
                (long long)need, (long long)ws_bytes);
  return launched(w8a8::launch_w4a16_linear(x, M, K, reinterpret_cast<const uint8_t*>(w_packed), N, y, workspace,
                                            (hipStream_t)stream),
                  "w4a16_linear");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// static W8A8
// ---------------------------------------------------------------------------

static bool finite_f(float v) { return v == v && v - v == 0.0f; }

int w8a8_static_quant(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                      float input_offset, int8_t* q, void* stream) {
  if (M < 0 || K < 1 || M >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "static_quant: need M >= 0, 1 <= K <= %d", W8A8_MAX_K);
  if (!(input_scale > 0.0f) || !finite_f(input_scale) || !finite_f(input_offset))
    return fail(W8A8_ERR_SHAPE, "static_quant: input_scale must be > 0 and finite, input_offset finite");
  if (M == 0) return ok();
  if (!x || !q) return fail(W8A8_ERR_NULL, "static_quant: null pointer");
  if (!aligned(x, 2)) return fail(W8A8_ERR_ALIGN, "static_quant: x not 2-byte aligned");
  return launched(w8a8::launch_static_quant(x, M * K, input_scale, input_offset, q, (hipStream_t)stream),
                  "static_quant");
}

int w8a8_static_quant_packed(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                             float input_offset, void* q_packed, void* stream) {
  if (M < 0 || K < 1 || M >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "static_quant_packed: need M >= 0, 1 <= K <= %d", W8A8_MAX_K);
  if (!(input_scale > 0.0f) || !finite_f(input_scale) || !finite_f(input_offset))
    return fail(W8A8_ERR_SHAPE, "static_quant_packed: input_scale must be > 0 and finite, input_offset finite");
  if (w8a8::round_up(M, 16) * w8a8::round_up(K, 64) >= ((int64_t)1 << 32))
    return fail(W8A8_ERR_UNSUPPORTED, "static_quant_packed: packed activations past 4 GB");
  if (M == 0) return ok();
  if (!x || !q_packed) return fail(W8A8_ERR_NULL, "static_quant_packed: null pointer");
  if (!aligned(x, 2) || !aligned(q_packed, 16))
    return fail(W8A8_ERR_ALIGN, "static_quant_packed: x 2-byte, q_packed 16-byte alignment");
  return launched(w8a8::launch_static_quant_packed(x, M, K, input_scale, input_offset, q_packed,
                                                   (hipStream_t)stream),
                  "static_quant_packed");
}

int w8a8_static_prepare(const int8_t* w, int64_t N, int64_t K, const float* w_scale,
                        const uint16_t* bias, float input_scale, float input_offset,
                        float* deq_scale, int32_t* quant_bias, void* stream) {
  if (N < 1 || K < 1 || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "static_prepare: need N >= 1, 1 <= K <= %d", W8A8_MAX_K);
  if (!(input_scale > 0.0f) || !finite_f(input_scale) || !finite_f(input_offset))
    return fail(W8A8_ERR_SHAPE, "static_prepare: input_scale must be > 0 and finite, input_offset finite");
  if (!w || !w_scale || !deq_scale || !quant_bias) return fail(W8A8_ERR_NULL, "static_prepare: null pointer");
  if (!aligned(w_scale, 4) || !aligned(deq_scale, 4) || !aligned(quant_bias, 4) || (bias && !aligned(bias, 2)))
    return fail(W8A8_ERR_ALIGN, "static_prepare: scales and quant_bias 4-byte, bias 2-byte alignment");
  return launched(w8a8::launch_static_prepare(w, N, K, w_scale, bias, input_scale, input_offset, deq_scale,
                                              quant_bias, (hipStream_t)stream),
                  "static_prepare");
}

int w8a8_static_linear(const int8_t* q, int64_t M, int64_t K, const void* w_packed,
                       const float* deq_scale, const int32_t* quant_bias, int64_t N, void* y,
                       int out, void* stream) {
  if (M < 0 || K < 1 || N < 1 || M >= kMaxDim || N >= kMaxDim || K > W8A8_MAX_K)
    return fail(W8A8_ERR_SHAPE, "static_linear: need M >= 0, N >= 1, 1 <= K <= %d", W8A8_MAX_K);
  const bool packed = (out & W8A8_A_PACKED) != 0;
  out &= ~W8A8_A_PACKED;
  if (out != W8A8_OUT_BF16 && out != W8A8_OUT_I32)
    return fail(W8A8_ERR_UNSUPPORTED, "static_linear: unknown output kind %d", out);
  if (packed && w8a8::round_up(M, 16) * w8a8::round_up(K, 64) >= ((int64_t)1 << 32))
    return fail(W8A8_ERR_UNSUPPORTED, "static_linear: packed activations past 4 GB");
  if (M == 0) return ok();
  if (!q || !w_packed || !deq_scale || !quant_bias || !y) return fail(W8A8_ERR_NULL, "static_linear: null pointer");
  if (!aligned(w_packed, 16) || !aligned(deq_scale, 4) || !aligned(quant_bias, 4) || !aligned(y, 4) ||
      (packed && !aligned(q, 16)))
    return fail(W8A8_ERR_ALIGN,
                "static_linear: w_packed (and packed q) 16-byte, deq_scale, quant_bias and y 4-byte alignment");
  const w8a8::DensePlan plan = w8a8::plan_dense(M, N, K);
  return launched(w8a8::launch_dense_gemm(plan, q, nullptr, M, K, w_packed, deq_scale, N, nullptr, y, out,
                                          packed, nullptr, (hipStream_t)stream, quant_bias),
                  "static_linear");
}

// ---------------------------------------------------------------------------
// Grouped GEMM without a caller workspace. Its schedule goes to `scratch`, a
// device array of this library: each GPU holds its own copy at its own
// address until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory, so the device address is taken once per
// device with hipGetSymbolAddress and only that address reaches a kernel.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = w8a8::group_sched_bytes(kMaxExperts);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchDevices];  // device address of `scratch`, per device

// device address of the current device's `scratch` (taken on its first use)
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W8A8_ERR_LAUNCH, "grouped_gemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(W8A8_ERR_UNSUPPORTED, "grouped_gemm_noalloc: device %d past the %d this library tracks", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(W8A8_ERR_LAUNCH, "grouped_gemm_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return W8A8_OK;
}
}  // namespace

int w8a8_grouped_gemm_noalloc(const int8_t* a, const float* a_scale, const int64_t* group_list, int64_t R,
                              int64_t E, int64_t N, int64_t K, const void* w_packed, const float* w_scale,
                              void* y, int out, void* stream) {
  int st = check_grouped_call("grouped_gemm_noalloc", a, a_scale, group_list, R, E, N, K, w_packed, w_scale, y,
                              out);
  if (st) return st;
  if (R == 0) return ok();
  st = check_group_list("grouped_gemm_noalloc", group_list, E, R, stream);
  if (st) return st;
  const int64_t need = w8a8::grouped_ws_bytes(R, E, N, K);
  if (need > kScratchBytes)
    return fail(W8A8_ERR_UNSUPPORTED, "grouped_gemm_noalloc: the schedule of %lld experts needs %lld bytes, "
                "past the library's %lld-byte scratch", (long long)E, (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa) return sa;
  // the schedule kernel rewrites every byte the GEMM reads (work-queue
  // counters included), so nothing left by an earlier call matters
  return launched(w8a8::launch_grouped_gemm(a, a_scale, group_list, R, E, N, K, w_packed, w_scale, y, out, ws,
                                            (hipStream_t)stream),
                  "grouped_gemm_noalloc");
}
