// C ABI of the library (declared in include/svdq.h): argument validation on
// the host, workspace layout, and the launch sequence of each entry point.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "kernels.h"
#include "svdq.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SVDQ_OK;
}

// Debug mode: SVDQ_DEBUG set to 1, true, yes or on (any case), read once per
// process. Every entry point then synchronises its stream after each launch
// (unless the stream is being captured into a graph) and reports any error the
// kernels raised as SVDQ_ERR_HIP, naming the launch.
bool parse_debug_flag(const char* v) {
  if (v == nullptr) return false;
  char b[8] = {0};
  for (int i = 0; i < 7 && v[i]; ++i) b[i] = (char)((v[i] >= 'A' && v[i] <= 'Z') ? v[i] - 'A' + 'a' : v[i]);
  if (strlen(v) > 7) return false;
  return !strcmp(b, "1") || !strcmp(b, "true") || !strcmp(b, "yes") || !strcmp(b, "on");
}

bool debug_mode() {
  static const bool on = parse_debug_flag(getenv("SVDQ_DEBUG"));
  return on;
}

// After a launch (or an entry point's launch sequence): a launch error becomes
// SVDQ_ERR_HIP; in debug mode the stream is synchronised and checked too.
int launched(hipError_t e, const char* what, hipStream_t s) {
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  if (debug_mode()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e == hipSuccess && cs == hipStreamCaptureStatusNone) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s (checked after the launch): %s", what, hipGetErrorString(e));
  }
  return SVDQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;
};
Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{name, b, b + bytes};
}
bool overlaps(const Range& a, const Range& b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// every output against every input and every other output
int check_alias(const Range* in, int n_in, const Range* out, int n_out) {
  for (int o = 0; o < n_out; ++o) {
    if (out[o].lo == 0) continue;
    for (int i = 0; i < n_in; ++i)
      if (in[i].lo != 0 && overlaps(out[o], in[i]))
        return fail(SVDQ_ERR_ALIAS, "output %s overlaps input %s", out[o].name, in[i].name);
    for (int p = o + 1; p < n_out; ++p)
      if (out[p].lo != 0 && overlaps(out[o], out[p]))
        return fail(SVDQ_ERR_ALIAS, "output %s overlaps output %s", out[o].name, out[p].name);
  }
  return SVDQ_OK;
}

constexpr int64_t kMaxDim = int64_t(1) << 24;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int check_mk(int64_t M, int64_t K, int64_t R) {
  if (M < 0) return fail(SVDQ_ERR_SHAPE, "M = %lld is negative", (long long)M);
  if (K <= 0 || K % 16 != 0)
    return fail(SVDQ_ERR_SHAPE, "K = %lld must be a positive multiple of 16", (long long)K);
  if (R < 0) return fail(SVDQ_ERR_SHAPE, "R = %lld is negative", (long long)R);
  if (R % 16 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "R = %lld: the kernels need R to be a multiple of 16", (long long)R);
  if (M > kMaxDim || K > kMaxDim || R > kMaxDim)
    return fail(SVDQ_ERR_UNSUPPORTED, "dimension above 2^24 (M=%lld K=%lld R=%lld)", (long long)M,
                (long long)K, (long long)R);
  return SVDQ_OK;
}

// The quantisation kernels address x, proj_down, lora_act and the code buffers
// through buffer descriptors with 32-bit sizes; keep each under 2 GiB.
int check_rsrc_sizes(int64_t M, int64_t K, int64_t R) {
  const int64_t lim = int64_t(1) << 31;
  if (M * K * 2 >= lim || K * R * 2 >= lim || M * R * 2 >= lim ||
      (int64_t)svdq::packed_weight_bytes(M, K) >= lim)
    return fail(SVDQ_ERR_UNSUPPORTED, "a tensor of the quantisation step exceeds 2 GiB (M=%lld K=%lld R=%lld)",
                (long long)M, (long long)K, (long long)R);
  return SVDQ_OK;
}

// The packed-operand GEMM addresses both packed buffers through 32-bit buffer
// offsets (out-of-range panels read as zero).
int check_packed_gemm_sizes(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = int64_t(1) << 31;
  if ((int64_t)svdq::packed_weight_bytes(M, K) >= lim || (int64_t)svdq::packed_weight_bytes(N, K) >= lim)
    return fail(SVDQ_ERR_UNSUPPORTED, "a packed GEMM operand exceeds 2 GiB (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  return SVDQ_OK;
}

int check_ptrs(const char* const* names, const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return fail(SVDQ_ERR_NULL, "%s is NULL", names[i]);
  for (int i = 0; i < n; ++i)
    if (!aligned16(ptrs[i])) return fail(SVDQ_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  return SVDQ_OK;
}

// Scratch of the quantisation step: fp32 partial sums of the down-projection
// when it splits K across workgroups (small M), otherwise none.
size_t quant_ws_bytes(int64_t M, int64_t K, int64_t R) {
  return R > 0 ? align256(svdq::quant_lora_workspace_bytes(M, K, R)) : 0;
}

// Whole-layer workspace: the quantised activations (canonical, or packed when
// the weight is packed: the packed form is never smaller), lora_act, and the
// quantisation step's scratch.
struct LinearWs {
  size_t act, ascales, lora, partial, total;
};
LinearWs linear_ws(int64_t M, int64_t K, int64_t R) {
  LinearWs w;
  w.act = 0;
  w.ascales = align256((size_t)M * (size_t)(K / 2));
  const size_t canonical_end = align256(w.ascales + (size_t)(K / 16) * (size_t)M);
  const size_t packed_end = align256(svdq::packed_weight_bytes(M, K));
  w.lora = canonical_end > packed_end ? canonical_end : packed_end;
  w.partial = align256(w.lora + (size_t)M * (size_t)R * 2);
  w.total = w.partial + quant_ws_bytes(M, K, R);
  return w;
}

// enqueue a1 (+ a2): pointers already validated
int run_quantize(const void* x, const void* smooth, int64_t M, int64_t K, const void* proj_down,
                 int64_t R, void* qact, void* ascales, void* lora_act, void* scratch, bool packed_out,
                 hipStream_t s, const void* gscale = nullptr) {
  hipError_t e;
  const uint16_t* gs = static_cast<const uint16_t*>(gscale);
  if (R == 0 && !packed_out) {
    e = svdq::launch_quant_act(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth),
                               static_cast<uint8_t*>(qact), static_cast<uint8_t*>(ascales), M, K, s, gs);
  } else {
    e = svdq::launch_quant_lora(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth),
                                static_cast<const uint16_t*>(proj_down), static_cast<uint8_t*>(qact),
                                static_cast<uint8_t*>(ascales), static_cast<uint16_t*>(lora_act),
                                static_cast<float*>(scratch), M, K, R, packed_out, s, gs);
  }
  if (int st = launched(e, "quantisation", s)) return st;
  return ok();
}

int check_gemm_weight(int weight_layout, const void* wscales) {
  if (weight_layout != SVDQ_WEIGHT_CANONICAL && weight_layout != SVDQ_WEIGHT_PACKED)
    return fail(SVDQ_ERR_INVALID, "weight_layout %d is not a known layout", weight_layout);
  if (weight_layout == SVDQ_WEIGHT_PACKED && wscales != nullptr)
    return fail(SVDQ_ERR_INVALID, "wscales must be NULL with the packed layout (the buffer holds them)");
  if (weight_layout == SVDQ_WEIGHT_CANONICAL && wscales == nullptr)
    return fail(SVDQ_ERR_NULL, "wscales is NULL");
  return SVDQ_OK;
}

size_t weight_bytes(int weight_layout, int64_t N, int64_t K) {
  return weight_layout == SVDQ_WEIGHT_PACKED ? svdq::packed_weight_bytes(N, K)
                                             : (size_t)N * (size_t)(K / 2);
}

}  // namespace

extern "C" {

int svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_NULL: return "null pointer";
    case SVDQ_ERR_SHAPE: return "invalid shape";
    case SVDQ_ERR_UNSUPPORTED: return "unsupported by these kernels";
    case SVDQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SVDQ_ERR_WORKSPACE: return "workspace too small";
    case SVDQ_ERR_ALIAS: return "output overlaps another buffer";
    case SVDQ_ERR_HIP: return "HIP error";
    case SVDQ_ERR_INVALID: return "invalid argument";
    default: return "unknown status";
  }
}

const char* svdq_last_error(void) { return g_last_error.c_str(); }

int svdq_debug_mode(void) { return debug_mode() ? 1 : 0; }

int svdq_set_gemm_tile(int tile, int* previous) {
  if (tile < 0 || tile > 4) return fail(SVDQ_ERR_INVALID, "tile = %d is not 0..4", tile);
  const int prev = svdq::set_gemm_tile(tile);
  if (previous != nullptr) *previous = prev;
  return SVDQ_OK;
}

size_t svdq_quantize_act_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  if (M <= 0 || K <= 0 || R <= 0) return 0;
  return quant_ws_bytes(M, K, R);
}

size_t svdq_packed_act_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 16 != 0) return 0;
  return svdq::packed_weight_bytes(M, K);
}

static int quantize_act_impl(const void* x, const void* smooth, const void* gscale, int64_t M, int64_t K,
                             const void* proj_down, int64_t R, int act_layout, void* qact, void* ascales,
                             void* lora_act, void* workspace, size_t workspace_bytes, void* stream);

int svdq_quantize_act(const void* x, const void* smooth, int64_t M, int64_t K,
                      const void* proj_down, int64_t R, int act_layout, void* qact,
                      void* ascales, void* lora_act, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return quantize_act_impl(x, smooth, nullptr, M, K, proj_down, R, act_layout, qact, ascales, lora_act, workspace,
                           workspace_bytes, stream);
}

int svdq_quantize_act_static(const void* x, const void* smooth, const void* act_gscale, int64_t M, int64_t K,
                             const void* proj_down, int64_t R, int act_layout, void* qact, void* ascales,
                             void* lora_act, void* workspace, size_t workspace_bytes, void* stream) {
  if (act_gscale == nullptr) return fail(SVDQ_ERR_NULL, "act_gscale is NULL");
  return quantize_act_impl(x, smooth, act_gscale, M, K, proj_down, R, act_layout, qact, ascales, lora_act,
                           workspace, workspace_bytes, stream);
}

static int quantize_act_impl(const void* x, const void* smooth, const void* gscale, int64_t M, int64_t K,
                             const void* proj_down, int64_t R, int act_layout, void* qact, void* ascales,
                             void* lora_act, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_rsrc_sizes(M, K, R))) return st;
  if (act_layout != SVDQ_ACT_CANONICAL && act_layout != SVDQ_ACT_PACKED && act_layout != SVDQ_ACT_MXFP4)
    return fail(SVDQ_ERR_INVALID, "act_layout %d is not a known layout", act_layout);
  const bool packed = act_layout == SVDQ_ACT_PACKED;
  const bool mx = act_layout == SVDQ_ACT_MXFP4;
  if (mx && K % 128 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "K = %lld: the MXFP4 layout needs K a multiple of 128", (long long)K);
  if (mx && gscale != nullptr) return fail(SVDQ_ERR_UNSUPPORTED, "the MXFP4 layout has no static-scale form");
  if (packed && ascales != nullptr)
    return fail(SVDQ_ERR_INVALID, "ascales must be NULL with the packed layout (the buffer holds them)");
  if (M == 0) return ok();
  {
    const char* names[] = {"x", "smooth", "qact"};
    const void* ptrs[] = {x, smooth, qact};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (!packed) {
    const char* names[] = {"ascales"};
    const void* ptrs[] = {ascales};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_down", "lora_act"};
    const void* ptrs[] = {proj_down, lora_act};
    if ((st = check_ptrs(names, ptrs, 2))) return st;
  }
  const size_t ws_need = quant_ws_bytes(M, K, R);
  if (ws_need > 0) {
    if (workspace_bytes < ws_need)
      return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws_need);
    const char* names[] = {"workspace"};
    const void* ptrs[] = {workspace};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if (gscale != nullptr && !aligned16(gscale)) return fail(SVDQ_ERR_ALIGN, "act_gscale is not 16-byte aligned");
  const size_t qbytes = mx ? svdq::mx_codes_bytes(M, K) : packed ? svdq::packed_weight_bytes(M, K) : (size_t)M * (K / 2);
  const size_t sbytes = mx ? (size_t)((M + 31) / 32) * 32 * (size_t)(K / 32) : (size_t)(K / 16) * M;
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("smooth", smooth, (size_t)K * 2),
                      range("proj_down", R > 0 ? proj_down : nullptr, (size_t)K * R * 2),
                      range("act_gscale", gscale, 2)};
  const Range out[] = {range("qact", qact, qbytes),
                       range("ascales", packed ? nullptr : ascales, sbytes),
                       range("lora_act", R > 0 ? lora_act : nullptr, (size_t)M * R * 2),
                       range("workspace", ws_need > 0 ? workspace : nullptr, ws_need)};
  if ((st = check_alias(in, 4, out, 4))) return st;
  if (mx) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = svdq::launch_quant_lora_mx(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth), static_cast<const uint16_t*>(proj_down),
        static_cast<uint8_t*>(qact), static_cast<uint8_t*>(ascales), static_cast<uint16_t*>(lora_act),
        static_cast<float*>(ws_need > 0 ? workspace : nullptr), M, K, R, s);
    if (int st_ = launched(e, "MX quantisation", s)) return st_;
    return ok();
  }
  return run_quantize(x, smooth, M, K, proj_down, R, qact, ascales, lora_act,
                      ws_need > 0 ? workspace : nullptr, packed, static_cast<hipStream_t>(stream), gscale);
}

size_t svdq_repack_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % 16 != 0) return 0;
  return svdq::packed_weight_bytes(N, K);
}

static int check_nk(int64_t N, int64_t K) {
  if (N < 0) return fail(SVDQ_ERR_SHAPE, "N = %lld is negative", (long long)N);
  if (K <= 0 || K % 16 != 0)
    return fail(SVDQ_ERR_SHAPE, "K = %lld must be a positive multiple of 16", (long long)K);
  if (N > kMaxDim || K > kMaxDim)
    return fail(SVDQ_ERR_UNSUPPORTED, "dimension above 2^24 (N=%lld K=%lld)", (long long)N, (long long)K);
  return SVDQ_OK;
}

int svdq_repack_weight(const void* qweight, const void* wscales, int64_t N, int64_t K,
                       void* packed, size_t packed_bytes, void* stream) {
  int st = check_nk(N, K);
  if (st) return st;
  if (N == 0) return ok();
  const char* names[] = {"qweight", "wscales", "packed"};
  const void* ptrs[] = {qweight, wscales, packed};
  if ((st = check_ptrs(names, ptrs, 3))) return st;
  const size_t need = svdq::packed_weight_bytes(N, K);
  if (packed_bytes < need)
    return fail(SVDQ_ERR_WORKSPACE, "packed buffer has %zu bytes, %zu needed", packed_bytes, need);
  const Range in[] = {range("qweight", qweight, (size_t)N * (K / 2)),
                      range("wscales", wscales, (size_t)(K / 16) * N)};
  const Range out[] = {range("packed", packed, need)};
  if ((st = check_alias(in, 2, out, 1))) return st;
  hipError_t e = svdq::launch_repack(static_cast<const uint8_t*>(qweight),
                                     static_cast<const uint8_t*>(wscales),
                                     static_cast<uint8_t*>(packed), N, K,
                                     static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "repack", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_unpack_weight(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                       void* qweight_out, void* wscales_out, void* stream) {
  int st = check_nk(N, K);
  if (st) return st;
  if (N == 0) return ok();
  const char* names[] = {"packed", "qweight_out", "wscales_out"};
  const void* ptrs[] = {packed, qweight_out, wscales_out};
  if ((st = check_ptrs(names, ptrs, 3))) return st;
  const size_t need = svdq::packed_weight_bytes(N, K);
  if (packed_bytes < need)
    return fail(SVDQ_ERR_WORKSPACE, "packed buffer has %zu bytes, %zu needed", packed_bytes, need);
  const Range in[] = {range("packed", packed, need)};
  const Range out[] = {range("qweight_out", qweight_out, (size_t)N * (K / 2)),
                       range("wscales_out", wscales_out, (size_t)(K / 16) * N)};
  if ((st = check_alias(in, 1, out, 2))) return st;
  hipError_t e = svdq::launch_unpack(static_cast<const uint8_t*>(packed),
                                     static_cast<uint8_t*>(qweight_out),
                                     static_cast<uint8_t*>(wscales_out), N, K,
                                     static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "unpack", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

static int validate_gemm(const void* qact, const void* ascales, int act_layout, const void* lora_act,
                         const void* weight, const void* wscales, int weight_layout,
                         const void* wcscales, const void* wtscale, const void* proj_up,
                         const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                         const void* y, bool check_act) {
  int st;
  if ((st = check_gemm_weight(weight_layout, wscales))) return st;
  {
    const char* names[] = {"weight", "wcscales", "wtscale", "y"};
    const void* ptrs[] = {weight, wcscales, wtscale, y};
    if ((st = check_ptrs(names, ptrs, 4))) return st;
  }
  if (check_act) {
    if (act_layout != SVDQ_ACT_CANONICAL && act_layout != SVDQ_ACT_PACKED)
      return fail(SVDQ_ERR_INVALID, "act_layout %d is not a known layout", act_layout);
    if (act_layout == SVDQ_ACT_PACKED) {
      if (ascales != nullptr)
        return fail(SVDQ_ERR_INVALID, "ascales must be NULL with packed activations");
      const char* names[] = {"qact"};
      const void* ptrs[] = {qact};
      if ((st = check_ptrs(names, ptrs, 1))) return st;
    } else {
      const char* names[] = {"qact", "ascales"};
      const void* ptrs[] = {qact, ascales};
      if ((st = check_ptrs(names, ptrs, 2))) return st;
    }
  }
  if (weight_layout == SVDQ_WEIGHT_CANONICAL && !aligned16(wscales))
    return fail(SVDQ_ERR_ALIGN, "wscales is not 16-byte aligned");
  if (R > 0) {
    if (check_act) {
      const char* names[] = {"lora_act"};
      const void* ptrs[] = {lora_act};
      if ((st = check_ptrs(names, ptrs, 1))) return st;
    }
    const char* names[] = {"proj_up"};
    const void* ptrs[] = {proj_up};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if (bias != nullptr && !aligned16(bias)) return fail(SVDQ_ERR_ALIGN, "bias is not 16-byte aligned");
  return SVDQ_OK;
}

int svdq_gemm_w4a4(const void* qact, const void* ascales, int act_layout, const void* lora_act,
                   const void* weight, const void* wscales, int weight_layout,
                   const void* wcscales, const void* wtscale, const void* proj_up,
                   const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                   void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_nk(N, K))) return st;
  if (act_layout == SVDQ_ACT_PACKED && (st = check_packed_gemm_sizes(M, N, K))) return st;
  if (M == 0 || N == 0) return ok();
  if ((st = validate_gemm(qact, ascales, act_layout, lora_act, weight, wscales, weight_layout, wcscales,
                          wtscale, proj_up, bias, M, N, K, R, y, true)))
    return st;
  const bool act_packed = act_layout == SVDQ_ACT_PACKED;
  const Range in[] = {range("qact", qact, act_packed ? svdq::packed_weight_bytes(M, K) : (size_t)M * (K / 2)),
                      range("ascales", act_packed ? nullptr : ascales, (size_t)(K / 16) * M),
                      range("lora_act", R > 0 ? lora_act : nullptr, (size_t)M * R * 2),
                      range("weight", weight, weight_bytes(weight_layout, N, K)),
                      range("wscales", wscales, (size_t)(K / 16) * N),
                      range("wcscales", wcscales, (size_t)N * 2),
                      range("wtscale", wtscale, 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("y", y, (size_t)M * N * 2)};
  if ((st = check_alias(in, 9, out, 1))) return st;
  svdq::GemmArgs a{};
  a.qact = static_cast<const uint8_t*>(qact);
  a.ascales = static_cast<const uint8_t*>(ascales);
  a.lora_act = static_cast<const uint16_t*>(lora_act);
  a.weight = static_cast<const uint8_t*>(weight);
  a.wscales = static_cast<const uint8_t*>(wscales);
  a.wcscales = static_cast<const uint16_t*>(wcscales);
  a.wtscale = static_cast<const uint16_t*>(wtscale);
  a.proj_up = static_cast<const uint16_t*>(proj_up);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.M = M; a.N = N; a.K = K; a.R = R;
  a.packed = weight_layout == SVDQ_WEIGHT_PACKED;
  // the LDS-dequantising kernel unless both operands are canonical
  a.act_canonical = act_packed ? 0 : 1;
  hipError_t e = act_packed || a.packed ? svdq::launch_gemm_lds(a, static_cast<hipStream_t>(stream))
                                        : svdq::launch_gemm_w4a4(a, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

size_t svdq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t R) {
  (void)N;
  if (M <= 0 || K <= 0 || K % 16 != 0 || R < 0) return 0;
  return linear_ws(M, K, R).total;
}

static int linear_impl(const void* x, const void* smooth, const void* gscale, const void* weight,
                       const void* wscales, int weight_layout, const void* wcscales, const void* wtscale,
                       const void* proj_down, const void* proj_up, const void* bias, int64_t M, int64_t N,
                       int64_t K, int64_t R, void* y, void* workspace, size_t workspace_bytes, void* stream);

int svdq_linear_w4a4(const void* x, const void* smooth, const void* weight, const void* wscales,
                     int weight_layout, const void* wcscales, const void* wtscale,
                     const void* proj_down, const void* proj_up, const void* bias, int64_t M,
                     int64_t N, int64_t K, int64_t R, void* y, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return linear_impl(x, smooth, nullptr, weight, wscales, weight_layout, wcscales, wtscale, proj_down, proj_up,
                     bias, M, N, K, R, y, workspace, workspace_bytes, stream);
}

int svdq_linear_w4a4_static(const void* x, const void* smooth, const void* act_gscale, const void* weight,
                            const void* wscales, int weight_layout, const void* wcscales, const void* wtscale,
                            const void* proj_down, const void* proj_up, const void* bias, int64_t M, int64_t N,
                            int64_t K, int64_t R, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (act_gscale == nullptr) return fail(SVDQ_ERR_NULL, "act_gscale is NULL");
  return linear_impl(x, smooth, act_gscale, weight, wscales, weight_layout, wcscales, wtscale, proj_down, proj_up,
                     bias, M, N, K, R, y, workspace, workspace_bytes, stream);
}

static int linear_impl(const void* x, const void* smooth, const void* gscale, const void* weight,
                       const void* wscales, int weight_layout, const void* wcscales, const void* wtscale,
                       const void* proj_down, const void* proj_up, const void* bias, int64_t M, int64_t N,
                       int64_t K, int64_t R, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_rsrc_sizes(M, K, R))) return st;
  if ((st = check_nk(N, K))) return st;
  if (weight_layout == SVDQ_WEIGHT_PACKED && (st = check_packed_gemm_sizes(M, N, K))) return st;
  if (M == 0 || N == 0) return ok();
  {
    const char* names[] = {"x", "smooth", "workspace"};
    const void* ptrs[] = {x, smooth, workspace};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_down"};
    const void* ptrs[] = {proj_down};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if ((st = validate_gemm(nullptr, nullptr, SVDQ_ACT_CANONICAL, nullptr, weight, wscales,
                          weight_layout, wcscales, wtscale, proj_up, bias, M, N, K, R, y, false)))
    return st;
  const LinearWs ws = linear_ws(M, K, R);
  if (workspace_bytes < ws.total)
    return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws.total);
  const Range in[] = {range("x", x, (size_t)M * K * 2),
                      range("smooth", smooth, (size_t)K * 2),
                      range("weight", weight, weight_bytes(weight_layout, N, K)),
                      range("wscales", wscales, (size_t)(K / 16) * N),
                      range("wcscales", wcscales, (size_t)N * 2),
                      range("wtscale", wtscale, 2),
                      range("proj_down", R > 0 ? proj_down : nullptr, (size_t)K * R * 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2), range("act_gscale", gscale, 2)};
  const Range out[] = {range("y", y, (size_t)M * N * 2), range("workspace", workspace, ws.total)};
  if ((st = check_alias(in, 10, out, 2))) return st;
  if (gscale != nullptr && !aligned16(gscale)) return fail(SVDQ_ERR_ALIGN, "act_gscale is not 16-byte aligned");

  char* w = static_cast<char*>(workspace);
  const bool packed = weight_layout == SVDQ_WEIGHT_PACKED;
  // activations always go to the packed layout; the GEMM reads either weight layout
  void* qact = w + ws.act;
  void* lora = R > 0 ? (void*)(w + ws.lora) : nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = ws.total > ws.partial ? (void*)(w + ws.partial) : nullptr;
  if ((st = run_quantize(x, smooth, M, K, proj_down, R, qact, nullptr, lora, scratch, true, s, gscale))) return st;
  svdq::GemmArgs a{};
  a.qact = static_cast<const uint8_t*>(qact);
  a.lora_act = static_cast<const uint16_t*>(lora);
  a.weight = static_cast<const uint8_t*>(weight);
  a.wscales = static_cast<const uint8_t*>(wscales);
  a.wcscales = static_cast<const uint16_t*>(wcscales);
  a.wtscale = static_cast<const uint16_t*>(wtscale);
  a.proj_up = static_cast<const uint16_t*>(proj_up);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.M = M; a.N = N; a.K = K; a.R = R;
  a.packed = packed;
  a.act_gscale = static_cast<const uint16_t*>(gscale);
  hipError_t e = svdq::launch_gemm_lds(a, s);
  if (int st_ = launched(e, "gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

// ---- gated FFN neighbour: the 2F-wide w1/w3 layer with silu(gate) * up ----

static int check_gated_f(int64_t F) {
  if (F < 0) return fail(SVDQ_ERR_SHAPE, "F = %lld is negative", (long long)F);
  if (F % 32 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "F = %lld: the gated kernels need F to be a multiple of 32", (long long)F);
  return SVDQ_OK;
}

static svdq::GemmArgs gated_args(const void* qact, const void* lora, const void* weight,
                                 const void* wcscales, const void* wtscale, const void* proj_up,
                                 const void* bias, int64_t M, int64_t F, int64_t K, int64_t R, void* h) {
  svdq::GemmArgs a{};
  a.qact = static_cast<const uint8_t*>(qact);
  a.lora_act = static_cast<const uint16_t*>(lora);
  a.weight = static_cast<const uint8_t*>(weight);
  a.wcscales = static_cast<const uint16_t*>(wcscales);
  a.wtscale = static_cast<const uint16_t*>(wtscale);
  a.proj_up = static_cast<const uint16_t*>(proj_up);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(h);
  a.M = M; a.N = 2 * F; a.K = K; a.R = R;
  a.packed = 1;
  a.gated_f = F;
  return a;
}

int svdq_gemm_w4a4_gated(const void* qact, const void* lora_act, const void* weight,
                         const void* wcscales, const void* wtscale, const void* proj_up,
                         const void* bias, int64_t M, int64_t F, int64_t K, int64_t R, void* h,
                         void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_gated_f(F))) return st;
  const int64_t N = 2 * F;
  if ((st = check_nk(N, K))) return st;
  if ((st = check_packed_gemm_sizes(M, N, K))) return st;
  if (M == 0 || F == 0) return ok();
  if ((st = validate_gemm(qact, nullptr, SVDQ_ACT_PACKED, lora_act, weight, nullptr, SVDQ_WEIGHT_PACKED,
                          wcscales, wtscale, proj_up, bias, M, N, K, R, h, true)))
    return st;
  const Range in[] = {range("qact", qact, svdq::packed_weight_bytes(M, K)),
                      range("lora_act", R > 0 ? lora_act : nullptr, (size_t)M * R * 2),
                      range("weight", weight, svdq::packed_weight_bytes(N, K)),
                      range("wcscales", wcscales, (size_t)N * 2),
                      range("wtscale", wtscale, 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("h", h, (size_t)M * F * 2)};
  if ((st = check_alias(in, 7, out, 1))) return st;
  const svdq::GemmArgs a = gated_args(qact, lora_act, weight, wcscales, wtscale, proj_up, bias, M, F, K, R, h);
  hipError_t e = svdq::launch_gemm_lds(a, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_gemm_w4a4_gated_quant(const void* qact, const void* lora_act, const void* weight,
                               const void* wcscales, const void* wtscale, const void* proj_up,
                               const void* bias, int64_t M, int64_t F, int64_t K, int64_t R, void* h,
                               const void* next_smooth, void* next_qact, size_t next_qact_bytes, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_gated_f(F))) return st;
  if (F % 64 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "F = %lld: quantising h for the next layer needs F to be a multiple of 64",
                (long long)F);
  const int64_t N = 2 * F;
  if ((st = check_nk(N, K))) return st;
  if ((st = check_packed_gemm_sizes(M, N, K))) return st;
  if ((st = check_rsrc_sizes(M, F, 0))) return st;
  if (M == 0 || F == 0) return ok();
  if ((st = validate_gemm(qact, nullptr, SVDQ_ACT_PACKED, lora_act, weight, nullptr, SVDQ_WEIGHT_PACKED,
                          wcscales, wtscale, proj_up, bias, M, N, K, R, h, true)))
    return st;
  {
    const char* names[] = {"next_smooth", "next_qact"};
    const void* ptrs[] = {next_smooth, next_qact};
    if ((st = check_ptrs(names, ptrs, 2))) return st;
  }
  const size_t q2 = svdq::packed_weight_bytes(M, F);
  if (next_qact_bytes < q2)
    return fail(SVDQ_ERR_WORKSPACE, "next_qact has %zu bytes, %zu needed", next_qact_bytes, q2);
  const Range in[] = {range("qact", qact, svdq::packed_weight_bytes(M, K)),
                      range("lora_act", R > 0 ? lora_act : nullptr, (size_t)M * R * 2),
                      range("weight", weight, svdq::packed_weight_bytes(N, K)),
                      range("wcscales", wcscales, (size_t)N * 2),
                      range("wtscale", wtscale, 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2),
                      range("next_smooth", next_smooth, (size_t)F * 2)};
  const Range out[] = {range("h", h, (size_t)M * F * 2), range("next_qact", next_qact, q2)};
  if ((st = check_alias(in, 8, out, 2))) return st;
  svdq::GemmArgs a = gated_args(qact, lora_act, weight, wcscales, wtscale, proj_up, bias, M, F, K, R, h);
  a.next_smooth = static_cast<const uint16_t*>(next_smooth);
  a.next_qact = static_cast<uint8_t*>(next_qact);
  hipError_t e = svdq::launch_gemm_lds(a, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_lowrank_down(const void* x, const void* proj_down, int64_t M, int64_t K, int64_t R, void* lora_act,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_rsrc_sizes(M, K, R))) return st;
  if (M == 0 || R == 0) return ok();
  const char* names[] = {"x", "proj_down", "lora_act"};
  const void* ptrs[] = {x, proj_down, lora_act};
  if ((st = check_ptrs(names, ptrs, 3))) return st;
  const size_t ws_need = quant_ws_bytes(M, K, R);
  if (ws_need > 0) {
    if (workspace_bytes < ws_need)
      return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws_need);
    const char* wn[] = {"workspace"};
    const void* wp[] = {workspace};
    if ((st = check_ptrs(wn, wp, 1))) return st;
  }
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("proj_down", proj_down, (size_t)K * R * 2)};
  const Range out[] = {range("lora_act", lora_act, (size_t)M * R * 2),
                       range("workspace", ws_need > 0 ? workspace : nullptr, ws_need)};
  if ((st = check_alias(in, 2, out, 2))) return st;
  hipError_t e = svdq::launch_lowrank_down(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(proj_down),
                                           static_cast<uint16_t*>(lora_act),
                                           ws_need > 0 ? static_cast<float*>(workspace) : nullptr, M, K, R,
                                           static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "down-projection", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

size_t svdq_linear_gated_workspace_bytes(int64_t M, int64_t F, int64_t K, int64_t R) {
  (void)F;
  if (M <= 0 || K <= 0 || K % 16 != 0 || R < 0) return 0;
  return linear_ws(M, K, R).total;
}

int svdq_linear_w4a4_gated(const void* x, const void* smooth, const void* weight,
                           const void* wcscales, const void* wtscale, const void* proj_down,
                           const void* proj_up, const void* bias, int64_t M, int64_t F, int64_t K,
                           int64_t R, void* h, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_rsrc_sizes(M, K, R))) return st;
  if ((st = check_gated_f(F))) return st;
  const int64_t N = 2 * F;
  if ((st = check_nk(N, K))) return st;
  if ((st = check_packed_gemm_sizes(M, N, K))) return st;
  if (M == 0 || F == 0) return ok();
  {
    const char* names[] = {"x", "smooth", "workspace"};
    const void* ptrs[] = {x, smooth, workspace};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_down"};
    const void* ptrs[] = {proj_down};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if ((st = validate_gemm(nullptr, nullptr, SVDQ_ACT_CANONICAL, nullptr, weight, nullptr,
                          SVDQ_WEIGHT_PACKED, wcscales, wtscale, proj_up, bias, M, N, K, R, h, false)))
    return st;
  const LinearWs ws = linear_ws(M, K, R);
  if (workspace_bytes < ws.total)
    return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, ws.total);
  const Range in[] = {range("x", x, (size_t)M * K * 2),
                      range("smooth", smooth, (size_t)K * 2),
                      range("weight", weight, svdq::packed_weight_bytes(N, K)),
                      range("wcscales", wcscales, (size_t)N * 2),
                      range("wtscale", wtscale, 2),
                      range("proj_down", R > 0 ? proj_down : nullptr, (size_t)K * R * 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("h", h, (size_t)M * F * 2), range("workspace", workspace, ws.total)};
  if ((st = check_alias(in, 8, out, 2))) return st;

  char* w = static_cast<char*>(workspace);
  void* qact = w + ws.act;
  void* lora = R > 0 ? (void*)(w + ws.lora) : nullptr;
  void* scratch = ws.total > ws.partial ? (void*)(w + ws.partial) : nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_quantize(x, smooth, M, K, proj_down, R, qact, nullptr, lora, scratch, true, s))) return st;
  const svdq::GemmArgs a = gated_args(qact, lora, weight, wcscales, wtscale, proj_up, bias, M, F, K, R, h);
  hipError_t e = svdq::launch_gemm_lds(a, s);
  if (int st_ = launched(e, "gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

// Which product runs a bf16 linear. SVDQ_BF16_GEMM=hip or =blaslt forces one
// (read on every call); otherwise hipBLASLt takes the large products whose
// 256 x 320 tile grid leaves a partial last round on 256 CUs (M = 4096: qkv,
// out and w2 of the 1024^2 DiT), where the hand-written kernel measured slower,
// and the hand-written kernel keeps the rest (w1/w3 fill two whole rounds).
static bool use_blaslt_bf16(int64_t M, int64_t N, int64_t K) {
  const char* v = getenv("SVDQ_BF16_GEMM");
  if (v != nullptr && strcmp(v, "hip") == 0) return false;
  if (v != nullptr && strcmp(v, "blaslt") == 0) return true;
  const int64_t tiles320 = ((M + 255) / 256) * ((N + 319) / 320);
  return (double)M * (double)N * (double)K >= 1.6e10 && tiles320 % 256 != 0;
}

int svdq_linear_bf16(const void* x, const void* weight, const void* bias, int64_t M, int64_t N,
                     int64_t K, void* y, void* stream) {
  int st = check_mk(M, K, 0);
  if (st) return st;
  if (N < 0) return fail(SVDQ_ERR_SHAPE, "N = %lld is negative", (long long)N);
  if (N > kMaxDim) return fail(SVDQ_ERR_UNSUPPORTED, "dimension above 2^24 (N=%lld)", (long long)N);
  if (M == 0 || N == 0) return ok();
  {
    const char* names[] = {"x", "weight", "y"};
    const void* ptrs[] = {x, weight, y};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (bias != nullptr && !aligned16(bias)) return fail(SVDQ_ERR_ALIGN, "bias is not 16-byte aligned");
  if (svdq::gemm_bf16_tiles(M, N) >= (int64_t(1) << 30))
    return fail(SVDQ_ERR_UNSUPPORTED, "too many output tiles (M=%lld N=%lld)", (long long)M, (long long)N);
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("weight", weight, (size_t)N * K * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("y", y, (size_t)M * N * 2)};
  if ((st = check_alias(in, 3, out, 1))) return st;
  svdq::Bf16GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(weight);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.N = N;
  a.K = K;
  hipError_t e = hipSuccess;
  bool done = false;
  if (use_blaslt_bf16(M, N, K)) e = svdq::blaslt_linear_bf16(a, static_cast<hipStream_t>(stream), &done);
  if (e == hipSuccess && !done) e = svdq::launch_gemm_bf16(a, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "bf16 gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

size_t svdq_prepare_workspace_bytes(int64_t N, int64_t K, int64_t R) {
  if (N <= 0 || K <= 0 || K % 16 != 0 || R < 0) return 0;
  return svdq::prep_workspace_bytes(N, K, R);
}

static int check_prep(int64_t N, int64_t K, int64_t R, int iters) {
  int st = check_nk(N, K);
  if (st) return st;
  if (R < 0) return fail(SVDQ_ERR_SHAPE, "R = %lld is negative", (long long)R);
  if (R % 16 != 0 || R > 128)
    return fail(SVDQ_ERR_UNSUPPORTED, "R = %lld: preparation needs R a multiple of 16, at most 128", (long long)R);
  if (N > 0 && (R > N || R > K))
    return fail(SVDQ_ERR_UNSUPPORTED, "R = %lld exceeds min(N, K) = %lld", (long long)R,
                (long long)(N < K ? N : K));
  if (iters < 0 || iters > 16) return fail(SVDQ_ERR_INVALID, "iters = %d outside 0..16", iters);
  if (N > 0 && (st = check_rsrc_sizes(N, K, 0))) return st;
  return SVDQ_OK;
}

static int prep_common(const void* weight, const void* smooth, const void* omega, const void* proj_down,
                       const void* proj_up, bool factors_out, int64_t N, int64_t K, int64_t R, void* qweight,
                       void* wscales, void* wcscales, void* wtscale, void* workspace, size_t workspace_bytes) {
  int st;
  {
    const char* names[] = {"weight", "smooth", "qweight", "wscales", "wcscales", "wtscale", "workspace"};
    const void* ptrs[] = {weight, smooth, qweight, wscales, wcscales, wtscale, workspace};
    if ((st = check_ptrs(names, ptrs, 7))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_down", "proj_up"};
    const void* ptrs[] = {proj_down, proj_up};
    if ((st = check_ptrs(names, ptrs, 2))) return st;
    if (factors_out) {
      const char* n2[] = {"omega"};
      const void* p2[] = {omega};
      if ((st = check_ptrs(n2, p2, 1))) return st;
    }
  }
  const size_t need = svdq::prep_workspace_bytes(N, K, R);
  if (workspace_bytes < need)
    return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const size_t fb_d = (size_t)K * R * 2, fb_u = (size_t)N * R * 2;
  const Range in[] = {range("weight", weight, (size_t)N * K * 2), range("smooth", smooth, (size_t)K * 2),
                      range("omega", factors_out && R > 0 ? omega : nullptr, (size_t)K * R * 4),
                      range("proj_down", !factors_out && R > 0 ? proj_down : nullptr, fb_d),
                      range("proj_up", !factors_out && R > 0 ? proj_up : nullptr, fb_u)};
  const Range out[] = {range("qweight", qweight, (size_t)N * (K / 2)),
                       range("wscales", wscales, (size_t)(K / 16) * N),
                       range("wcscales", wcscales, (size_t)N * 2), range("wtscale", wtscale, 2),
                       range("proj_down", factors_out && R > 0 ? proj_down : nullptr, fb_d),
                       range("proj_up", factors_out && R > 0 ? proj_up : nullptr, fb_u),
                       range("workspace", workspace, need)};
  if ((st = check_alias(in, 5, out, 7))) return st;
  return SVDQ_OK;
}

int svdq_prepare_weight(const void* weight, const void* smooth, const void* omega, int64_t N, int64_t K,
                        int64_t R, int iters, void* qweight, void* wscales, void* wcscales, void* wtscale,
                        void* proj_down, void* proj_up, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prep(N, K, R, iters);
  if (st) return st;
  if (N == 0) return ok();
  if ((st = prep_common(weight, smooth, omega, proj_down, proj_up, true, N, K, R, qweight, wscales, wcscales,
                        wtscale, workspace, workspace_bytes)))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e = hipSuccess;
  if (R > 0) {
    e = svdq::launch_prepare_lowrank(static_cast<const uint16_t*>(weight), static_cast<const uint16_t*>(smooth),
                                     static_cast<const float*>(omega), N, K, R, iters,
                                     static_cast<uint16_t*>(proj_down), static_cast<uint16_t*>(proj_up), ws, s);
    if (int st_ = launched(e, "rank-R split", s)) return st_;
  }
  e = svdq::launch_prepare_residual(static_cast<const uint16_t*>(weight), static_cast<const uint16_t*>(smooth),
                                      static_cast<const uint16_t*>(proj_down), static_cast<const uint16_t*>(proj_up),
                                      N, K, R, static_cast<uint8_t*>(qweight), static_cast<uint8_t*>(wscales),
                                      static_cast<uint16_t*>(wcscales), static_cast<uint16_t*>(wtscale), ws, s);
  if (int st_ = launched(e, "preparation", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_prepare_residual(const void* weight, const void* smooth, const void* proj_down, const void* proj_up,
                          int64_t N, int64_t K, int64_t R, void* qweight, void* wscales, void* wcscales,
                          void* wtscale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_prep(N, K, R, 0);
  if (st) return st;
  if (N == 0) return ok();
  if ((st = prep_common(weight, smooth, nullptr, proj_down, proj_up, false, N, K, R, qweight, wscales, wcscales,
                        wtscale, workspace, workspace_bytes)))
    return st;
  hipError_t e = svdq::launch_prepare_residual(
      static_cast<const uint16_t*>(weight), static_cast<const uint16_t*>(smooth),
      static_cast<const uint16_t*>(proj_down), static_cast<const uint16_t*>(proj_up), N, K, R,
      static_cast<uint8_t*>(qweight), static_cast<uint8_t*>(wscales), static_cast<uint16_t*>(wcscales),
      static_cast<uint16_t*>(wtscale), static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "preparation", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

size_t svdq_mx_codes_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0 || K % 128 != 0) return 0;
  return svdq::mx_codes_bytes(rows, K);
}

size_t svdq_mx_scales_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0 || K % 128 != 0) return 0;
  return (size_t)((rows + 31) / 32) * 32 * (size_t)(K / 32);
}

static int check_mx(int64_t rows, int64_t K, int64_t R) {
  int st = check_mk(rows, K, R);
  if (st) return st;
  if (K % 128 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "K = %lld: the MXFP4 variant needs K a multiple of 128", (long long)K);
  if ((int64_t)svdq::mx_codes_bytes(rows, K) >= (int64_t(1) << 31) || rows * R * 2 >= (int64_t(1) << 31))
    return fail(SVDQ_ERR_UNSUPPORTED, "MXFP4 operand or low-rank factor of %lld rows exceeds 2 GiB", (long long)rows);
  return SVDQ_OK;
}

int svdq_reround_weight_mxfp4(const void* qweight, const void* wscales, int64_t N, int64_t K, void* mx_codes,
                              void* mx_scales, void* stream) {
  int st = check_mx(N, K, 0);
  if (st) return st;
  if (N == 0) return ok();
  const char* names[] = {"qweight", "wscales", "mx_codes", "mx_scales"};
  const void* ptrs[] = {qweight, wscales, mx_codes, mx_scales};
  if ((st = check_ptrs(names, ptrs, 4))) return st;
  const Range in[] = {range("qweight", qweight, (size_t)N * (K / 2)), range("wscales", wscales, (size_t)(K / 16) * N)};
  const Range out[] = {range("mx_codes", mx_codes, svdq::mx_codes_bytes(N, K)),
                       range("mx_scales", mx_scales, svdq_mx_scales_bytes(N, K))};
  if ((st = check_alias(in, 2, out, 2))) return st;
  hipError_t e = svdq::launch_reround_mx(static_cast<const uint8_t*>(qweight), static_cast<const uint8_t*>(wscales),
                                         static_cast<uint8_t*>(mx_codes), static_cast<uint8_t*>(mx_scales), N, K,
                                         static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "re-round", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_quantize_act_mxfp4(const void* x, const void* smooth, int64_t M, int64_t K, void* mx_codes,
                            void* mx_scales, void* stream) {
  int st = check_mx(M, K, 0);
  if (st) return st;
  if (M == 0) return ok();
  const char* names[] = {"x", "smooth", "mx_codes", "mx_scales"};
  const void* ptrs[] = {x, smooth, mx_codes, mx_scales};
  if ((st = check_ptrs(names, ptrs, 4))) return st;
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("smooth", smooth, (size_t)K * 2)};
  const Range out[] = {range("mx_codes", mx_codes, svdq::mx_codes_bytes(M, K)),
                       range("mx_scales", mx_scales, svdq_mx_scales_bytes(M, K))};
  if ((st = check_alias(in, 2, out, 2))) return st;
  hipError_t e = svdq::launch_quant_act_mx(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth),
                                           static_cast<uint8_t*>(mx_codes), static_cast<uint8_t*>(mx_scales), M, K,
                                           static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "MX quantisation", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

static int validate_mx_gemm(const void* act_codes, const void* act_scales, const void* lora_act, const void* w_codes,
                            const void* w_scales, const void* wcscales, const void* wtscale, const void* proj_up,
                            const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, const void* y,
                            bool check_act) {
  int st;
  {
    const char* names[] = {"w_codes", "w_scales", "wcscales", "wtscale", "y"};
    const void* ptrs[] = {w_codes, w_scales, wcscales, wtscale, y};
    if ((st = check_ptrs(names, ptrs, 5))) return st;
  }
  if (check_act) {
    const char* names[] = {"act_codes", "act_scales"};
    const void* ptrs[] = {act_codes, act_scales};
    if ((st = check_ptrs(names, ptrs, 2))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_up"};
    const void* ptrs[] = {proj_up};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
    if (check_act) {
      const char* n2[] = {"lora_act"};
      const void* p2[] = {lora_act};
      if ((st = check_ptrs(n2, p2, 1))) return st;
    }
  }
  if (bias != nullptr && !aligned16(bias)) return fail(SVDQ_ERR_ALIGN, "bias is not 16-byte aligned");
  if (svdq::gemm_bf16_tiles(M, N) >= (int64_t(1) << 30))
    return fail(SVDQ_ERR_UNSUPPORTED, "too many output tiles (M=%lld N=%lld)", (long long)M, (long long)N);
  return SVDQ_OK;
}

static svdq::MxGemmArgs mx_args(const void* act_codes, const void* act_scales, const void* lora_act,
                                const void* w_codes, const void* w_scales, const void* wcscales, const void* wtscale,
                                const void* proj_up, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                void* y) {
  svdq::MxGemmArgs a{};
  a.act_codes = static_cast<const uint8_t*>(act_codes);
  a.act_scales = static_cast<const uint8_t*>(act_scales);
  a.lora_act = static_cast<const uint16_t*>(lora_act);
  a.w_codes = static_cast<const uint8_t*>(w_codes);
  a.w_scales = static_cast<const uint8_t*>(w_scales);
  a.wcscales = static_cast<const uint16_t*>(wcscales);
  a.wtscale = static_cast<const uint16_t*>(wtscale);
  a.proj_up = static_cast<const uint16_t*>(proj_up);
  a.bias = static_cast<const uint16_t*>(bias);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.N = N;
  a.K = K;
  a.R = R;
  return a;
}

int svdq_gemm_mxfp4(const void* act_codes, const void* act_scales, const void* lora_act, const void* w_codes,
                    const void* w_scales, const void* wcscales, const void* wtscale, const void* proj_up,
                    const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream) {
  int st = check_mx(M, K, R);
  if (st) return st;
  if ((st = check_mx(N, K, R))) return st;
  if (M == 0 || N == 0) return ok();
  if ((st = validate_mx_gemm(act_codes, act_scales, lora_act, w_codes, w_scales, wcscales, wtscale, proj_up, bias,
                             M, N, K, R, y, true)))
    return st;
  const Range in[] = {range("act_codes", act_codes, svdq::mx_codes_bytes(M, K)),
                      range("act_scales", act_scales, svdq_mx_scales_bytes(M, K)),
                      range("lora_act", R > 0 ? lora_act : nullptr, (size_t)M * R * 2),
                      range("w_codes", w_codes, svdq::mx_codes_bytes(N, K)),
                      range("w_scales", w_scales, svdq_mx_scales_bytes(N, K)),
                      range("wcscales", wcscales, (size_t)N * 2), range("wtscale", wtscale, 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("y", y, (size_t)M * N * 2)};
  if ((st = check_alias(in, 9, out, 1))) return st;
  const svdq::MxGemmArgs a = mx_args(act_codes, act_scales, lora_act, w_codes, w_scales, wcscales, wtscale, proj_up,
                                     bias, M, N, K, R, y);
  hipError_t e = svdq::launch_gemm_mx(a, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "MX gemm", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

struct MxWs {
  size_t codes, scales, lora, partial, total;
};
static MxWs mx_ws(int64_t M, int64_t K, int64_t R) {
  MxWs w{};
  w.codes = 0;
  w.scales = align256(svdq::mx_codes_bytes(M, K));
  w.lora = align256(w.scales + svdq_mx_scales_bytes(M, K));
  w.partial = align256(w.lora + (size_t)M * R * 2);
  w.total = w.partial + quant_ws_bytes(M, K, R);
  return w;
}

size_t svdq_linear_mxfp4_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  if (M <= 0 || K <= 0 || K % 128 != 0 || R < 0) return 0;
  return mx_ws(M, K, R).total;
}

int svdq_linear_mxfp4(const void* x, const void* smooth, const void* w_codes, const void* w_scales,
                      const void* wcscales, const void* wtscale, const void* proj_down, const void* proj_up,
                      const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_mx(M, K, R);
  if (st) return st;
  if ((st = check_mx(N, K, R))) return st;
  if ((st = check_rsrc_sizes(M, K, R))) return st;
  if (M == 0 || N == 0) return ok();
  {
    const char* names[] = {"x", "smooth", "workspace"};
    const void* ptrs[] = {x, smooth, workspace};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (R > 0) {
    const char* names[] = {"proj_down"};
    const void* ptrs[] = {proj_down};
    if ((st = check_ptrs(names, ptrs, 1))) return st;
  }
  if ((st = validate_mx_gemm(nullptr, nullptr, nullptr, w_codes, w_scales, wcscales, wtscale, proj_up, bias, M, N,
                             K, R, y, false)))
    return st;
  const MxWs w = mx_ws(M, K, R);
  if (workspace_bytes < w.total)
    return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("smooth", smooth, (size_t)K * 2),
                      range("w_codes", w_codes, svdq::mx_codes_bytes(N, K)),
                      range("w_scales", w_scales, svdq_mx_scales_bytes(N, K)),
                      range("wcscales", wcscales, (size_t)N * 2), range("wtscale", wtscale, 2),
                      range("proj_down", R > 0 ? proj_down : nullptr, (size_t)K * R * 2),
                      range("proj_up", R > 0 ? proj_up : nullptr, (size_t)N * R * 2),
                      range("bias", bias, (size_t)N * 2)};
  const Range out[] = {range("y", y, (size_t)M * N * 2), range("workspace", workspace, w.total)};
  if ((st = check_alias(in, 9, out, 2))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* lora = reinterpret_cast<uint16_t*>(ws + w.lora);
  // one pass over x: MX codes and scales, and lora_act when R > 0
  hipError_t e = svdq::launch_quant_lora_mx(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth),
                                            static_cast<const uint16_t*>(proj_down), ws + w.codes, ws + w.scales,
                                            lora, reinterpret_cast<float*>(ws + w.partial), M, K, R, s);
  if (int st_ = launched(e, "MX quantisation and down-projection", s)) return st_;
  const svdq::MxGemmArgs a = mx_args(ws + w.codes, ws + w.scales, lora, w_codes, w_scales, wcscales, wtscale,
                                     proj_up, bias, M, N, K, R, y);
  e = svdq::launch_gemm_mx(a, s);
  if (int st_ = launched(e, "MX gemm", s)) return st_;
  return ok();
}

size_t svdq_calibrate_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 16 != 0) return 0;
  return svdq::calibrate_workspace_bytes(M, K);
}

int svdq_calibrate_act_gscale(const void* x, const void* smooth, int64_t M, int64_t K, void* act_gscale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mk(M, K, 0);
  if (st) return st;
  if (M == 0) return fail(SVDQ_ERR_SHAPE, "calibration needs at least one row");
  if ((int64_t)M * K * 2 >= (int64_t(1) << 31))
    return fail(SVDQ_ERR_UNSUPPORTED, "calibration batch above 2 GiB (M=%lld K=%lld)", (long long)M, (long long)K);
  const char* names[] = {"x", "smooth", "act_gscale", "workspace"};
  const void* ptrs[] = {x, smooth, act_gscale, workspace};
  if ((st = check_ptrs(names, ptrs, 4))) return st;
  const size_t need = svdq::calibrate_workspace_bytes(M, K);
  if (workspace_bytes < need)
    return fail(SVDQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const Range in[] = {range("x", x, (size_t)M * K * 2), range("smooth", smooth, (size_t)K * 2)};
  const Range out[] = {range("act_gscale", act_gscale, 2), range("workspace", workspace, need)};
  if ((st = check_alias(in, 2, out, 2))) return st;
  hipError_t e = svdq::launch_calibrate(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(smooth), M, K,
                                        static_cast<uint16_t*>(act_gscale), static_cast<float*>(workspace),
                                        static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "calibration", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

}  // extern "C"

// ---- the layer without allocation: workspace in a static device array ----
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid it): svdq_linear_w4a4_noalloc runs the same
// launches as svdq_linear_w4a4 with its workspace in `scratch`, a file-scope
// device array every GPU the library runs on holds until the process ends. In
// host code `scratch` only names the symbol; its device address on the current
// device comes from hipGetSymbolAddress, taken once per device on the first
// call there and kept. Nothing in the workspace needs initialising (each call
// writes everything it later reads), so no clearing step is needed; calls
// that overlap on one GPU share the array and race.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SVDQ_ERR_UNSUPPORTED, "device ordinal %d is beyond the %d this library tracks", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(SVDQ_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SVDQ_OK;
}

}  // namespace

extern "C" {

size_t svdq_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

int svdq_linear_w4a4_noalloc(const void* x, const void* smooth, const void* weight, const void* wscales,
                             int weight_layout, const void* wcscales, const void* wtscale, const void* proj_down,
                             const void* proj_up, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                             void* y, void* stream) {
  int st = check_mk(M, K, R);
  if (st) return st;
  if ((st = check_nk(N, K))) return st;
  if (M == 0 || N == 0) return ok();
  const size_t need = linear_ws(M, K, R).total;
  if (need > kNoallocScratchBytes)
    return fail(SVDQ_ERR_WORKSPACE,
                "M=%lld K=%lld R=%lld needs %zu bytes of workspace; the static scratch holds %zu "
                "(use svdq_linear_w4a4 with a caller workspace)",
                (long long)M, (long long)K, (long long)R, need, kNoallocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws))) return st;
  return svdq_linear_w4a4(x, smooth, weight, wscales, weight_layout, wcscales, wtscale, proj_down, proj_up, bias,
                          M, N, K, R, y, ws, kNoallocScratchBytes, stream);
}

// ---- measurement helpers (not part of the layer) ----

size_t svdq_calib_table_bytes(void) { return svdq::calib_table_bytes(); }

int64_t svdq_calib_flop_per_iteration(int64_t workgroups) {
  if (workgroups <= 0) return 0;
  return workgroups * svdq::calib_waves_per_workgroup() * svdq::calib_flop_per_wave_iteration();
}

namespace {
// argument checks shared by the two sustained-rate kernels
int calib_mfma_checks(const void* table, size_t table_bytes, int64_t iters, int64_t workgroups, void* out,
                      size_t out_bytes, void* clocks, size_t clocks_bytes) {
  if (iters < 1 || workgroups < 1 || workgroups > (int64_t(1) << 20))
    return fail(SVDQ_ERR_SHAPE, "iters = %lld and workgroups = %lld must be positive (workgroups <= 2^20)",
                (long long)iters, (long long)workgroups);
  int st;
  {
    const char* names[] = {"table", "out", "clocks"};
    const void* ptrs[] = {table, out, clocks};
    if ((st = check_ptrs(names, ptrs, 3))) return st;
  }
  if (table_bytes < svdq::calib_table_bytes())
    return fail(SVDQ_ERR_WORKSPACE, "table has %zu bytes, %zu needed", table_bytes, svdq::calib_table_bytes());
  const size_t need_out = (size_t)workgroups * 64 * svdq::calib_waves_per_workgroup() * 4;
  const size_t need_clk = (size_t)workgroups * 4 * 8;
  if (out_bytes < need_out || clocks_bytes < need_clk)
    return fail(SVDQ_ERR_WORKSPACE, "out has %zu bytes (%zu needed), clocks %zu (%zu needed)", out_bytes, need_out,
                clocks_bytes, need_clk);
  const Range in[] = {range("table", table, svdq::calib_table_bytes())};
  const Range outs[] = {range("out", out, need_out), range("clocks", clocks, need_clk)};
  return check_alias(in, 1, outs, 2);
}
}  // namespace

int svdq_calib_mfma(const void* table, size_t table_bytes, int64_t iters, int64_t workgroups, void* out,
                    size_t out_bytes, void* clocks, size_t clocks_bytes, void* stream) {
  if (int st = calib_mfma_checks(table, table_bytes, iters, workgroups, out, out_bytes, clocks, clocks_bytes))
    return st;
  hipError_t e = svdq::launch_calib_mfma(table, iters, workgroups, static_cast<float*>(out),
                                         static_cast<uint64_t*>(clocks), static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "calibration", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int64_t svdq_calib_scaled_flop_per_iteration(int64_t workgroups) {
  if (workgroups <= 0) return 0;
  return workgroups * svdq::calib_waves_per_workgroup() * svdq::calib_scaled_flop_per_wave_iteration();
}

int svdq_calib_mfma_scaled(const void* table, size_t table_bytes, int64_t iters, int64_t workgroups, int fmt,
                           void* out, size_t out_bytes, void* clocks, size_t clocks_bytes, void* stream) {
  if (fmt != 0 && fmt != 4) return fail(SVDQ_ERR_UNSUPPORTED, "fmt = %d (0 = fp8 e4m3 or 4 = fp4 E2M1)", fmt);
  if (int st = calib_mfma_checks(table, table_bytes, iters, workgroups, out, out_bytes, clocks, clocks_bytes))
    return st;
  hipError_t e = svdq::launch_calib_mfma_scaled(table, iters, workgroups, fmt, static_cast<float*>(out),
                                                static_cast<uint64_t*>(clocks), static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "calibration", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int64_t svdq_calib_lds_bytes_per_iteration(int64_t workgroups) {
  if (workgroups <= 0) return 0;
  return svdq::calib_lds_bytes_per_iteration(workgroups);
}

int svdq_calib_lds(int64_t iters, int64_t workgroups, int mode, void* out, size_t out_bytes, void* stream) {
  if (mode < 0 || mode > 2) return fail(SVDQ_ERR_UNSUPPORTED, "mode = %d (0 reads, 1 writes, 2 three to one)", mode);
  if (iters < 1 || workgroups < 1 || workgroups > (int64_t(1) << 20))
    return fail(SVDQ_ERR_SHAPE, "iters = %lld and workgroups = %lld must be positive (workgroups <= 2^20)",
                (long long)iters, (long long)workgroups);
  if (out == nullptr) return fail(SVDQ_ERR_NULL, "out is NULL");
  const size_t need = (size_t)workgroups * 64 * svdq::calib_waves_per_workgroup() * 4;
  if (out_bytes < need) return fail(SVDQ_ERR_WORKSPACE, "out has %zu bytes, %zu needed", out_bytes, need);
  hipError_t e = svdq::launch_calib_lds(iters, workgroups, mode, static_cast<float*>(out),
                                        static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "calibration", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16 != 0) return fail(SVDQ_ERR_SHAPE, "bytes = %zu is not a multiple of 16", bytes);
  if (bytes == 0) return ok();
  int st;
  const char* names[] = {"src", "dst"};
  const void* ptrs[] = {src, dst};
  if ((st = check_ptrs(names, ptrs, 2))) return st;
  const Range in[] = {range("src", src, bytes)};
  const Range outs[] = {range("dst", dst, bytes)};
  if ((st = check_alias(in, 1, outs, 1))) return st;
  hipError_t e = svdq::launch_calib_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (int st_ = launched(e, "copy", static_cast<hipStream_t>(stream))) return st_;
  return ok();
}

int svdq_calib_wall_clock_khz(int* khz) {
  if (khz == nullptr) return fail(SVDQ_ERR_NULL, "khz is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "wall clock rate: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
