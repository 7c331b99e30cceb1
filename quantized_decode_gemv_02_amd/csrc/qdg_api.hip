// qdg_api.hip -- the C ABI of libqdg.so (include/qdg.h): argument checks, then
// dispatch to the gfx950 kernels.  Nothing is enqueued unless every check passes.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/qdg.h"
#include "qdg_device.h"

namespace {

thread_local int g_last_hip_error = 0;
// qdg_time_next_launch's events, taken by the thread's next launch
thread_local qdg::LaunchTiming g_timing = {nullptr, nullptr};

// qdg_set_tuning's knobs (-1: the library's own choice)
std::atomic<int> g_tune[QDG_TUNE_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
static_assert(QDG_TUNE_COUNT == 17, "one initializer a knob");

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool shape_ok(int64_t rows, int64_t K) {
  if (rows < 1 || K < qdg::QK || K % qdg::QK) return false;
  if (K > ((int64_t)1 << 31) || rows > ((int64_t)1 << 40)) return false;
  return rows <= (((int64_t)1 << 62) / K);
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QDG_OK;
  g_last_hip_error = (int)e;
  return QDG_EHIP;
}

hipStream_t as_stream(qdg_stream s) { return (hipStream_t)s; }

}  // namespace

namespace qdg {
int tune(int knob) { return g_tune[knob].load(std::memory_order_relaxed); }
LaunchTiming take_launch_timing() {
  const LaunchTiming t = g_timing;
  g_timing = LaunchTiming{nullptr, nullptr};
  return t;
}
}  // namespace qdg

extern "C" {

int qdg_set_tuning(int knob, int value) {
  if (knob < 0 || knob >= QDG_TUNE_COUNT) return QDG_EINVAL;
  g_tune[knob].store(value < 0 ? -1 : value, std::memory_order_relaxed);
  return QDG_OK;
}

int qdg_get_tuning(int knob) {
  if (knob < 0 || knob >= QDG_TUNE_COUNT) return QDG_EINVAL;
  return g_tune[knob].load(std::memory_order_relaxed);
}

int qdg_time_next_launch(void* start, void* stop) {
  g_timing = qdg::LaunchTiming{(hipEvent_t)start, (hipEvent_t)stop};
  return QDG_OK;
}

int qdg_abi_version(void) { return QDG_ABI_VERSION; }

const char* qdg_status_str(int status) {
  switch (status) {
    case QDG_OK: return "ok";
    case QDG_EINVAL: return "invalid argument (null pointer or unknown mode)";
    case QDG_ESHAPE: return "shape out of range (K must be a positive multiple of 32)";
    case QDG_EALIGN: return "misaligned pointer";
    case QDG_EMODE: return "mode does not support this batch / split combination";
    case QDG_EWORKSPACE: return "workspace too small";
    case QDG_EHIP: return "HIP launch failed (see qdg_last_hip_error)";
    default: return "unknown status";
  }
}

int qdg_last_hip_error(void) { return g_last_hip_error; }

int qdg_quantize_act(int mode, const float* x, int64_t B, int64_t K, int8_t* xq, int8_t* xl, float* xs,
                     qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!x || !xq || !xs) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!shape_ok(B, K)) return QDG_ESHAPE;
  if ((B * K / qdg::QK) * 8 / 256 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(x, 16) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4)) return QDG_EALIGN;
  return hip_status(qdg::launch_quantize(mode, x, B * K / qdg::QK, xq, xl, xs, as_stream(stream)));
}

int qdg_gemv_q8(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits, float* out,
                qdg_stream stream) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS) return QDG_EINVAL;
  if (!wq || !ws || !out) return QDG_EINVAL;
  if (mode == QDG_DEQUANT && (!x || xq || xl || xs)) return QDG_EINVAL;
  if (mode != QDG_DEQUANT && (x || !xq || !xs)) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!shape_ok(N, K)) return QDG_ESHAPE;
  if (B < 1 || B > QDG_MAX_B) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if ((N / 16 + 1) * splits >= ((int64_t)1 << 31)) return QDG_ESHAPE;  // a 1-D grid of tiles x chunks
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(out, 4)) return QDG_EALIGN;
  if (x && !aligned(x, 16)) return QDG_EALIGN;
  if (xq && !aligned(xq, 16)) return QDG_EALIGN;
  if (xl && !aligned(xl, 16)) return QDG_EALIGN;
  if (xs && !aligned(xs, 4)) return QDG_EALIGN;
  if (mode == QDG_DEQUANT && (B != 1 || splits != 1)) return QDG_EMODE;
  // more than 16 activation rows run on the LDS-direct MFMA layout: whole 8-block
  // steps (K a multiple of 256) and 16-byte weight-scale words
  if (B > 16 && ((K / qdg::QK) % 8 != 0 || !aligned(ws, 16))) return QDG_EMODE;
  const hipStream_t st = as_stream(stream);
  if (mode == QDG_DEQUANT) return hip_status(qdg::launch_gemv_dequant(wq, ws, N, K, x, out, st));
  if (B == 1) return hip_status(qdg::launch_gemv_dot4(mode, wq, ws, N, K, xq, xl, xs, splits, out, st));
  return hip_status(qdg::launch_gemv_mfma(mode, wq, ws, N, K, xq, xl, xs, B, splits, out, st));
}

int qdg_sk_combine(const float* partials, int splits, int64_t B, int64_t N, float* y, qdg_stream stream) {
  if (!partials || !y) return QDG_EINVAL;
  if (splits < 1 || splits > QDG_MAX_SPLITS || B < 1 || N < 1) return QDG_ESHAPE;
  if (B > ((int64_t)1 << 40) / N) return QDG_ESHAPE;
  if (!aligned(partials, 4) || !aligned(y, 4)) return QDG_EALIGN;
  return hip_status(qdg::launch_combine(partials, splits, B * N, y, as_stream(stream)));
}

size_t qdg_gemv_sk_workspace_bytes(int64_t B, int64_t N, int splits) {
  if (B != 1 || N < 1 || N > ((int64_t)1 << 40) || splits < 1 || splits > QDG_MAX_SPLITS) return 0;
  return qdg::sk_workspace_bytes(N, splits);
}

int qdg_gemv_q8_sk(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                   const int8_t* xl, const float* xs, int64_t B, int splits, float* y, void* workspace,
                   size_t workspace_bytes, qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return mode == QDG_DEQUANT ? QDG_EMODE : QDG_EINVAL;
  if (!wq || !ws || !xq || !xs || !y || !workspace) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!shape_ok(N, K)) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if ((N / 16 + 1) * splits >= ((int64_t)1 << 31)) return QDG_ESHAPE;  // a 1-D grid of tiles x chunks
  if (B < 1 || B > QDG_MAX_B) return QDG_ESHAPE;
  if (B != 1) return QDG_EMODE;
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4) ||
      !aligned(y, 4))
    return QDG_EALIGN;
  if (!aligned(workspace, 256)) return QDG_EALIGN;
  if (workspace_bytes < qdg::sk_workspace_bytes(N, splits)) return QDG_EWORKSPACE;
  return hip_status(qdg::launch_gemv_sk(mode, wq, ws, N, K, xq, xl, xs, splits, y, workspace, as_stream(stream)));
}

int qdg_q8_tile_rows(const int8_t* wq, int64_t N, int64_t K, int8_t* wt, qdg_stream stream) {
  if (!wq || !wt) return QDG_EINVAL;
  if (N < 4 || N % 4 || K < 256 || K % 256 || N > ((int64_t)1 << 40) / K) return QDG_ESHAPE;
  if (!aligned(wq, 16) || !aligned(wt, 16)) return QDG_EALIGN;
  const uintptr_t a = (uintptr_t)wq, b = (uintptr_t)wt, n = (uintptr_t)(N * K);
  if (a < b + n && b < a + n) return QDG_EINVAL;
  return hip_status(qdg::launch_tile_rows(wq, N, K, wt, as_stream(stream)));
}

int qdg_gemv_q8_sk_tiled(int mode, const int8_t* wt, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                         const int8_t* xl, const float* xs, int splits, float* y, qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return mode == QDG_DEQUANT ? QDG_EMODE : QDG_EINVAL;
  if (!wt || !ws || !xq || !xs || !y) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!shape_ok(N, K) || N % 4 || K % 256 || N / 4 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if (!qdg::wsplit_fits(mode, K, splits)) return QDG_EMODE;
  if (!aligned(wt, 16) || !aligned(ws, 2) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4) ||
      !aligned(y, 4))
    return QDG_EALIGN;
  return hip_status(qdg::launch_gemv_wsplit(mode, wt, ws, N, K, xq, xl, xs, splits, y, as_stream(stream), true));
}

// MFMA-tiled weights: K a multiple of 256, the record grid within a 1-D launch
static bool mma_tiled_shape(int64_t N, int64_t K) {
  if (!shape_ok(N, K) || K < 256 || K % 256 || K >= ((int64_t)1 << 30)) return false;
  return (N + 63) / 64 * (K / 256) * 4 < ((int64_t)1 << 31);
}

int64_t qdg_q8_tile_mma_bytes(int64_t N, int64_t K) {
  return mma_tiled_shape(N, K) ? qdg::tile_mma_bytes(N, K) : 0;
}

int qdg_q8_tile_mma(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, uint8_t* wt, qdg_stream stream) {
  if (!wq || !ws || !wt) return QDG_EINVAL;
  if (!mma_tiled_shape(N, K)) return QDG_ESHAPE;
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(wt, 16)) return QDG_EALIGN;
  const uintptr_t t0 = (uintptr_t)wt, t1 = t0 + (uintptr_t)qdg::tile_mma_bytes(N, K);
  const uintptr_t q0 = (uintptr_t)wq, q1 = q0 + (uintptr_t)(N * K);
  const uintptr_t s0 = (uintptr_t)ws, s1 = s0 + (uintptr_t)(N * (K / qdg::QK)) * 2;
  if ((q0 < t1 && t0 < q1) || (s0 < t1 && t0 < s1)) return QDG_EINVAL;
  return hip_status(qdg::launch_tile_mma(wq, ws, N, K, wt, as_stream(stream)));
}

int qdg_quantize_act_mma(int mode, const float* x, int64_t B, int64_t K, int8_t* xq, int8_t* xl, float* xs,
                         qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!x || !xq || !xs) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!mma_tiled_shape(1, K) || B < 1 || B > QDG_MAX_B) return QDG_ESHAPE;
  if (!aligned(x, 16) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4)) return QDG_EALIGN;
  return hip_status(qdg::launch_quantize_mma(mode, x, B, K, xq, xl, xs, as_stream(stream)));
}

int qdg_gemv_q8_mma_tiled(int mode, const uint8_t* wt, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                          const float* xs, int64_t B, int splits, float* out, qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return mode == QDG_DEQUANT ? QDG_EMODE : QDG_EINVAL;
  if (!wt || !xq || !xs || !out) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!mma_tiled_shape(N, K)) return QDG_ESHAPE;
  if (B < 1 || B > QDG_MAX_B || splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if (!aligned(wt, 16) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4) || !aligned(out, 4))
    return QDG_EALIGN;
  return hip_status(qdg::launch_gemv_mma_tiled(mode, wt, N, K, xq, xl, xs, B, splits, out, as_stream(stream)));
}

int qdg_gemv_glu_mma_tiled(int act, int mode, const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K,
                           const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, float* h, int8_t* hq,
                           int8_t* hl, float* hs, qdg_stream stream) {
  if (act < QDG_ACT_SILU || act > QDG_ACT_GELU_TANH) return QDG_EINVAL;
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!wgt || !wut || !xq || !xs || !hq || !hs) return QDG_EINVAL;
  if ((mode == QDG_TWOPASS) != (xl != nullptr) || (mode == QDG_TWOPASS) != (hl != nullptr)) return QDG_EINVAL;
  if (!mma_tiled_shape(F, K) || F % 256 != 0 || F >= ((int64_t)1 << 30)) return QDG_ESHAPE;
  if (B < 1 || B > QDG_MAX_B) return QDG_ESHAPE;
  if (!aligned(wgt, 16) || !aligned(wut, 16) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4) ||
      (h && !aligned(h, 16)) || !aligned(hq, 4) || (hl && !aligned(hl, 4)) || !aligned(hs, 4))
    return QDG_EALIGN;
  // the outputs are written while other workgroups still read the inputs
  const int64_t T = qdg::mma_act_tiles(B), wb = qdg::tile_mma_bytes(F, K);
  const uintptr_t in[5][2] = {{(uintptr_t)wgt, (uintptr_t)wgt + (uintptr_t)wb},
                              {(uintptr_t)wut, (uintptr_t)wut + (uintptr_t)wb},
                              {(uintptr_t)xq, (uintptr_t)xq + (uintptr_t)(16 * T * K)},
                              {(uintptr_t)xl, xl ? (uintptr_t)xl + (uintptr_t)(16 * T * K) : (uintptr_t)xl},
                              {(uintptr_t)xs, (uintptr_t)xs + (uintptr_t)(16 * T * (K / qdg::QK)) * 4}};
  const uintptr_t out[4][2] = {{(uintptr_t)h, h ? (uintptr_t)h + (uintptr_t)(B * F) * 4 : (uintptr_t)h},
                               {(uintptr_t)hq, (uintptr_t)hq + (uintptr_t)(16 * T * F)},
                               {(uintptr_t)hl, hl ? (uintptr_t)hl + (uintptr_t)(16 * T * F) : (uintptr_t)hl},
                               {(uintptr_t)hs, (uintptr_t)hs + (uintptr_t)(16 * T * (F / qdg::QK)) * 4}};
  for (const auto& a : in)
    for (const auto& b : out)
      if (a[0] < b[1] && b[0] < a[1]) return QDG_EINVAL;  // an empty span (NULL) meets nothing
  return hip_status(
      qdg::launch_gemv_glu_mma(act, mode, wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, as_stream(stream)));
}

int qdg_gemv_sk_combines_in_workgroup(int mode, int64_t K, int splits, int32_t* shape) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (K < qdg::QK || K % qdg::QK || splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  int rows = 0, waves = 0;
  const bool in_wg = splits > 1 && qdg::wsplit_fits(mode, K, splits);
  if (in_wg) qdg::wsplit_shape(K, splits, rows, waves);
  if (shape) {
    shape[0] = rows;
    shape[1] = waves;
  }
  return in_wg ? 1 : 0;
}

int qdg_gemv_q8_fused(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                      int splits, float* y, void* workspace, size_t workspace_bytes, qdg_stream stream) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS) return QDG_EINVAL;
  if (!wq || !ws || !x || !y) return QDG_EINVAL;
  if (!shape_ok(N, K)) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if ((N / 16 + 1) * splits >= ((int64_t)1 << 31)) return QDG_ESHAPE;  // a 1-D grid of tiles x chunks
  if (splits > 1 && !workspace) return QDG_EINVAL;
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(x, 16) || !aligned(y, 4)) return QDG_EALIGN;
  if (splits > 1 && !aligned(workspace, 256)) return QDG_EALIGN;
  if (splits > 1 && workspace_bytes < qdg::sk_workspace_bytes(N, splits)) return QDG_EWORKSPACE;
  const hipStream_t st = as_stream(stream);
  if (mode == QDG_DEQUANT) return hip_status(qdg::launch_gemv_dequant_sk(wq, ws, N, K, x, splits, y, workspace, st));
  return hip_status(qdg::launch_gemv_x(mode, wq, ws, N, K, x, splits, y, workspace, st));
}

size_t qdg_gemv_argmax_workspace_bytes(int64_t N) {
  if (N < 1 || N >= ((int64_t)1 << 31)) return 0;
  return (size_t)qdg::gemv_tiles(N) * sizeof(unsigned long long);
}

int qdg_gemv_q8_argmax(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                       const int8_t* xq, const int8_t* xl, const float* xs, float* y, int32_t* idx,
                       void* workspace, size_t workspace_bytes, qdg_stream stream) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS) return QDG_EINVAL;
  if (!wq || !ws || !y || !idx || !workspace) return QDG_EINVAL;
  if (mode == QDG_DEQUANT && (!x || xq || xl || xs)) return QDG_EINVAL;
  if (mode != QDG_DEQUANT && (x || !xq || !xs)) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && !xl) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && xl) return QDG_EINVAL;
  if (!shape_ok(N, K) || N >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(y, 4) || !aligned(idx, 4) || !aligned(workspace, 8))
    return QDG_EALIGN;
  if (x && !aligned(x, 16)) return QDG_EALIGN;
  if (xq && !aligned(xq, 16)) return QDG_EALIGN;
  if (xl && !aligned(xl, 16)) return QDG_EALIGN;
  if (xs && !aligned(xs, 4)) return QDG_EALIGN;
  if (workspace_bytes < qdg_gemv_argmax_workspace_bytes(N)) return QDG_EWORKSPACE;
  return hip_status(qdg::launch_gemv_argmax(mode, wq, ws, N, K, x, xq, xl, xs, y, idx,
                                            (unsigned long long*)workspace, as_stream(stream)));
}

}  // extern "C"

// The arg-max keys of qdg_gemv_q8_argmax_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  In host code
// its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and that
// address is what the launches receive.
namespace {
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)1 << 20;
static __device__ __align__(256) unsigned long long scratch[NOALLOC_SCRATCH_BYTES / sizeof(unsigned long long)];
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// The current device's address of `scratch` (looked up at the first call on that device).
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int qdg_gemv_q8_argmax_noalloc(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                               const int8_t* xq, const int8_t* xl, const float* xs, float* y, int32_t* idx,
                               qdg_stream stream) {
  if (N < 1 || N >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (qdg_gemv_argmax_workspace_bytes(N) > NOALLOC_SCRATCH_BYTES) return QDG_EWORKSPACE;
  void* keys = nullptr;
  const hipError_t e = device_scratch(&keys);
  if (e != hipSuccess) return hip_status(e);
  // every key the final pass reads is written by the GEMV of the same call, so
  // nothing in the scratch needs clearing
  return qdg_gemv_q8_argmax(mode, wq, ws, N, K, x, xq, xl, xs, y, idx, keys, NOALLOC_SCRATCH_BYTES, stream);
}

size_t qdg_argmax_workspace_bytes(int64_t B, int64_t N) {
  if (B < 1 || N < 1) return 0;
  return (size_t)B * (size_t)qdg::argmax_groups(N) * sizeof(unsigned long long);
}

int qdg_gemv_q8_parts(int mode, const qdg_part* parts, int nparts, int64_t K, const float* x, const int8_t* xq,
                      const int8_t* xl, const float* xs, int splits, qdg_stream stream) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS || !parts) return QDG_EINVAL;
  if (nparts < 1 || nparts > QDG_MAX_PARTS) return QDG_ESHAPE;
  if (mode == QDG_DEQUANT) {
    if (!x || xq || xl || xs) return QDG_EINVAL;
  } else {
    if (x || !xq || !xs) return QDG_EINVAL;
    if ((mode == QDG_TWOPASS) != (xl != nullptr)) return QDG_EINVAL;
  }
  const int8_t* wq[QDG_MAX_PARTS];
  const uint16_t* ws[QDG_MAX_PARTS];
  float* y[QDG_MAX_PARTS];
  int64_t N[QDG_MAX_PARTS];
  for (int p = 0; p < nparts; ++p) {
    if (!parts[p].wq || !parts[p].ws || !parts[p].y) return QDG_EINVAL;
    if (!shape_ok(parts[p].N, K)) return QDG_ESHAPE;
    if (!aligned(parts[p].wq, 16) || !aligned(parts[p].ws, 2) || !aligned(parts[p].y, 4)) return QDG_EALIGN;
    wq[p] = parts[p].wq;
    ws[p] = parts[p].ws;
    y[p] = parts[p].y;
    N[p] = parts[p].N;
  }
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if (mode == QDG_DEQUANT) {
    if (!aligned(x, 16)) return QDG_EALIGN;
    if (qdg::dq_seg_chunks(K, splits) == 0) return QDG_EMODE;
  } else {
    if (!aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4)) return QDG_EALIGN;
    if (splits < 2 || !qdg::wsplit_fits(mode, K, splits)) return QDG_EMODE;
  }
  // the grid (every part's row tiles) must fit an int: at least 4 rows a workgroup
  int64_t tiles = 0;
  for (int p = 0; p < nparts; ++p) tiles += (N[p] + 3) / 4;
  if (tiles >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (mode == QDG_DEQUANT)
    return hip_status(qdg::launch_gemv_dq_seg_parts(nparts, wq, ws, N, y, K, x, splits, as_stream(stream)));
  return hip_status(
      qdg::launch_gemv_wsplit_parts(mode, nparts, wq, ws, N, y, K, xq, xl, xs, splits, as_stream(stream)));
}

int qdg_gemv_glu_q8(int mode, const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su, int64_t F,
                    int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, float* h, int8_t* hq, int8_t* hl,
                    float* hs, qdg_stream stream) {
  return qdg_gemv_glu_act_q8(QDG_ACT_SILU, mode, wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, stream);
}

int qdg_gemv_glu_act_q8(int act, int mode, const int8_t* wg, const uint16_t* sg, const int8_t* wu,
                        const uint16_t* su, int64_t F, int64_t K, const int8_t* xq, const int8_t* xl,
                        const float* xs, float* h, int8_t* hq, int8_t* hl, float* hs, qdg_stream stream) {
  if (act < QDG_ACT_SILU || act > QDG_ACT_GELU_TANH) return QDG_EINVAL;
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!wg || !sg || !wu || !su || !xq || !xs || !hq || !hs) return QDG_EINVAL;
  if ((mode == QDG_TWOPASS) != (xl != nullptr) || (mode == QDG_TWOPASS) != (hl != nullptr)) return QDG_EINVAL;
  if (!shape_ok(F, K) || F % qdg::QK != 0 || F / qdg::QK >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(wg, 16) || !aligned(wu, 16) || !aligned(sg, 2) || !aligned(su, 2) || !aligned(xq, 16) ||
      (xl && !aligned(xl, 16)) || !aligned(xs, 4) || (h && !aligned(h, 16)) || !aligned(hq, 4) ||
      (hl && !aligned(hl, 4)) || !aligned(hs, 4))
    return QDG_EALIGN;
  if (!qdg::glu_fits(mode, K)) return QDG_EMODE;
  return hip_status(
      qdg::launch_gemv_glu(act, mode, wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, as_stream(stream)));
}

int64_t qdg_fmt_row_bytes(int fmt, int64_t K) {
  int values, bytes;
  qdg::fmt_geometry(fmt, values, bytes);
  if (!values || K < values || K % values) return 0;
  return K / values * bytes;
}

int qdg_gemv_fmt_chunk_waves(int fmt, int mode, int64_t N, int64_t K, int splits) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS) return QDG_EINVAL;
  int values, bytes;
  qdg::fmt_geometry(fmt, values, bytes);
  if (!values) return QDG_EINVAL;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_EINVAL;
  if (!shape_ok(N, K) || K % values || N / 8 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  return qdg::fmt_chunk_waves(fmt, mode, N, K, splits);
}

int qdg_gemv_dq_chunk_waves(int64_t N, int64_t K, int splits) {
  if (!shape_ok(N, K)) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  const int w = qdg::dq_chunk_waves(N, K, splits);
  return w > 0 ? w : QDG_EMODE;
}

int qdg_gemv_fmt(int fmt, int mode, const uint8_t* w, int64_t N, int64_t K, const float* x, const int8_t* xq,
                 const int8_t* xl, const float* xs, int splits, float* y, qdg_stream stream) {
  if (mode < QDG_DEQUANT || mode > QDG_TWOPASS || !w || !y) return QDG_EINVAL;
  int values, bytes;
  qdg::fmt_geometry(fmt, values, bytes);
  if (!values) return QDG_EINVAL;
  if (mode == QDG_DEQUANT && (!x || xq || xl || xs)) return QDG_EINVAL;
  if (mode != QDG_DEQUANT && (x || !xq || !xs)) return QDG_EINVAL;
  if ((mode == QDG_TWOPASS) != (xl != nullptr)) return QDG_EINVAL;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_EINVAL;
  if (!shape_ok(N, K) || K % values || N / 8 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(w, 16) || !aligned(y, 4) || (x && !aligned(x, 16)) || (xq && !aligned(xq, 16)) ||
      (xl && !aligned(xl, 16)) || (xs && !aligned(xs, 4)))
    return QDG_EALIGN;
  return hip_status(qdg::launch_gemv_fmt(fmt, mode, w, N, K, x, xq, xl, xs, splits, y, as_stream(stream)));
}

int qdg_argmax(const float* y, int64_t B, int64_t N, int32_t* idx, void* workspace, size_t workspace_bytes,
               qdg_stream stream) {
  if (!y || !idx || !workspace) return QDG_EINVAL;
  if (B < 1 || B > 65535 || N < 1 || N >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(y, 4) || !aligned(idx, 4) || !aligned(workspace, 8)) return QDG_EALIGN;
  if (workspace_bytes < qdg_argmax_workspace_bytes(B, N)) return QDG_EWORKSPACE;
  return hip_status(
      qdg::launch_argmax(y, B, N, idx, (unsigned long long*)workspace, as_stream(stream)));
}

namespace {
// The output arguments of a producer: QDG_DEQUANT writes only the f32 vector; the
// quantized modes need their words (xl exactly under QDG_TWOPASS).
int producer_outputs(int mode, const float* f, const int8_t* xq, const int8_t* xl, const float* xs) {
  if (mode == QDG_DEQUANT) return (f && !xq && !xl && !xs) ? QDG_OK : QDG_EINVAL;
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!xq || !xs) return QDG_EINVAL;
  if ((mode == QDG_TWOPASS) != (xl != nullptr)) return QDG_EINVAL;
  return QDG_OK;
}
bool words_aligned(const float* f, const int8_t* xq, const int8_t* xl, const float* xs) {
  return (!f || aligned(f, 16)) && (!xq || aligned(xq, 16)) && (!xl || aligned(xl, 16)) && (!xs || aligned(xs, 4));
}
}  // namespace

int64_t qdg_rmsnorm_max_k(void) { return qdg::rmsnorm_max_k(); }

int qdg_rmsnorm_quantize(int mode, const float* x, const float* r, float* s, const float* w, float eps, int64_t B,
                         int64_t K, float* y, int8_t* xq, int8_t* xl, float* xs, qdg_stream stream) {
  if (!x) return QDG_EINVAL;
  const int st = producer_outputs(mode, y, xq, xl, xs);
  if (st != QDG_OK) return st;
  if (s && !r) return QDG_EINVAL;
  if (!(eps >= 0.0f) || eps > 3.4e38f) return QDG_EINVAL;
  if (B < 1 || B >= ((int64_t)1 << 31) || K < qdg::QK || K % qdg::QK || K > qdg::rmsnorm_max_k()) return QDG_ESHAPE;
  if (!aligned(x, 16) || (r && !aligned(r, 16)) || (s && !aligned(s, 16)) || (w && !aligned(w, 16)) ||
      !words_aligned(y, xq, xl, xs))
    return QDG_EALIGN;
  return hip_status(qdg::launch_rmsnorm_quant(mode, x, r, s, w, eps, B, K, y, xq, xl, xs, as_stream(stream)));
}

size_t qdg_gemv_rmsnorm_workspace_bytes(int64_t N) {
  if (N < qdg::QK || N % qdg::QK || N > qdg::gemv_norm_max_n()) return 0;
  return qdg::gemv_norm_workspace_bytes(N);
}

int64_t qdg_gemv_rmsnorm_max_n(void) {
  const int64_t a = qdg::gemv_norm_max_n(), b = qdg::rmsnorm_max_k();
  return (a < b ? a : b) / qdg::QK * qdg::QK;
}

int qdg_gemv_q8_rmsnorm(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                        const int8_t* xl, const float* xs, int splits, float* y, const float* r, float* s,
                        const float* w, float eps, int qmode, float* yn, int8_t* hq, int8_t* hl, float* hs,
                        void* workspace, size_t workspace_bytes, qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return mode == QDG_DEQUANT ? QDG_EMODE : QDG_EINVAL;
  if (!wq || !ws || !xq || !xs || !workspace) return QDG_EINVAL;
  if ((mode == QDG_TWOPASS) != (xl != nullptr)) return QDG_EINVAL;
  const int st = producer_outputs(qmode, yn, hq, hl, hs);
  if (st != QDG_OK) return st;
  if (s && !r) return QDG_EINVAL;
  if (!(eps >= 0.0f) || eps > 3.4e38f) return QDG_EINVAL;
  if (!shape_ok(N, K)) return QDG_ESHAPE;
  if (N < qdg::QK || N % qdg::QK || N > qdg_gemv_rmsnorm_max_n()) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  if (!qdg::wsplit_fits(mode, K, splits)) return QDG_EMODE;
  if (!aligned(wq, 16) || !aligned(ws, 2) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(xs, 4) ||
      (y && !aligned(y, 4)) || (r && !aligned(r, 16)) || (s && !aligned(s, 16)) || (w && !aligned(w, 16)) ||
      !words_aligned(yn, hq, hl, hs))
    return QDG_EALIGN;
  if (!aligned(workspace, 256)) return QDG_EALIGN;
  if (workspace_bytes < qdg::gemv_norm_workspace_bytes(N)) return QDG_EWORKSPACE;
  return hip_status(qdg::launch_gemv_wsplit_norm(mode, wq, ws, N, K, xq, xl, xs, splits, y, r, s, w, eps, qmode, yn,
                                                 hq, hl, hs, workspace, as_stream(stream)));
}

int qdg_gemv_glu_dequant(int act, const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                         int64_t F, int64_t K, const float* x, float* h, qdg_stream stream) {
  if (act < QDG_ACT_SILU || act > QDG_ACT_GELU_TANH) return QDG_EINVAL;
  if (!wg || !sg || !wu || !su || !x || !h) return QDG_EINVAL;
  if (!shape_ok(F, K) || (F + 3) / 4 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(wg, 16) || !aligned(wu, 16) || !aligned(sg, 2) || !aligned(su, 2) || !aligned(x, 16) ||
      !aligned(h, 4))
    return QDG_EALIGN;
  // h is written while other workgroups still read the operands
  const uintptr_t h0 = (uintptr_t)h, h1 = h0 + (uintptr_t)F * 4;
  const uintptr_t spans[5][2] = {{(uintptr_t)x, (uintptr_t)x + (uintptr_t)K * 4},
                                 {(uintptr_t)wg, (uintptr_t)wg + (uintptr_t)(F * K)},
                                 {(uintptr_t)wu, (uintptr_t)wu + (uintptr_t)(F * K)},
                                 {(uintptr_t)sg, (uintptr_t)sg + (uintptr_t)(F * (K / qdg::QK)) * 2},
                                 {(uintptr_t)su, (uintptr_t)su + (uintptr_t)(F * (K / qdg::QK)) * 2}};
  for (const auto& sp : spans)
    if (sp[0] < h1 && h0 < sp[1]) return QDG_EINVAL;
  return hip_status(
      qdg::launch_gemv_dq_glu(act, wg, sg, wu, su, F, K, x, qdg::dq_unsplit_order(F), h, as_stream(stream)));
}

int qdg_swiglu_quantize(int mode, const float* g, const float* u, int64_t B, int64_t K, float* h, int8_t* xq,
                        int8_t* xl, float* xs, qdg_stream stream) {
  return qdg_glu_quantize(QDG_ACT_SILU, mode, g, u, B, K, h, xq, xl, xs, stream);
}

int qdg_glu_quantize(int act, int mode, const float* g, const float* u, int64_t B, int64_t K, float* h, int8_t* xq,
                     int8_t* xl, float* xs, qdg_stream stream) {
  if (act < QDG_ACT_SILU || act > QDG_ACT_GELU_TANH) return QDG_EINVAL;
  if (!g || !u) return QDG_EINVAL;
  const int st = producer_outputs(mode, h, xq, xl, xs);
  if (st != QDG_OK) return st;
  if (!shape_ok(B, K)) return QDG_ESHAPE;
  if ((B * K / qdg::QK) * 8 / 256 >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(g, 16) || !aligned(u, 16) || !words_aligned(h, xq, xl, xs)) return QDG_EALIGN;
  return hip_status(qdg::launch_glu_quant(act, mode, g, u, B * K / qdg::QK, h, xq, xl, xs, as_stream(stream)));
}

int qdg_block_dots(int mode, const int8_t* wq, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                   int64_t B, int32_t* dh, int32_t* dl, qdg_stream stream) {
  if (mode != QDG_INT8ACT && mode != QDG_TWOPASS) return QDG_EINVAL;
  if (!wq || !xq || !dh) return QDG_EINVAL;
  if (mode == QDG_TWOPASS && (!xl || !dl)) return QDG_EINVAL;
  if (mode == QDG_INT8ACT && (xl || dl)) return QDG_EINVAL;
  if (!shape_ok(N, K) || N > 65535 || B < 1 || B > QDG_MAX_B) return QDG_ESHAPE;
  if (!aligned(wq, 16) || !aligned(xq, 16) || (xl && !aligned(xl, 16)) || !aligned(dh, 4) ||
      (dl && !aligned(dl, 4)))
    return QDG_EALIGN;
  return hip_status(qdg::launch_block_dots(mode, wq, N, K, xq, xl, B, dh, dl, as_stream(stream)));
}

int qdg_stream_read(const void* buf, int64_t bytes, uint32_t* sink, qdg_stream stream) {
  if (!buf || !sink) return QDG_EINVAL;
  if (bytes < 16 || bytes % 16 || bytes / (64 * 1024) >= ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QDG_EALIGN;
  return hip_status(qdg::launch_stream_read(buf, bytes, sink, as_stream(stream)));
}

int qdg_split_bounds(int64_t K, int splits, int32_t* first_block) {
  if (!first_block) return QDG_EINVAL;
  if (K < qdg::QK || K % qdg::QK || K > ((int64_t)1 << 31)) return QDG_ESHAPE;
  if (splits < 1 || splits > QDG_MAX_SPLITS) return QDG_ESHAPE;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    qdg::split_range(K, splits, s, g0, g1);
    first_block[s] = g0;
  }
  first_block[splits] = (int32_t)(K / qdg::QK);
  return QDG_OK;
}

}  // extern "C"
