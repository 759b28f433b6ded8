// The whole deflated-ASP NVFP4 layer: activation prep then the 4-bit GEMM
// with its low-rank/bias epilogue, enqueued on one stream, with the
// activation codes, scales, u and the prep's partial sums of u in the caller's
// workspace.  A group of layers with the same M, K and r (for example the
// projections that read one input) runs as one launch per kernel.
#include "asp_device.h"

#include <mutex>

namespace asp {
namespace {

struct WsLayout {
  size_t codes, scales, u, scratch, total;
};

WsLayout ws_layout(int64_t M, int64_t K, int32_t r) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  WsLayout L;
  L.codes = 0;
  L.scales = up((size_t)M * K / 2);
  L.u = L.scales + up((size_t)M * K / 16);
  L.scratch = L.u + up((size_t)M * r * 4);
  L.total = L.scratch + up(act_prep_scratch_bytes(M, K, r));
  return L;
}

}  // namespace
}  // namespace asp

// The allocation-free forward's workspace: one array per GPU, held for the
// life of the process.  In host code `scratch` names a host-side stand-in, so
// its device address is taken with hipGetSymbolAddress once per device and
// only that address is used.
static __device__ __align__(256) uint8_t scratch[ASP_NOALLOC_SCRATCH_BYTES];

namespace asp {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, resolved on the first call
// for that device with the device current (the caller's current device is
// restored), then cached.
int32_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ASP_ERR_ARG, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return fail(ASP_ERR_HIP, "hipGetDevice failed");
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
      return fail(ASP_ERR_HIP, "hipSetDevice(%d) failed", dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p)
      return fail(ASP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ASP_OK;
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, size_t* bytes) {
  clear_error();
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (N < 1) return fail(ASP_ERR_SHAPE, "N=%lld must be >= 1", (long long)N);
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  *bytes = ws_layout(M, K, r).total;
  return ASP_OK;
}

int32_t asp_forward_group_stages(int32_t stages, int32_t n_layers, const void* const* x,
                                 int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                                 const uint8_t* const* prep_pack, const uint8_t* const* w_codes,
                                 const uint8_t* const* w_scales, const uint16_t* const* wv,
                                 const float* const* bias, const int64_t* N, void* const* y,
                                 int32_t y_dtype, void* const* workspace,
                                 const size_t* workspace_bytes, void* stream) {
  clear_error();
  if (stages < 1 || stages > 7) return fail(ASP_ERR_ARG, "stages=%d outside [1, 7]", stages);
  if (n_layers < 1 || n_layers > kMaxGroup)
    return fail(ASP_ERR_ARG, "n_layers=%d outside [1, %d]", n_layers, kMaxGroup);
  if (!x || !prep_pack || !w_codes || !w_scales || !N || !y || !workspace || !workspace_bytes ||
      (r > 0 && !wv))
    return fail(ASP_ERR_ARG, "a per-layer array is NULL");
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  for (int i = 0; i < n_layers; ++i) ASP_TRY(gemm_check(M, N[i], K, r, y_dtype));
  if (M == 0) return ASP_OK;
  const WsLayout L = ws_layout(M, K, r);
  PrepCall pc[kMaxGroup];
  GemmCall gc[kMaxGroup];
  for (int i = 0; i < n_layers; ++i) {
    if (!workspace[i]) return fail(ASP_ERR_ARG, "workspace of layer %d is NULL", i);
    if (((uintptr_t)workspace[i] & 255u) != 0)
      return fail(ASP_ERR_ALIGN, "workspace of layer %d must be 256-byte aligned", i);
    if (workspace_bytes[i] < L.total)
      return fail(ASP_ERR_WORKSPACE, "workspace of layer %d: %zu bytes, need %zu", i,
                  workspace_bytes[i], L.total);
    uint8_t* base = static_cast<uint8_t*>(workspace[i]);
    float* u = r > 0 ? reinterpret_cast<float*>(base + L.u) : nullptr;
    pc[i] = {x[i], prep_pack[i], base + L.codes, base + L.scales, u, nullptr, base + L.scratch,
             L.total - L.scratch};
    gc[i] = {base + L.codes, base + L.scales, u, w_codes[i], w_scales[i], r > 0 ? wv[i] : nullptr,
             bias ? bias[i] : nullptr, y[i], N[i]};
    // validate the GEMM's own pointers before enqueuing anything
    ASP_TRY(check_ptr(gc[i].w_codes, "w_codes", true));
    ASP_TRY(check_ptr(gc[i].w_scales, "w_scales", true));
    ASP_TRY(check_ptr(gc[i].wv, "wv", r > 0));
    ASP_TRY(check_ptr(gc[i].bias, "bias", false));
    ASP_TRY(check_ptr(gc[i].y, "y", true));
  }
  if (stages & 3) ASP_TRY(act_prep_impl(stages & 3, n_layers, pc, x_dtype, M, K, r, (hipStream_t)stream));
  if (stages & 4) return gemm_impl(n_layers, gc, M, K, r, y_dtype, (hipStream_t)stream);
  return ASP_OK;
}

int32_t asp_forward_group(int32_t n_layers, const void* const* x, int32_t x_dtype, int64_t M,
                          int64_t K, int32_t r, const uint8_t* const* prep_pack,
                          const uint8_t* const* w_codes, const uint8_t* const* w_scales,
                          const uint16_t* const* wv, const float* const* bias, const int64_t* N,
                          void* const* y, int32_t y_dtype, void* const* workspace,
                          const size_t* workspace_bytes, void* stream) {
  return asp_forward_group_stages(7, n_layers, x, x_dtype, M, K, r, prep_pack, w_codes, w_scales,
                                  wv, bias, N, y, y_dtype, workspace, workspace_bytes, stream);
}

int32_t asp_forward_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t N, int64_t K,
                            int32_t r, const uint8_t* prep_pack, const uint8_t* w_codes,
                            const uint8_t* w_scales, const uint16_t* wv, const float* bias,
                            void* y, int32_t y_dtype, void* stream) {
  clear_error();
  ASP_TRY(gemm_check(M, N, K, r, y_dtype));
  const size_t need = ws_layout(M, K, r).total;
  if (need > (size_t)ASP_NOALLOC_SCRATCH_BYTES)
    return fail(ASP_ERR_WORKSPACE,
                "M=%lld K=%lld r=%d needs %zu bytes of workspace, above the %zu the "
                "allocation-free forward holds; call asp_forward with a workspace",
                (long long)M, (long long)K, r, need, (size_t)ASP_NOALLOC_SCRATCH_BYTES);
  if (M == 0) return ASP_OK;
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ASP_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  void* ws = nullptr;
  ASP_TRY(scratch_on(dev, &ws));
  // the same launches as asp_forward; every byte of the workspace they read
  // is written earlier in the same call, so nothing needs clearing
  return asp_forward_group_stages(7, 1, &x, x_dtype, M, K, r, &prep_pack, &w_codes, &w_scales,
                                  &wv, &bias, &N, &y, y_dtype, &ws, &need, stream);
}

int32_t asp_forward(const void* x, int32_t x_dtype, int64_t M, int64_t N, int64_t K, int32_t r,
                    const uint8_t* prep_pack, const uint8_t* w_codes, const uint8_t* w_scales,
                    const uint16_t* wv, const float* bias, void* y, int32_t y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return asp_forward_group(1, &x, x_dtype, M, K, r, &prep_pack, &w_codes, &w_scales, &wv, &bias,
                           &N, &y, y_dtype, &workspace, &workspace_bytes, stream);
}

}  // extern "C"
