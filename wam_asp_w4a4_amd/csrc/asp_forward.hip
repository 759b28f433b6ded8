// The whole deflated-ASP NVFP4 layer: activation prep then the 4-bit GEMM
// with its low-rank/bias epilogue, enqueued on one stream, with the
// activation codes, scales, u and the prep's partial sums of u in the caller's
// workspace.
#include "asp_device.h"

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

int32_t asp_forward(const void* x, int32_t x_dtype, int64_t M, int64_t N, int64_t K, int32_t r,
                    const uint8_t* prep_pack, const uint8_t* w_codes, const uint8_t* w_scales,
                    const uint16_t* wv, const float* bias, void* y, int32_t y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  ASP_TRY(gemm_check(M, N, K, r, y_dtype));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (M == 0) return ASP_OK;
  const WsLayout L = ws_layout(M, K, r);
  if (!workspace) return fail(ASP_ERR_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(ASP_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(ASP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  // validate the GEMM's own pointers before enqueuing anything
  ASP_TRY(check_ptr(w_codes, "w_codes", true));
  ASP_TRY(check_ptr(w_scales, "w_scales", true));
  ASP_TRY(check_ptr(wv, "wv", r > 0));
  ASP_TRY(check_ptr(bias, "bias", false));
  ASP_TRY(check_ptr(y, "y", true));
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* xc = base + L.codes;
  uint8_t* xs = base + L.scales;
  float* u = r > 0 ? reinterpret_cast<float*>(base + L.u) : nullptr;
  ASP_TRY(act_prep_impl(3, x, x_dtype, M, K, r, prep_pack, xc, xs, u, nullptr, base + L.scratch,
                        L.total - L.scratch, (hipStream_t)stream));
  return gemm_impl(xc, xs, u, M, N, K, r, w_codes, w_scales, wv, bias, y, y_dtype,
                   (hipStream_t)stream);
}

}  // extern "C"
