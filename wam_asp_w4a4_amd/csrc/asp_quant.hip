// Standalone NVFP4 quantiser and dequantiser kernels (gfx950) and their C
// entry points.  Format: model card "FastWAM UR3 3-task -- 4-bit
// quantisations", method table (E2M1 elements, block 16, E4M3 block scales).
#include "asp_device.h"

namespace asp {
namespace {

// One lane per 16-element block.
__global__ void __launch_bounds__(256) k_quantize(const float* __restrict__ in, int64_t n_blk,
                                                  uint2* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_blk) return;
  const float4* p = reinterpret_cast<const float4*>(in) + 4 * i;
  float v[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = p[k];
    v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
  }
  uint32_t sc;
  codes[i] = quantize_block(v, sc);
  scales[i] = (uint8_t)sc;
}

__global__ void __launch_bounds__(256) k_dequantize(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    int64_t n_half, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_half) return;
  const uint32_t w = codes[i];
  const float sd = e4m3_decode(scales[i >> 1]);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = e2m1_decode((w >> (4 * e)) & 15u) * sd;
  reinterpret_cast<float4*>(out)[2 * i] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(out)[2 * i + 1] = make_float4(v[4], v[5], v[6], v[7]);
}

int32_t check_rows_cols(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || cols % 16)
    return fail(ASP_ERR_SHAPE, "rows=%lld cols=%lld: need rows >= 0, cols a positive multiple of 16",
                (long long)rows, (long long)cols);
  if ((rows * cols / 8 + 255) / 256 > INT32_MAX)
    return fail(ASP_ERR_SHAPE, "input too large for one launch");
  return ASP_OK;
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_quantize_nvfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  clear_error();
  ASP_TRY(check_rows_cols(rows, cols));
  if (rows == 0) return ASP_OK;
  ASP_TRY(check_ptr(in, "in", true));
  ASP_TRY(check_ptr(codes, "codes", true));
  ASP_TRY(check_ptr(scales, "scales", true));
  const int64_t n_blk = rows * cols / 16;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)((n_blk + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, in, n_blk, reinterpret_cast<uint2*>(codes), scales);
  return launch_status("quantize");
}

int32_t asp_dequantize_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, float* out, void* stream) {
  clear_error();
  ASP_TRY(check_rows_cols(rows, cols));
  if (rows == 0) return ASP_OK;
  ASP_TRY(check_ptr(codes, "codes", true));
  ASP_TRY(check_ptr(scales, "scales", true));
  ASP_TRY(check_ptr(out, "out", true));
  const int64_t n_half = rows * cols / 8;
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)((n_half + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, reinterpret_cast<const uint32_t*>(codes), scales,
                     n_half, out);
  return launch_status("dequantize");
}

}  // extern "C"
