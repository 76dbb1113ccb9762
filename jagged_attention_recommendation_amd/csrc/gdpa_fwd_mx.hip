// MX-fp8 inputs (e4m3 Q/K/V with e8m0 scales per 32 elements along D, OCP Microscaling v1.0;
// page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model",
// low-precision part): the forward launches (kernel template in gdpa_fwd_kernel.h) and the exact
// dequantisation that feeds the backward. D = 128 only.
#include "gdpa_fwd_kernel.h"

namespace gdpa {

// [rows, H, 128] e4m3 codes with [rows, H, 4] e8m0 scales -> [rows, H, 128] bf16. Every value is
// an e4m3 value (at most 4 significant bits) times a power of two, which bf16 holds exactly; the
// scaled conversion instruction forms two of them per step. One thread per 16 codes (a quarter
// block: chunk c uses scale c / 2).
__global__ __launch_bounds__(256) void mx_dequant_kernel(const uint8_t* codes, const uint8_t* scales,
                                                         __bf16* out, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const i32x4 v = *(const i32x4*)(codes + c * 16);
  const float sc = fwdk::e8m0_value(scales[c >> 1]);
  bf16x2 pv[8];
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    pv[2 * wd] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[wd], sc, false);
    pv[2 * wd + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[wd], sc, true);
  }
  *(bf16x8*)(out + c * 16) = bf16x8{pv[0][0], pv[0][1], pv[1][0], pv[1][1], pv[2][0], pv[2][1], pv[3][0], pv[3][1]};
  *(bf16x8*)(out + c * 16 + 8) = bf16x8{pv[4][0], pv[4][1], pv[5][0], pv[5][1], pv[6][0], pv[6][1], pv[7][0], pv[7][1]};
}

hipError_t launch_mx_dequant(const uint8_t* codes, const uint8_t* scales, void* out, int64_t rows,
                             int H, int D, hipStream_t s) {
  if (D != 128) return hipErrorNotSupported;
  const int64_t chunks = rows * H * (D / 16);
  if (chunks <= 0) return hipSuccess;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales,
                     (__bf16*)out, chunks);
  return hipGetLastError();
}

hipError_t launch_fwd_mx(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (p.D != 128) return hipErrorNotSupported;
  return fwdk::launch_d<128, true>(p, a, grid, s);
}

}  // namespace gdpa
