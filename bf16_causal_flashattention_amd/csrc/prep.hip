// Input preparation kernels (outside the timed attention kernel).
//
// "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4", Sec. V-E with
// footnote 17: FP8 inputs are e4m3 with one power-of-two descale per tensor, from
// the absolute maximum of the tensor in each call.  Reading used here: the scale is
// the largest 2^k with amax * 2^k <= 448 (nothing saturates), k clamped to
// [-126, 126], k = 0 for an all-zero tensor; values are rounded to nearest even.
// BF16 inputs are the fp32 values rounded to nearest even.
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

constexpr int kPrepThreads = 256;

__global__ void clear_u32_kernel(uint32_t* ws) { ws[0] = 0u; }

// |x| as fp32 bits orders like the magnitude, so an unsigned atomic max finds amax.
__global__ __launch_bounds__(kPrepThreads) void amax_kernel(const float* __restrict__ x, int64_t n,
                                                            uint32_t* ws) {
  uint32_t mx = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t u = __float_as_uint(x[i]) & 0x7FFFFFFFu;
    mx = u > mx ? u : mx;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mx, off);
    mx = o > mx ? o : mx;
  }
  if ((threadIdx.x & 63) == 0) atomicMax(ws, mx);
}

__global__ __launch_bounds__(kPrepThreads) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                                uint8_t* __restrict__ codes, float* descale,
                                                                const uint32_t* ws) {
  const int k = pow2_exponent_e4m3(__uint_as_float(ws[0]));
  const float scale = __int_as_float((127 + k) << 23);
  if (blockIdx.x == 0 && threadIdx.x == 0) *descale = __int_as_float((127 - k) << 23);
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = ((const float4*)x)[i];
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v.x * scale, v.y * scale, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v.z * scale, v.w * scale, w, true);
    ((int*)codes)[i] = w;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = n4 * 4 + threadIdx.x;
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[i] * scale, 0.f, 0, false);
    codes[i] = (uint8_t)(w & 0xFF);
  }
}

__global__ __launch_bounds__(kPrepThreads) void round_bf16_kernel(const float* __restrict__ x, int64_t n,
                                                                  uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = x[i];
    out[i] = (v != v) ? (uint16_t)((__float_as_uint(v) >> 16) | 0x40u) : (uint16_t)bf16_bits_rne(v);
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + kPrepThreads * 8 - 1) / (kPrepThreads * 8);
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (int)g;
}

}  // namespace

hipError_t launch_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* ws,
                                hipStream_t stream) {
  hipLaunchKernelGGL(clear_u32_kernel, dim3(1), dim3(1), 0, stream, ws);
  hipLaunchKernelGGL(amax_kernel, dim3(grid_for(n)), dim3(kPrepThreads), 0, stream, x, n, ws);
  hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(n / 4 + 1)), dim3(kPrepThreads), 0, stream, x, n, codes,
                     descale, (const uint32_t*)ws);
  return hipGetLastError();
}

hipError_t launch_round_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(round_bf16_kernel, dim3(grid_for(n)), dim3(kPrepThreads), 0, stream, x, n, out);
  return hipGetLastError();
}

}  // namespace cfa
