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

__device__ __forceinline__ uint32_t umax4(uint32_t m, float4 v) {
  const uint32_t a = __float_as_uint(v.x) & 0x7FFFFFFFu, b = __float_as_uint(v.y) & 0x7FFFFFFFu;
  const uint32_t c = __float_as_uint(v.z) & 0x7FFFFFFFu, d = __float_as_uint(v.w) & 0x7FFFFFFFu;
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d, abcd = ab > cd ? ab : cd;
  return abcd > m ? abcd : m;
}

// |x| as fp32 bits orders like the magnitude, so an unsigned atomic max finds amax.
// 16-byte loads, four in flight per thread, one atomic per block.
__global__ __launch_bounds__(kPrepThreads) void amax_kernel(const float* __restrict__ x, int64_t n,
                                                            uint32_t* ws) {
  const float4* x4 = (const float4*)x;
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t mx = 0;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 v0 = x4[i], v1 = x4[i + stride], v2 = x4[i + 2 * stride], v3 = x4[i + 3 * stride];
    mx = umax4(umax4(umax4(umax4(mx, v0), v1), v2), v3);
  }
  for (; i < n4; i += stride) mx = umax4(mx, x4[i]);
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const uint32_t u = __float_as_uint(x[n4 * 4 + threadIdx.x]) & 0x7FFFFFFFu;
    mx = u > mx ? u : mx;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mx, off);
    mx = o > mx ? o : mx;
  }
  __shared__ uint32_t red[kPrepThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int j = 1; j < kPrepThreads / 64; ++j) m = red[j] > m ? red[j] : m;
    atomicMax(ws, m);
  }
}

__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// STATIC: the scale is the argument and scaled values saturate at +-448; otherwise the
// scale comes from the maximum in ws and nothing exceeds 448.
template <bool STATIC>
__global__ __launch_bounds__(kPrepThreads) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                                uint8_t* __restrict__ codes, float* descale,
                                                                const uint32_t* ws, float static_scale) {
  float scale = static_scale;
  if constexpr (!STATIC) {
    const int k = pow2_exponent_e4m3(__uint_as_float(ws[0]));
    scale = __int_as_float((127 + k) << 23);
    if (blockIdx.x == 0 && threadIdx.x == 0) *descale = __int_as_float((127 - k) << 23);
  }
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = ((const float4*)x)[i];
    float a = v.x * scale, b = v.y * scale, c = v.z * scale, d = v.w * scale;
    if constexpr (STATIC) a = sat448(a), b = sat448(b), c = sat448(c), d = sat448(d);
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    ((int*)codes)[i] = w;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = n4 * 4 + threadIdx.x;
    float a = x[i] * scale;
    if constexpr (STATIC) a = sat448(a);
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, 0.f, 0, false);
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

int amax_grid(int64_t n) {  // 16 floats per thread per step
  int64_t g = (n + kPrepThreads * 16 - 1) / (kPrepThreads * 16);
  if (g < 1) g = 1;
  if (g > 2048) g = 2048;
  return (int)g;
}

}  // namespace

hipError_t launch_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* ws,
                                hipStream_t stream) {
  hipLaunchKernelGGL(clear_u32_kernel, dim3(1), dim3(1), 0, stream, ws);
  hipLaunchKernelGGL(amax_kernel, dim3(amax_grid(n)), dim3(kPrepThreads), 0, stream, x, n, ws);
  hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid_for(n / 4 + 1)), dim3(kPrepThreads), 0, stream, x, n, codes,
                     descale, (const uint32_t*)ws, 1.f);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3_static(const float* x, int64_t n, float scale, uint8_t* codes, hipStream_t stream) {
  hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid_for(n / 4 + 1)), dim3(kPrepThreads), 0, stream, x, n, codes,
                     (float*)nullptr, (const uint32_t*)nullptr, scale);
  return hipGetLastError();
}

hipError_t launch_round_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(round_bf16_kernel, dim3(grid_for(n)), dim3(kPrepThreads), 0, stream, x, n, out);
  return hipGetLastError();
}

}  // namespace cfa
