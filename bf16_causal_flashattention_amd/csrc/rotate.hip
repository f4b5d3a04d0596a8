// Quantisation pre-pass with rotation and K smoothing (outside the timed attention kernel).
//
// "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4", Sec. V-E, "Rotation and
// K smoothing": Q and K are multiplied by one orthogonal R = diag(s) (C_m kron H_{D/m})
// before FP8 quantisation (H the normalised Sylvester-Hadamard matrix, C_m the
// orthonormal DCT-II, m = 1 at D = 128 and 3 at D = 192); K smoothing subtracts the mean
// key of each head over the sequence first; the per-tensor FP8 scale is taken after the
// rotation.  Element (a, b) -> (a', b') of C kron H is C[a][a'] H[b][b'] with index
// a * (D/m) + b.
//
// Row transform on one wave: lane l holds elements l + 64 a (a < D/64).  The Hadamard
// transform over the 64 positions of a segment is six butterfly stages across lanes
// (v_i + v_j at the lane whose bit is clear, v_i - v_j at the other); at D = 128 the
// seventh stage pairs the lane's two segments; at D = 192 the three segments are mixed by
// the 3x3 DCT-II after the per-segment transform.  The transform runs twice, for the
// maximum and for the codes, with the same instructions, so both see identical values and
// the rotated tensor is never stored.
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

constexpr int kRotThreads = 256;  // 4 waves, one row per wave at a time

__global__ void rot_clear_kernel(uint32_t* ws) { ws[0] = 0u; }

struct RotArgs {
  const float* x;      // [rows][D] fp32 (dense BSHD: row = (b S + s) H + h)
  const float* mean;   // [B][H][D] or null
  const float* signs;  // [D], each +1 or -1
  int64_t rows;
  int S, H;
  float c3[9];  // DCT-II of size 3, C[k][n] at c3[3 k + n] (D = 192 only)
};

template <int D>
__device__ __forceinline__ void rotate_row(const RotArgs& a, int64_t r, int lane, float y[D / 64]) {
  constexpr int NS = D / 64;
  const float* xr = a.x + r * D;
  const float* mr = nullptr;
  if (a.mean) {
    const int64_t b = r / ((int64_t)a.S * a.H);
    const int h = (int)(r % a.H);
    mr = a.mean + (b * a.H + h) * D;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float v = xr[lane + 64 * s];
    if (mr) v = v - mr[lane + 64 * s];
    y[s] = v * a.signs[lane + 64 * s];
  }
#pragma unroll
  for (int st = 1; st < 64; st <<= 1) {
    const bool hi = (lane & st) != 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float p = __shfl_xor(y[s], st);
      y[s] = hi ? p - y[s] : y[s] + p;
    }
  }
  if constexpr (D == 128) {
    const float u = y[0], w = y[1];
    y[0] = (u + w) * 0.088388347648318440550f;  // 1 / sqrt(128)
    y[1] = (u - w) * 0.088388347648318440550f;
  } else {
    float z[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) z[s] = y[s] * 0.125f;  // 1 / sqrt(64)
#pragma unroll
    for (int ap = 0; ap < 3; ++ap) y[ap] = (z[0] * a.c3[ap] + z[1] * a.c3[3 + ap]) + z[2] * a.c3[6 + ap];
  }
}

template <int D>
__global__ __launch_bounds__(kRotThreads) void rotate_amax_kernel(RotArgs a, uint32_t* ws) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kRotThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kRotThreads / 64);
  uint32_t mx = 0;
  for (int64_t r = wave; r < a.rows; r += nw) {
    float y[D / 64];
    rotate_row<D>(a, r, lane, y);
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      const uint32_t u = __float_as_uint(y[s]) & 0x7FFFFFFFu;
      mx = u > mx ? u : mx;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mx, off);
    mx = o > mx ? o : mx;
  }
  __shared__ uint32_t red[kRotThreads / 64];
  if (lane == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int i = 1; i < kRotThreads / 64; ++i) m = red[i] > m ? red[i] : m;
    atomicMax(ws, m);
  }
}

template <int D>
__global__ __launch_bounds__(kRotThreads) void rotate_quantize_kernel(RotArgs a, uint8_t* __restrict__ codes,
                                                                      float* descale, const uint32_t* ws) {
  const int k = pow2_exponent_e4m3(__uint_as_float(ws[0]));
  const float scale = __int_as_float((127 + k) << 23);
  if (blockIdx.x == 0 && threadIdx.x == 0) *descale = __int_as_float((127 - k) << 23);
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kRotThreads / 64) + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (kRotThreads / 64);
  for (int64_t r = wave; r < a.rows; r += nw) {
    float y[D / 64];
    rotate_row<D>(a, r, lane, y);
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[s] * scale, 0.f, 0, false);
      codes[r * D + lane + 64 * s] = (uint8_t)(w & 0xFF);
    }
  }
}

// Mean key per (b, h), two fixed-order stages (deterministic): partial sums over chunks
// of 256 keys, then the chunks in order, both in fp64, then one rounding to fp32.  A sum
// of fp32 values in fp64 is exact while their exponents span fewer than 29 binades, so
// the mean of identical keys is that key exactly and smoothing leaves exact zeros.
// One thread per channel d.
__global__ void key_mean_partial_kernel(const float* __restrict__ k, int S, int H, int D, int nchunk,
                                        double* __restrict__ part) {
  const int bh = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  const int b = bh / H, h = bh % H;
  const int s0 = c * 256, s1 = s0 + 256 < S ? s0 + 256 : S;
  const float* p = k + (((int64_t)b * S + s0) * H + h) * D + d;
  double acc = 0.0;
  for (int s = s0; s < s1; ++s, p += (int64_t)H * D) acc += (double)*p;
  part[((int64_t)bh * nchunk + c) * D + d] = acc;
}

__global__ void key_mean_final_kernel(const double* __restrict__ part, int S, int D, int nchunk,
                                      float* __restrict__ mean) {
  const int bh = blockIdx.x, d = threadIdx.x;
  double acc = 0.0;
  for (int c = 0; c < nchunk; ++c) acc += part[((int64_t)bh * nchunk + c) * D + d];
  mean[(int64_t)bh * D + d] = (float)(acc / (double)S);
}

int rot_grid(int64_t rows) {
  int64_t g = (rows + 4 * 16 - 1) / (4 * 16);  // about 16 rows per wave
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  return (int)g;
}

}  // namespace

int64_t key_mean_workspace_bytes(int B, int S, int H, int D) {
  const int64_t nchunk = (S + 255) / 256;
  return (int64_t)B * H * nchunk * D * (int64_t)sizeof(double);
}

hipError_t launch_key_mean(const float* k, int B, int S, int H, int D, float* mean, void* ws,
                           hipStream_t stream) {
  const int nchunk = (S + 255) / 256;
  double* part = (double*)ws;
  hipLaunchKernelGGL(key_mean_partial_kernel, dim3(B * H, nchunk), dim3(D), 0, stream, k, S, H, D, nchunk, part);
  hipLaunchKernelGGL(key_mean_final_kernel, dim3(B * H), dim3(D), 0, stream, (const double*)part, S, D, nchunk,
                     mean);
  return hipGetLastError();
}

hipError_t launch_rotate_quantize(const float* x, const float* mean, const float* signs, int B, int S, int H,
                                  int D, const float c3[9], uint8_t* codes, float* descale, uint32_t* ws,
                                  hipStream_t stream) {
  RotArgs a;
  a.x = x;
  a.mean = mean;
  a.signs = signs;
  a.rows = (int64_t)B * S * H;
  a.S = S;
  a.H = H;
  for (int i = 0; i < 9; ++i) a.c3[i] = c3[i];
  const int g = rot_grid(a.rows);
  hipLaunchKernelGGL(rot_clear_kernel, dim3(1), dim3(1), 0, stream, ws);
  if (D == 128) {
    hipLaunchKernelGGL(rotate_amax_kernel<128>, dim3(g), dim3(kRotThreads), 0, stream, a, ws);
    hipLaunchKernelGGL(rotate_quantize_kernel<128>, dim3(g), dim3(kRotThreads), 0, stream, a, codes, descale,
                       (const uint32_t*)ws);
  } else {
    hipLaunchKernelGGL(rotate_amax_kernel<192>, dim3(g), dim3(kRotThreads), 0, stream, a, ws);
    hipLaunchKernelGGL(rotate_quantize_kernel<192>, dim3(g), dim3(kRotThreads), 0, stream, a, codes, descale,
                       (const uint32_t*)ws);
  }
  return hipGetLastError();
}

}  // namespace cfa
