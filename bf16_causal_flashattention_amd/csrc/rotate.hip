// Quantisation pre-pass with rotation and K smoothing (outside the timed attention kernel).
//
// "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4", Sec. V-E, "Rotation and
// K smoothing": Q and K are multiplied by one orthogonal R = diag(s) (C_m kron H_{D/m})
// before FP8 quantisation (H the normalised Sylvester-Hadamard matrix, C_m the
// orthonormal DCT-II, m = 1 at D = 128 and 3 at D = 192); K smoothing subtracts the mean
// key of each head over the sequence first; the per-tensor FP8 scale is taken after the
// rotation, either from the rotated tensor's maximum (two passes over x) or given as a
// static power-of-two scale (one pass, the paper's fused quantisation pass).  Element
// (a, b) -> (a', b') of C kron H is C[a][a'] H[b][b'] with index a * (D/m) + b.
//
// Row transform on one wave: lane l holds elements l + 64 a (a < D/64).  The Hadamard
// transform over the 64 positions of a segment is six butterfly stages across lanes
// (v_i + v_j at the lane whose bit is clear, v_j - v_i at the other, both as one
// fma(v_i, +-1, v_j), which rounds exactly like the add or subtract); the partner value
// comes from DPP quad permutes (bits 0, 1), ds_swizzle xor masks (bits 2, 3) and the
// gfx950 row swaps v_permlane16_swap / v_permlane32_swap (bits 4, 5); at D = 128 the
// seventh stage pairs the lane's two segments; at D = 192 the three segments are mixed by
// the 3x3 DCT-II after the per-segment transform.  Two segments of a lane go through the
// bit-4 and bit-5 stages together: a row swap of segment A against segment B leaves each
// lane with both members of one butterfly pair, and a second swap after the add and
// subtract restores the layout.
//
// Work: a wave stays on one head (b, h) and takes kRotRows sequence positions of it at a
// time, so their loads are in flight together and the head's mean key, times the signs,
// stays in registers; (x - m) s is then one exact fma(x, s, -m s).  In the two-pass form
// both passes run the same instructions, so both see identical values and the rotated
// tensor is never stored.
#include <atomic>

#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

constexpr int kRotThreads = 256;  // 4 waves
constexpr int kRotRows = 4;       // consecutive rows per wave per step
constexpr int kMeanSub = 4;       // threads per channel in the key-mean partial sums
constexpr int kMeanChunk = 1024;  // keys per partial sum

__global__ void rot_clear_kernel(uint32_t* ws) { ws[0] = 0u; }

struct RotArgs {
  const float* x;      // [B][S][H][D] fp32, dense
  const float* mean;   // [B][H][D] (used only when the kernel is built with MEAN)
  const float* signs;  // [D], each +1 or -1
  uint32_t S, H, BH;   // B S H D < 2^31
  uint32_t n_items;    // BH * ceil(S / kRotRows); item i = (head i % BH, positions kRotRows (i / BH) ...)
  float c3[9];         // DCT-II of size 3, C[k][n] at c3[3 k + n] (D = 192 only)
};

// The wave's current head: row pointer step and the signed mean -m s (zero without MEAN).
template <int D>
struct HeadState {
  uint32_t bh = 0xFFFFFFFFu;
  float nms[D / 64];
};

template <int D, bool MEAN>
__device__ __forceinline__ void set_head(const RotArgs& a, uint32_t bh, int lane, const float (&sg)[D / 64],
                                         HeadState<D>& hs) {
  if (hs.bh == bh) return;  // wave-uniform
  hs.bh = bh;
#pragma unroll
  for (int s = 0; s < D / 64; ++s) hs.nms[s] = MEAN ? -(a.mean[(size_t)bh * D + lane + 64 * s] * sg[s]) : 0.f;
}

// rows of item i: positions p0 .. p0 + kRotRows - 1 (those below S) of head bh
template <int D, bool MEAN>
__device__ __forceinline__ void load_item(const RotArgs& a, uint32_t bh, uint32_t p0, int lane,
                                          const float (&sg)[D / 64], const HeadState<D>& hs,
                                          float (&y)[kRotRows][D / 64]) {
  constexpr int NS = D / 64;
  const uint32_t b = bh / a.H, h = bh % a.H;
  const float* x0 = a.x + (((size_t)b * a.S + p0) * a.H + h) * D + lane;
  const size_t step = (size_t)a.H * D;
#pragma unroll
  for (int j = 0; j < kRotRows; ++j) {
    if (p0 + j < a.S) {  // wave-uniform
#pragma unroll
      for (int s = 0; s < NS; ++s) y[j][s] = x0[j * step + 64 * s];
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) y[j][s] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < kRotRows; ++j)
#pragma unroll
    for (int s = 0; s < NS; ++s) y[j][s] = MEAN ? fmaf(y[j][s], sg[s], hs.nms[s]) : y[j][s] * sg[s];
}

// Per-lane butterfly signs: +1 where bit b of the lane is clear, -1 where it is set.
struct Bfly {
  float sg[6];
  __device__ explicit Bfly(int lane) {
#pragma unroll
    for (int b = 0; b < 6; ++b) sg[b] = (lane >> b) & 1 ? -1.f : 1.f;
  }
};

__device__ __forceinline__ float dpp_quad(float v, int ctrl_is_xor2) {
  const int u = __float_as_int(v);
  return __int_as_float(ctrl_is_xor2 ? __builtin_amdgcn_mov_dpp(u, 0x4E, 0xF, 0xF, false)    // quad_perm 2,3,0,1
                                     : __builtin_amdgcn_mov_dpp(u, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
}

__device__ __forceinline__ void row_swap(float& a, float& b, bool by32) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const auto r = by32 ? __builtin_amdgcn_permlane32_swap(ua, ub, false, false)
                      : __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// One segment alone, partner at lane ^ 16 or lane ^ 32: after swapping a copy with itself,
// r[0] is the lane's own value where the bit is clear and the partner's where it is set.
__device__ __forceinline__ float swap_stage(float v, float sg, bool by32) {
  float a = v, b = v;
  row_swap(a, b, by32);
  return fmaf(b, sg, a);
}

// Two segments A, B together: the row swap gives every lane (own, partner) of one pair
// (of A where the bit is clear, of B where it is set), so A' + B' and A' - B' are that
// pair's butterfly outputs; swapping them back puts A and B in their places again.
__device__ __forceinline__ void pair_stage(float& a, float& b, bool by32) {
  row_swap(a, b, by32);
  const float s = a + b, d = a - b;
  a = s;
  b = d;
  row_swap(a, b, by32);
}

__device__ __forceinline__ float lane_stages(float v, const Bfly& bf) {
  v = fmaf(v, bf.sg[0], dpp_quad(v, 0));
  v = fmaf(v, bf.sg[1], dpp_quad(v, 1));
  v = fmaf(v, bf.sg[2], __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F)));  // xor 4
  v = fmaf(v, bf.sg[3], __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F)));  // xor 8
  return v;
}

template <int D>
__device__ __forceinline__ void transform(float (&y)[D / 64], const Bfly& bf, const float* c3) {
  constexpr int NS = D / 64;
#pragma unroll
  for (int s = 0; s < NS; ++s) y[s] = lane_stages(y[s], bf);
  pair_stage(y[0], y[1], false);
  pair_stage(y[0], y[1], true);
  if constexpr (NS == 3) {
    y[2] = swap_stage(y[2], bf.sg[4], false);
    y[2] = swap_stage(y[2], bf.sg[5], true);
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
    for (int ap = 0; ap < 3; ++ap) y[ap] = (z[0] * c3[ap] + z[1] * c3[3 + ap]) + z[2] * c3[6 + ap];
  }
}

template <int D>
__device__ __forceinline__ void load_signs(const RotArgs& a, int lane, float (&sg)[D / 64]) {
#pragma unroll
  for (int s = 0; s < D / 64; ++s) sg[s] = a.signs[lane + 64 * s];
}

template <int D, bool MEAN>
__global__ __launch_bounds__(kRotThreads) void rotate_amax_kernel(RotArgs a, uint32_t* ws) {
  constexpr int NS = D / 64;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kRotThreads / 64) + (threadIdx.x >> 6);
  const uint32_t nw = gridDim.x * (kRotThreads / 64);
  float sg[NS];
  load_signs<D>(a, lane, sg);
  const Bfly bf(lane);
  HeadState<D> hs;
  uint32_t mx = 0;
  for (uint32_t it = wave; it < a.n_items; it += nw) {
    const uint32_t bh = it % a.BH, p0 = (it / a.BH) * kRotRows;
    set_head<D, MEAN>(a, bh, lane, sg, hs);
    float y[kRotRows][NS];
    load_item<D, MEAN>(a, bh, p0, lane, sg, hs, y);
#pragma unroll
    for (int j = 0; j < kRotRows; ++j) {
      if (p0 + j >= a.S) break;  // wave-uniform; rows past the end hold -m s, not data
      transform<D>(y[j], bf, a.c3);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t u = __float_as_uint(y[j][s]) & 0x7FFFFFFFu;
        mx = u > mx ? u : mx;
      }
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

// STATIC: the scale is the argument and scaled values are clamped to +-448 (saturation);
// otherwise the scale comes from the maximum in ws and nothing exceeds 448.
template <int D, bool MEAN, bool STATIC>
__global__ __launch_bounds__(kRotThreads) void rotate_quantize_kernel(RotArgs a, uint8_t* __restrict__ codes,
                                                                      float* descale, const uint32_t* ws,
                                                                      float static_scale) {
  constexpr int NS = D / 64;
  float scale = static_scale;
  if constexpr (!STATIC) {
    const int k = pow2_exponent_e4m3(__uint_as_float(ws[0]));
    scale = __int_as_float((127 + k) << 23);
    if (blockIdx.x == 0 && threadIdx.x == 0) *descale = __int_as_float((127 - k) << 23);
  }
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kRotThreads / 64) + (threadIdx.x >> 6);
  const uint32_t nw = gridDim.x * (kRotThreads / 64);
  float sg[NS];
  load_signs<D>(a, lane, sg);
  const Bfly bf(lane);
  HeadState<D> hs;
  for (uint32_t it = wave; it < a.n_items; it += nw) {
    const uint32_t bh = it % a.BH, p0 = (it / a.BH) * kRotRows;
    set_head<D, MEAN>(a, bh, lane, sg, hs);
    float y[kRotRows][NS];
    load_item<D, MEAN>(a, bh, p0, lane, sg, hs, y);
    uint8_t* c0 = codes + (((size_t)(bh / a.H) * a.S + p0) * a.H + bh % a.H) * D + lane;
#pragma unroll
    for (int j = 0; j < kRotRows; ++j) {
      if (p0 + j >= a.S) break;  // wave-uniform
      transform<D>(y[j], bf, a.c3);
      uint8_t* cr = c0 + (size_t)j * a.H * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v = y[j][s] * scale;
        if constexpr (STATIC) v = fminf(fmaxf(v, -448.f), 448.f);
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false);
        cr[64 * s] = (uint8_t)(w & 0xFF);
      }
    }
  }
}

// Mean key per (b, h) in two fixed-order stages, in fp64 (deterministic): within a chunk
// of kMeanChunk keys, thread (sub, d) sums keys s0 + sub, s0 + sub + kMeanSub, ... and the
// kMeanSub sums are added in sub order; then the chunks are added in sequence and the
// total is divided by S and rounded once to fp32.  A sum of fp32 values in fp64 is exact
// while their exponents span fewer than 29 binades, so identical keys give their own
// value back and smoothing leaves exact zeros.
template <int D>
__global__ __launch_bounds__(kMeanSub * D) void key_mean_partial_kernel(const float* __restrict__ k, int S, int H,
                                                                        int nchunk, double* __restrict__ part) {
  const int bh = blockIdx.x, c = blockIdx.y;
  const int sub = threadIdx.x / D, d = threadIdx.x % D;
  const int b = bh / H, h = bh % H;
  const int s0 = c * kMeanChunk, s1 = s0 + kMeanChunk < S ? s0 + kMeanChunk : S;
  const size_t step = (size_t)kMeanSub * H * D;
  const float* p = k + (((size_t)b * S + s0 + sub) * H + h) * D + d;
  double acc = 0.0;
#pragma unroll 8
  for (int s = s0 + sub; s < s1; s += kMeanSub, p += step) acc += (double)*p;
  __shared__ double red[kMeanSub][D];
  red[sub][d] = acc;
  __syncthreads();
  if (sub == 0) {
    double t = red[0][d];
#pragma unroll
    for (int i = 1; i < kMeanSub; ++i) t += red[i][d];
    part[((size_t)bh * nchunk + c) * D + d] = t;
  }
}

__global__ void key_mean_final_kernel(const double* __restrict__ part, int S, int D, int nchunk,
                                      float* __restrict__ mean) {
  const int bh = blockIdx.x, d = threadIdx.x;
  double acc = 0.0;
  for (int c = 0; c < nchunk; ++c) acc += part[((size_t)bh * nchunk + c) * D + d];
  mean[(size_t)bh * D + d] = (float)(acc / (double)S);
}

// Waves in the grid: at most 8192 (8 per SIMD on 256 CUs), and where the heads allow, a
// multiple of B H that is also a multiple of 4 (4 waves per block), so that every wave
// keeps one head for all its items.
int rot_grid(uint32_t n_items, uint32_t BH) {
  int64_t waves = 8192;
  const int64_t per_head = BH == 0 ? 0 : 8192 / BH / 4 * 4;
  if (per_head >= 4) waves = per_head * BH;
  if (waves > n_items) waves = ((int64_t)n_items + 3) / 4 * 4;
  if (waves < 4) waves = 4;
  return (int)(waves / 4);
}

RotArgs make_rot_args(const float* x, const float* mean, const float* signs, int B, int S, int H,
                      const float c3[9]) {
  RotArgs a;
  a.x = x;
  a.mean = mean;
  a.signs = signs;
  a.S = (uint32_t)S;
  a.H = (uint32_t)H;
  a.BH = (uint32_t)B * (uint32_t)H;
  a.n_items = a.BH * (uint32_t)((S + kRotRows - 1) / kRotRows);
  for (int i = 0; i < 9; ++i) a.c3[i] = c3[i];
  return a;
}

template <int D, bool MEAN>
void launch_rq(const RotArgs& a, uint8_t* codes, float* descale, uint32_t* ws, float static_scale, bool is_static,
               hipStream_t stream) {
  const int g = rot_grid(a.n_items, a.BH);
  if (is_static) {
    hipLaunchKernelGGL((rotate_quantize_kernel<D, MEAN, true>), dim3(g), dim3(kRotThreads), 0, stream, a, codes,
                       descale, (const uint32_t*)ws, static_scale);
  } else {
    hipLaunchKernelGGL(rot_clear_kernel, dim3(1), dim3(1), 0, stream, ws);
    hipLaunchKernelGGL((rotate_amax_kernel<D, MEAN>), dim3(g), dim3(kRotThreads), 0, stream, a, ws);
    hipLaunchKernelGGL((rotate_quantize_kernel<D, MEAN, false>), dim3(g), dim3(kRotThreads), 0, stream, a, codes,
                       descale, (const uint32_t*)ws, 1.f);
  }
}

}  // namespace

int64_t key_mean_workspace_bytes(int B, int S, int H, int D) {
  const int64_t nchunk = ((int64_t)S + kMeanChunk - 1) / kMeanChunk;
  return (int64_t)B * H * nchunk * D * (int64_t)sizeof(double);
}

hipError_t launch_key_mean(const float* k, int B, int S, int H, int D, float* mean, void* ws,
                           hipStream_t stream) {
  const int nchunk = (S + kMeanChunk - 1) / kMeanChunk;
  double* part = (double*)ws;
  if (D == 128)
    hipLaunchKernelGGL(key_mean_partial_kernel<128>, dim3(B * H, nchunk), dim3(kMeanSub * 128), 0, stream, k, S,
                       H, nchunk, part);
  else
    hipLaunchKernelGGL(key_mean_partial_kernel<192>, dim3(B * H, nchunk), dim3(kMeanSub * 192), 0, stream, k, S,
                       H, nchunk, part);
  hipLaunchKernelGGL(key_mean_final_kernel, dim3(B * H), dim3(D), 0, stream, (const double*)part, S, D, nchunk,
                     mean);
  return hipGetLastError();
}

// Allocation-free key mean: the fp64 partial sums live in this file-scope device array
// instead of a caller workspace.  Every GPU that runs it holds its own copy until the process
// ends, at its own address; host code reaches it only through the address that
// hipGetSymbolAddress returns on that device (the array's name is not a device address in
// host code).  Every call on one GPU reuses that GPU's copy: the partial kernel overwrites
// each partial sum it later reads, so nothing needs clearing, and calls that overlap on one
// GPU race.
static __device__ __align__(256) double scratch[kKeyMeanScratchBytes / sizeof(double)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];  // per device; null until looked up
}  // namespace

hipError_t launch_key_mean_noalloc(const float* k, int B, int S, int H, int D, float* mean, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {  // first call on this device, which is current: look its copy up once
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return launch_key_mean(k, B, S, H, D, mean, p, stream);
}

hipError_t launch_rotate_quantize(const float* x, const float* mean, const float* signs, int B, int S, int H,
                                  int D, const float c3[9], uint8_t* codes, float* descale, uint32_t* ws,
                                  float static_scale, bool is_static, hipStream_t stream) {
  const RotArgs a = make_rot_args(x, mean, signs, B, S, H, c3);
  if (D == 128) {
    if (mean)
      launch_rq<128, true>(a, codes, descale, ws, static_scale, is_static, stream);
    else
      launch_rq<128, false>(a, codes, descale, ws, static_scale, is_static, stream);
  } else {
    if (mean)
      launch_rq<192, true>(a, codes, descale, ws, static_scale, is_static, stream);
    else
      launch_rq<192, false>(a, codes, descale, ws, static_scale, is_static, stream);
  }
  return hipGetLastError();
}

}  // namespace cfa
