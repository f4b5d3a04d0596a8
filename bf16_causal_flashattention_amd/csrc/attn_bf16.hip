// Causal attention forward with BF16 operands on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Follows "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4":
//   Sec. II-B  base-2 online softmax over 128-key blocks, LSE output;
//   Sec. IV-A  8 waves x 32 query rows, S^T = K Q^T so each lane holds one query's
//              scores, causal pairing, persistent grid, chiplet map;
//   Sec. IV-A  lazy rescaling with tau = 0.5 (the BF16 value at d = 128);
//   Sec. VI-A  the softmax scale is applied to the fp32 scores (not folded into bf16 Q).
// fp32 arithmetic: t = s * cp with cp = fp32(c log2 e); p = exp2(fmaf(s, cp, -m));
// l sums the fp32 p; O = bf16_rne(acc / l); LSE = ln 2 * (m + log2 l).
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

constexpr float kTauBf16 = 0.5f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kKBytes = 128 * 256;          // K block [128 keys][128 d] bf16
constexpr int kStage = kKBytes + 128 * 256;  // + V^T block [128 d][128 keys] bf16
constexpr int kLds = 2 * kStage;

__device__ __forceinline__ v8bf as_bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(Bf16Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H;
  const Schedule sch = make_schedule(a.B, H, S);
  const int logical = xcd_logical(blockIdx.x, gridDim.x);

  const int v_dc = tid & 15, v_kg = tid >> 4;
  const int64_t rs = (int64_t)H * 256;  // row stride in bytes (d = 128 bf16)
  const float cp = a.cp;

  for (int64_t item = logical; item < sch.items; item += gridDim.x) {
    int b, h, j;
    decode_item(item, H, sch.P, b, h, j);
    const uint8_t* kbh = (const uint8_t*)a.k + ((int64_t)b * S * H + h) * 256;
    const uint8_t* vbh = (const uint8_t*)a.v + ((int64_t)b * S * H + h) * 256;
    const uint8_t* qbh = (const uint8_t*)a.q + ((int64_t)b * S * H + h) * 256;

    for (int pass = 0; pass < 2; ++pass) {
      const int tile = pass == 0 ? j : sch.T - 1 - j;
      if (pass == 1 && tile == j) break;
      const int row0 = tile * kTileRows + wave * kWaveRows;
      const int qrow = row0 + l32;
      const int nb = 2 * tile + 2;

      // Q^T operand: lane holds Q[qrow][16m + 8hh .. +8] for m = 0..7
      v8bf qop[8];
      {
        const uint8_t* qp = qbh + (int64_t)qrow * rs + 16 * hh;
#pragma unroll
        for (int m = 0; m < 8; ++m) qop[m] = as_bf(*(const v4i*)(qp + 32 * m));
      }

      v16f oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
      float m = 0.f, l = 0.f;

      v4i kreg[4], vreg[4];
      auto load_kv = [&](int key0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int id = tid + kThreads * p;
          kreg[p] = *(const v4i*)(kbh + (int64_t)(key0 + (id >> 4)) * rs + 16 * (id & 15));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) vreg[i] = *(const v4i*)(vbh + (int64_t)(key0 + 4 * v_kg + i) * rs + 16 * v_dc);
      };
      auto store_kv = [&](int stage) {
        uint8_t* sb = smem + stage * kStage;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int id = tid + kThreads * p;
          *(v4i*)(sb + bf16_k_off(id >> 4, id & 15)) = kreg[p];
        }
        uint8_t* sv = sb + kKBytes;
        const int grp = v_kg >> 1, within = 8 * (v_kg & 1);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = (uint32_t)vreg[0][w], a1 = (uint32_t)vreg[1][w];
          const uint32_t a2 = (uint32_t)vreg[2][w], a3 = (uint32_t)vreg[3][w];
          v2i even, odd;  // d = 8dc + 2w (low halves) and 8dc + 2w + 1 (high halves), keys 0..3
          even[0] = (int)perm(a1, a0, 0x05040100u);
          even[1] = (int)perm(a3, a2, 0x05040100u);
          odd[0] = (int)perm(a1, a0, 0x07060302u);
          odd[1] = (int)perm(a3, a2, 0x07060302u);
          *(v2i*)(sv + bf16_vt_off(8 * v_dc + 2 * w, grp) + within) = even;
          *(v2i*)(sv + bf16_vt_off(8 * v_dc + 2 * w + 1, grp) + within) = odd;
        }
      };

      load_kv(0);
      store_kv(0);
      __syncthreads();

      for (int kb = 0; kb < nb; ++kb) {
        const int key0 = kb * kBlockKeys;
        const int cur = kb & 1;
        if (kb + 1 < nb) load_kv(key0 + kBlockKeys);

        if (key0 <= row0 + kWaveRows - 1) {
          const uint8_t* sk = smem + cur * kStage;
          const uint8_t* sv = sk + kKBytes;
          v16f sacc[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[u][r] = 0.f;
            const int row = 32 * u + key_perm_bf16(l32);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) {
              const v4i x = *(const v4i*)(sk + bf16_k_off(row, 2 * mm + hh));
              sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(x), qop[mm], sacc[u], 0, 0, 0);
            }
          }
          // causal mask: lane half hh, sub-tile u, register r holds key key0+32u+16(r/8)+8hh+r%8
          if (key0 + kBlockKeys - 1 > row0) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (key0 + 32 * u + 16 * (r >> 3) + 8 * hh + (r & 7) > qrow) sacc[u][r] = -INFINITY;
          }
          float x = -INFINITY;
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; r += 2) x = fmax3(x, sacc[u][r], sacc[u][r + 1]);
          const float tmax = max_with_partner(x) * cp;
          if (kb == 0) {
            m = tmax;
          } else {
            const float M = fmaxf(m, tmax);
            if (__any((M - m) >= kTauBf16)) {
              const float f = __builtin_amdgcn_exp2f(m - M);
#pragma unroll
              for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= f;
              l *= f;
              m = M;
            }
          }
          const float nm = -m;
          v4i pb[8];  // P^T operand per 16-key MFMA step: 8 bf16 of sub-tile mm/2, regs 8(mm%2)..
#pragma unroll
          for (int mm = 0; mm < 8; ++mm) {
            const int u = mm >> 1, r0 = 8 * (mm & 1);
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + e], cp, nm));
              l += p[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) pb[mm][e] = (int)pack_bf16x2(p[2 * e], p[2 * e + 1]);
          }
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int d = 32 * dt + l32;
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) {
              const v4i x = *(const v4i*)(sv + bf16_vt_off(d, 2 * mm + hh));
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(x), as_bf(pb[mm]), oacc[dt], 0, 0, 0);
            }
          }
        }

        if (kb + 1 < nb) store_kv(cur ^ 1);
        __syncthreads();
      }

      const float lt = sum_with_partner(l);
      const float inv = 1.0f / lt;
      uint16_t* op = a.out + ((int64_t)(b * S + qrow) * H + h) * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hh;
          uint2 w;
          w.x = pack_bf16x2(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
          w.y = pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
          *(uint2*)(op + d0) = w;
        }
      if (a.lse != nullptr && hh == 0) a.lse[(int64_t)(b * H + h) * S + qrow] = kLn2 * (m + __log2f(lt));
    }
  }
}

}  // namespace

hipError_t launch_bf16(const Bf16Args& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cfa
