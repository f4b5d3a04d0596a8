// Causal attention forward with FP8 e4m3 operands on gfx950 MFMA.
//
// Follows "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4":
//   Sec. II-B          base-2 online softmax over key blocks, LSE output;
//   Sec. II-C          per-tensor scales folded into the score scale and the output;
//   Sec. IV-A          8 waves x 32 query rows, S^T = K Q^T, lazy rescaling (tau = 0.125);
//   Sec. IV-B1, Eq. 2  lean P: one FMA + one integer conversion per probability (d_qk = 128);
//                      exact P: FMA + exp2 + e4m3 conversion (MLA shape, d_qk = 192);
//   Sec. IV-B2         per (query, 64-key block) power-of-two scale 2^o, removed by the
//                      E8M0 operand scale of the PV MFMA;
//   Sec. IV-B3         row sum of the rounded probabilities on the matrix unit;
//   Sec. IV-C, Fig. 6  two-wave ping-pong: the two waves of a SIMD alternate between an
//                      MFMA phase (row sums, S^T of the next block, PV of the current
//                      block, next block's maximum and rescale decision) and a softmax
//                      phase (the probability codes), with a workgroup barrier per phase.
//
// Schedule per 256-row tile with nb 128-key blocks.  Group g = wave / 4 (one wave of
// each group per SIMD).  Group 1 runs one phase behind group 0:
//   group 0:  M_pro S_pro M_0 S_0 M_1 S_1 ... M_{nb-1} S_{nb-1} idle
//   group 1:  idle  M_pro S_pro M_0 S_0 ... M_{nb-1} S_{nb-1}
// M_i: row sums of P(i); S(i+1) = K(i+1) Q^T; O += V(i)^T P(i); max of S(i+1), lazy
//      decision, o(i+1).   S_i: P(i+1) from S(i+1).
// Staging (global -> registers -> LDS within S_i): group 0 stages K(i+2), group 1
// stages V(i+2)^T.  With two LDS slots per operand every write lands one phase
// after the slot's last read and at least one phase before its first read.
//
// fp32 arithmetic (the order below is part of the contract with the test oracle):
//   cp   = fp32(c * dq * dk * log2 e), scores s are fp32 MFMA sums
//   t    = s * cp;  M = max(m, max t);  lazy: keep m unless some row of the wave
//          grows by >= tau; rescale factor 2^(m - M)
//   o    = clamp(floor(m - b), 0, 127), b = max t over the 64-key block
//   lean P:  y = fmaf(s, 8 cp, 8 ((13 + o) - m) - 0.35);  code = cvt_pk_u8(y)
//   exact P: x = fmaf(s, cp, (6 + o) - m);  code = e4m3_rne(exp2(x))
//   l   += 2^-o * (sum of decoded codes of the block)   [MFMA sum, then one fp32 FMA]
//   O    = bf16_rne(acc * (dv / l)),  LSE = ln 2 * (m + log2 l - 6)
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

constexpr float kTauFp8 = 0.125f;  // lazy-rescale threshold, base-2 units (Sec. IV-A)
constexpr int kSigma = 6;          // probability shift 2^6 (Sec. IV-B1)
constexpr float kBeta = 0.35f;     // lean-P bias (Sec. IV-B1, Eq. 2)
constexpr float kLn2 = 0.69314718055994530942f;

// LDS: two K slots then two V^T slots.
//   K slot: row 32*(key/32) + kinv(key%32) holds key `key`, row stride DQK + 16 bytes, so
//           lane i of a wave reads row 32u + i, which holds key 32u + key_perm_fp8(i).
//   V^T slot: row d (128 rows, stride 144 bytes) holds V[key][d] for the block's 128 keys,
//           16-byte key groups stored with bits 0 and 1 of the group index swapped, so a
//           lane's 32 PV operand bytes (keys 64n+16hh+j and 64n+32+16hh+j) are contiguous.
template <int DQK>
struct Fp8Lds {
  static constexpr int kKc = DQK / 64;
  static constexpr int kKStride = DQK + 16;
  static constexpr int kKSlot = 128 * kKStride;
  static constexpr int kVStride = 144;
  static constexpr int kVSlot = 128 * kVStride;
  static constexpr int kVBase = 2 * kKSlot;
  static constexpr int kBytes = 2 * kKSlot + 2 * kVSlot;
  static constexpr int kKChunksPerThread = 128 * DQK / 16 / 256;  // staged by 256 threads
};

__device__ __forceinline__ int kinv(int k) { return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3); }
__device__ __forceinline__ int vt_group(int g) { return (g & 4) | ((g & 1) << 1) | ((g >> 1) & 1); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DQK, bool EXACT_P, bool DEBUG>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(Fp8Args a) {
  using L = Fp8Lds<DQK>;
  constexpr int KC = L::kKc;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  const int S = a.S, H = a.H;
  const Schedule sch = make_schedule(a.B, H, S);
  const int logical = xcd_logical(blockIdx.x, gridDim.x);

  const int krs = H * DQK;  // BSHD key row stride in bytes (tensor < 2^31 elements)
  const int vrs = H * 128;

  // per-lane LDS read bases
  const int k_rd = l32 * L::kKStride + 32 * hh;
  const int v_rd = L::kVBase + l32 * L::kVStride + 32 * hh;

  // staging assignments: the 256 threads of group 0 stage K, those of group 1 stage V^T.
  // Both use one register array and the same load code; only the LDS store differs.
  constexpr int NST = L::kKChunksPerThread;  // 16-byte chunks per staging thread (>= 4)
  const int st = tid & 255;
  const bool stage_k = (grp == 0);
  const int st_rs = stage_k ? krs : vrs;  // global row stride of the staged tensor
  int st_goff[NST], k_soff[NST];
  const int v_kg = st & 31, v_dc = st >> 5;  // V: keys 4kg..4kg+3, d 16dc..16dc+15
#pragma unroll
  for (int p = 0; p < NST; ++p) {
    const int id = st + 256 * p, key = id / (DQK / 16), gg = id % (DQK / 16);
    st_goff[p] = stage_k ? key * krs + 16 * gg : (4 * v_kg + (p & 3)) * vrs + 16 * v_dc;
    k_soff[p] = ((key & ~31) | kinv(key & 31)) * L::kKStride + 16 * gg;
  }
  const int v_soff = L::kVBase + 16 * v_dc * L::kVStride + 16 * vt_group(v_kg >> 2) + 4 * (v_kg & 3);

  // row-sum selector (Sec. IV-B3): lane L of the 16x16x128 A operand is all ones
  // iff (L/16)%2 == ((L%16)/4)%2, so every lane receives the sum of its own query.
  const int sel_on = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1));
  const int selw = sel_on ? 0x38383838 : 0;
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  const v16f zero16 = {};

  const float cp = a.cp;
  const float cp8 = 8.0f * cp;

  for (int64_t item = logical; item < sch.items; item += gridDim.x) {
    int b, h, j;
    decode_item(item, H, sch.P, b, h, j);
    const uint8_t* qbh = a.q + ((int64_t)b * S * H + h) * DQK;
    const uint8_t* st_head = stage_k ? a.k + ((int64_t)b * S * H + h) * DQK : a.v + ((int64_t)b * S * H + h) * 128;

    for (int pass = 0; pass < 2; ++pass) {
      const int tile = pass == 0 ? j : sch.T - 1 - j;
      if (pass == 1 && tile == j) break;
      const int row0 = tile * kTileRows + wave * kWaveRows;  // first query row of this wave
      const int qrow = row0 + l32;
      const int nb = 2 * tile + 2;                             // 128-key blocks

      // ---------------------------------------------------------------- staging
      v4i stg[NST];
      auto stage_load = [&](int blk) {  // global -> registers for block blk
        const uint8_t* base = st_head + (int64_t)(blk * kBlockKeys) * st_rs;
#pragma unroll
        for (int p = 0; p < NST; ++p)
          if (p < 4 || stage_k) stg[p] = *(const v4i*)(base + st_goff[p]);
      };
      auto stage_store = [&](int blk) {  // registers -> LDS slot blk % 2
        const int slot = blk & 1;
        if (stage_k) {
          uint8_t* sk = smem + slot * L::kKSlot;
#pragma unroll
          for (int p = 0; p < NST; ++p) *(v4i*)(sk + k_soff[p]) = stg[p];
        } else {
          uint8_t* sv = smem + slot * L::kVSlot + v_soff;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {  // d 16dc + 4q4 .. +3
            uint32_t r[4], t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = (uint32_t)stg[i][q4];
            transpose4x4_u8(r, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) *(uint32_t*)(sv + (4 * q4 + e) * L::kVStride) = t[e];
          }
        }
      };

      // ---------------------------------------------------------------- per-wave state
      v8i qop[KC];
      {
        const uint8_t* qp = qbh + (int64_t)qrow * krs + 32 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) qop[c] = *(const v8i*)(qp + 64 * c);
      }
      v16f oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = zero16;
      v16f sacc[4];  // scores of the next block
      v8i pb[2];     // codes of the current block, per 64-key scale block
      float m = 0.f, l = 0.f, fres = 1.f;
      int o_cur[2] = {0, 0}, o_nxt[2] = {0, 0};
      bool rescale = false;

      auto live = [&](int blk) { return blk * kBlockKeys <= row0 + kWaveRows - 1; };

      // S^T(blk) = K(blk) Q^T into sacc.  Chunk-outer order keeps consecutive MFMAs
      // independent; the operand of the next MFMA is read before the current one issues.
      auto qk = [&](int blk) {
        const uint8_t* sk = smem + (blk & 1) * L::kKSlot + k_rd;
        constexpr int N = 4 * KC;
        v8i kop[2];
        kop[0] = *(const v8i*)(sk);
#pragma unroll
        for (int t = 0; t < N; ++t) {
          const int c = t / 4, u = t % 4;
          if (t + 1 < N) {
            const int c1 = (t + 1) / 4, u1 = (t + 1) % 4;
            kop[(t + 1) & 1] = *(const v8i*)(sk + 32 * u1 * L::kKStride + 64 * c1);
          }
          sacc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[t & 1], qop[c], c == 0 ? zero16 : sacc[u], 0,
                                                                     0, 0, 127, 0, 127);
        }
        if constexpr (DQK == 128) {  // keep one operand read in flight ahead of each MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int t = 0; t < N - 1; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      };
      // mask, block maxima, running max with the lazy decision, exponents o for blk
      auto max_step = [&](int blk, bool first) {
        const int key0 = blk * kBlockKeys;
        if (key0 + kBlockKeys - 1 > row0) {  // diagonal block: key key0+32u+16hh+r
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (key0 + 32 * u + 16 * hh + r > qrow) sacc[u][r] = -INFINITY;
        }
        float bm[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float x = fmaxf(sacc[2 * n][0], sacc[2 * n][1]);
#pragma unroll
          for (int r = 2; r < 16; r += 2) x = fmax3(x, sacc[2 * n][r], sacc[2 * n][r + 1]);
#pragma unroll
          for (int r = 0; r < 16; r += 2) x = fmax3(x, sacc[2 * n + 1][r], sacc[2 * n + 1][r + 1]);
          bm[n] = max_with_partner(x) * cp;
        }
        if (first) {
          m = fmaxf(bm[0], bm[1]);
        } else {
          const float M = fmax3(m, bm[0], bm[1]);
          rescale = __any((M - m) >= kTauFp8);
          if (rescale) {
            fres = __builtin_amdgcn_exp2f(m - M);
            m = M;
          }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) o_nxt[n] = (int)fminf(fmaxf(floorf(m - bm[n]), 0.f), 127.f);
      };
      // probability codes of the scores in sacc (Sec. IV-B1)
      auto codes = [&](int blk) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          if constexpr (!EXACT_P) {
            const float cst = 8.0f * ((float)(kSigma + 7 + o_nxt[n]) - m) - kBeta;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const int u = 2 * n + (w >> 2), r0 = 4 * (w & 3);
              uint32_t x = 0;
              x = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sacc[u][r0 + 0], cp8, cst), 0, x);
              x = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sacc[u][r0 + 1], cp8, cst), 1, x);
              x = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sacc[u][r0 + 2], cp8, cst), 2, x);
              x = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(sacc[u][r0 + 3], cp8, cst), 3, x);
              pb[n][w] = (int)x;
            }
          } else {
            const float cst = (float)(kSigma + o_nxt[n]) - m;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const int u = 2 * n + (w >> 2), r0 = 4 * (w & 3);
              const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + 0], cp, cst));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + 1], cp, cst));
              const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + 2], cp, cst));
              const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + 3], cp, cst));
              int x = 0;
              x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, x, false);
              x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
              pb[n][w] = x;
            }
          }
        }
        o_cur[0] = o_nxt[0];
        o_cur[1] = o_nxt[1];
        if constexpr (DEBUG) {
          const int key0 = blk * kBlockKeys;
          uint8_t* orow = a.dbg_o + ((int64_t)(b * H + h) * S + qrow) * (S / 64);
          uint8_t* crow = a.dbg_codes + ((int64_t)(b * H + h) * S + qrow) * S;
          if (hh == 0) {
            orow[key0 / 64] = (uint8_t)o_cur[0];
            orow[key0 / 64 + 1] = (uint8_t)o_cur[1];
          }
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const int u = 2 * n + (w >> 2), r0 = 4 * (w & 3);
              *(uint32_t*)(crow + key0 + 32 * u + 16 * hh + r0) = (uint32_t)pb[n][w];
            }
        }
      };
      // row sums of the codes (Sec. IV-B3) and O^T += V^T P^T with the 2^-o operand scale
      auto rowsum_pv = [&](int blk) {
        const v8i sel = {selw, selw, selw, selw, selw, selw, selw, selw};
        v4f bs0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb[0], zero4, 0, 0, 0, 127, 0, 127);
        v4f bs1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb[1], zero4, 0, 0, 0, 127, 0, 127);
        const uint8_t* sv = smem + (blk & 1) * L::kVSlot + v_rd;
        v8i vop[2];
        vop[0] = *(const v8i*)(sv);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int n = t / 4, dt = t % 4;
          if (t + 1 < 8) {
            const int n1 = (t + 1) / 4, dt1 = (t + 1) % 4;
            vop[(t + 1) & 1] = *(const v8i*)(sv + 32 * dt1 * L::kVStride + 64 * n1);
          }
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[t & 1], pb[n], oacc[dt], 0, 0, 0, 127, 0,
                                                                      127 - o_cur[n]);
        }
        if constexpr (DQK == 128) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
          for (int t = 0; t < 7; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        }
        return (v2f){bs0[0], bs1[0]};
      };

      // ---------------------------------------------------------------- prologue
      // K(0), K(1) by group 0 threads and V(0), V(1) by group 1 threads
      stage_load(0);
      stage_store(0);
      stage_load(1);
      stage_store(1);
      lds_barrier();
      if (grp == 1) lds_barrier();  // group 1 runs one phase behind

      // M_pro
      if (live(0)) {
        qk(0);
        max_step(0, true);
      }
      lds_barrier();
      // S_pro
      if (live(0)) codes(0);
      lds_barrier();

      for (int i = 0; i < nb; ++i) {
        // -------------------------------------------------------------- M_i
        __builtin_amdgcn_s_setprio(1);
        const bool live_i = live(i), live_n = (i + 1 < nb) && live(i + 1);
        if (rescale) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt] *= fres;
          rescale = false;
        }
        if (live_n) qk(i + 1);
        v2f bsum = {0.f, 0.f};
        if (live_i) bsum = rowsum_pv(i);
        if (live_i) l = fmaf(bsum[1], __int_as_float((127 - o_cur[1]) << 23),
                             fmaf(bsum[0], __int_as_float((127 - o_cur[0]) << 23), l));
        if (live_n) {
          max_step(i + 1, false);
          if (rescale) l *= fres;
        }
        lds_barrier();
        // -------------------------------------------------------------- S_i
        __builtin_amdgcn_s_setprio(0);
        if (i + 2 < nb) stage_load(i + 2);  // in flight while the codes are formed
        if (live_n) codes(i + 1);
        if (i + 2 < nb) stage_store(i + 2);
        lds_barrier();
      }
      if (grp == 0) lds_barrier();

      // ---------------------------------------------------------------- epilogue
      const float inv = a.v_descale / l;
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
      if (a.lse != nullptr && hh == 0)
        a.lse[(int64_t)(b * H + h) * S + qrow] = kLn2 * (m + __log2f(l) - (float)kSigma);
    }
  }
}

}  // namespace

hipError_t launch_fp8(const Fp8Args& a, int dqk, bool debug, int grid, hipStream_t stream) {
  if (dqk == 128) {
    if (debug)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if (debug)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, true, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, true, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cfa
