// Causal attention forward with BF16 operands on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Follows "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4":
//   Sec. II-B  base-2 online softmax over key blocks (128 keys at d_qk = 128, as the paper
//              prices a BF16 block in Table III; 64 at the MLA shape), LSE output;
//   Sec. IV-A  8 waves x 32 query rows, S^T = K Q^T so each lane holds one query's
//              scores, causal pairing (with grouped-query attention and an even group, a
//              tile is 128 rows of each of two query heads), persistent grid, chiplet map,
//              lazy rescaling with tau = 4 at d_qk = 128 and 8 at the MLA shape d_qk = 192;
//   Sec. VI-A  dead-block skip: in the diagonal blocks a wave skips the key blocks
//              that the causal mask hides from all its rows (loads and barriers still run);
//   Sec. IV-D  the 8-wave ping-pong of the BF16 d = 128 kernel: the two waves of a SIMD
//              alternate between issuing the block's matrix products and computing the
//              softmax, with a workgroup barrier per phase;
//   Sec. VI-A  the softmax scale multiplies the fp32 scores (not folded into bf16 Q).
//
// Schedule and barrier placement follow the FP8 kernel (attn_fp8.hip): group 1 (waves 4-7)
// runs one phase behind group 0; M_i issues O += V(i)^T P(i) and S(i+1) = K(i+1) Q^T as one
// stream of MFMAs and their operand reads (each operand read three MFMAs ahead through a
// ring of registers, consecutive MFMAs on different accumulators, the K reads of the QK
// part issued behind the last PV MFMAs); the first three V operands of M_i are read at the
// end of S_{i-1}, after its wait for the copies (V(i) has been in LDS since the phase
// before), so the matrix phase starts with its operands in registers.  On a wave's last
// live block the QK part still runs, on the other K slot (in-bounds LDS, scores unused),
// which keeps one shape of the stream.  S_i takes the next block's maximum, the lazy
// decision (with the rare rescale of O and l) and forms P(i+1).  K and V blocks move by DMA:
// group 0 copies K(i+2) into the slot of K(i) (two K slots) at the end of M_i, after the
// phase's last operand read.  With three V slots (d_qk = 192) group 1 copies V(i+2) into the
// slot of V(i-1) at the end of its M_i; with two (d_qk = 128, whose 128-key slots leave no room
// for a third) it copies V(i+2) into the slot of V(i) at the start of its S_i, once the barrier
// has closed both groups' reads of V(i).  Each wave waits for its copies at the end of S_i.
// Every target slot was last read before the copy's issuing barrier and every copy
// completes at least one phase before its first read.
// The epilogue first requests the Q rows of the wave's next tile, then stores O as whole rows
// through a per-wave LDS staging area, as in the FP8 kernel.
//
// fp32 arithmetic: t = s * cp with cp = fp32(c log2 e); p = exp2(fmaf(s, cp, -m));
// l sums the fp32 p; P is p rounded to bf16; O = bf16(acc / l); LSE = ln 2 (m + log2 l).
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace cfa {

namespace {

// lazy-rescale threshold in base-2 units of the score (Sec. IV-A): 4 at d_qk = 128 and 8 at
// the MLA shape d_qk = 192, so p stays below 2^4 or 2^8 in fp32 between rescales.  P is rounded
// to bf16 relative to its own size, so the threshold does not change the accuracy; a larger one
// saves rescales of O (measured at d_qk = 128: 0.5 -> 4 gave 2-4%, 8 no more).
template <int DQK>
constexpr float kTauBf16 = DQK == 128 ? 4.0f : 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;

// LDS: two K slots then two or three V slots, each a run of 16-byte cells filled by DMA
// (global_load_lds: lane L of a wave writes cell base + L); pad cells receive a copy of a
// data cell of the same row (no per-lane masking) and are never read.
//   K slot: row 32*(key/32) + key_perm_bf16(key%32) holds key `key` (key_perm_bf16 is an
//           involution), d_qk/8 + 1 cells per row (272 bytes at d_qk = 128, 400 at 192;
//           both keep each 16-lane group of a 16-byte read on distinct banks), so lane i
//           reads row 32u + i, which holds key 32u + key_perm_bf16(i).
//   V slot: row r holds V[key0 + r][0..127], 20 cells (320 bytes) per row; the PV operand
//           (V^T) comes from LDS transpose reads.  A transpose read takes 8 bytes per lane
//           from 4 consecutive rows per 16-lane group, and the two 16-lane groups of a lane
//           half read neighbouring 32-byte pieces of the same rows; with a 320-byte stride the
//           8 pieces of 32 lanes fall on distinct banks (a 288-byte stride made them collide,
//           measured as 5.4e8 bank-conflict cycles per call at B1 H32 S32768, now 3e6).
// keys per block (max update, ping-pong phase and LDS slot): 128 at d_qk = 128, where two K and
// two V slots fit LDS; 64 at d_qk = 192, whose 400-byte K rows leave room for three V slots
template <int DQK>
constexpr int kBlkOf = DQK == 128 ? 128 : 64;
template <int DQK>
struct Bf16Lds {
  static constexpr int kBlk = kBlkOf<DQK>;
  static constexpr int kVSlots = DQK == 128 ? 2 : 3;
  static constexpr int kKCols = DQK / 8;  // 16-byte data cells per K row
  static constexpr int kKSpr = kKCols + 1;
  static constexpr int kKStride = 16 * kKSpr;
  static constexpr int kKCells = kBlk * kKSpr;
  static constexpr int kKSlot = 16 * kKCells;
  static constexpr int kVSpr = 20;
  static constexpr int kVStride = 16 * kVSpr;
  static constexpr int kVCells = kBlk * kVSpr;
  static constexpr int kVSlot = 16 * kVCells;
  static constexpr int kVBase = 2 * kKSlot;
  static constexpr int kLdsBytes = 2 * kKSlot + kVSlots * kVSlot;
  static constexpr int kRounds = ((kKCells > kVCells ? kKCells : kVCells) + 255) / 256;
};

// max of two floats that are never NaN, as one v_max_f32 (fmaxf would first quiet both
// operands, which the compiler cannot prove unnecessary for MFMA and permlane results)
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// a barrier that leaves this wave's LDS reads in flight: for reads of data that no wave
// overwrites before the reading wave's next barrier (the compiler waits for them at first use)
__device__ __forceinline__ void barrier_reads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v8bf as_bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// maximum of N floats that are never NaN, as a tree of three-input maxima
template <int N>
__device__ __forceinline__ float max_tree(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return max2(x[0], x[1]);
  } else {
    constexpr int M = (N + 2) / 3;
    float y[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (3 * i + 2 < N)
        y[i] = fmax3(x[3 * i], x[3 * i + 1], x[3 * i + 2]);
      else if (3 * i + 1 < N)
        y[i] = max2(x[3 * i], x[3 * i + 1]);
      else
        y[i] = x[3 * i];
    }
    return max_tree<M>(y);
  }
}

// O staging for the epilogue: a 32-row area per wave with a 272-byte row pitch, so the
// 16-byte pieces that 16 consecutive rows write at one column fall on distinct banks
constexpr int kStgPitch = 272;
constexpr int kStgWave = kWaveRows * kStgPitch;
static_assert(kThreads / 64 * kStgWave <= Bf16Lds<128>::kLdsBytes, "O staging exceeds the LDS of the kernel");

template <int DQK>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(Bf16Args a) {
  using L = Bf16Lds<DQK>;
  constexpr int kKStride = L::kKStride, kKCells = L::kKCells, kKSlot = L::kKSlot, kKSpr = L::kKSpr;
  constexpr int kVStride = L::kVStride, kVCells = L::kVCells, kVSlot = L::kVSlot, kVSpr = L::kVSpr;
  constexpr int kVBase = L::kVBase, kRounds = L::kRounds;
  constexpr int kBlk = L::kBlk, kVS = L::kVSlots;
  constexpr int NU = kBlk / 32;  // 32-key sub-tiles of a block (score accumulators)
  constexpr int NM = kBlk / 16;  // 16-key steps of a block (P operands)
  constexpr int QM = DQK / 16;  // 16-deep k steps of S^T = K Q^T
  constexpr float kTau = kTauBf16<DQK>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;
  const int S = a.S, H = a.H;
  // head-pair mode: a tile is 128 rows of each of the heads h (waves 0-3) and h+1 (waves 4-7)
  const bool pair = a.pair_heads != 0;
  const Schedule sch = make_schedule(a.B, H, S, pair);
  const int hstep = pair ? 2 : 1;
  const int trows = pair ? kPairTileRows : kTileRows;
  const int wrow = pair ? (wave & 3) : wave;  // the wave's 32-row slot in the tile
  const ItemRange work = xcd_items(blockIdx.x, gridDim.x, sch.items);
  const int krs = a.mk.ss, vrs = a.mv.ss;  // key / value row strides in bytes

  const int k_rd = l32 * kKStride + 16 * hh;
  // V transpose-read base: 16-lane group G = lane/16, source lane s = lane%16 reads key
  // 8hh + s/4 (+ 16mm + 4q), bf16 elements 32dt + 16 (G%2) + 4 (s%4) .. +3
  const int v_tr = kVBase + (8 * hh + ((lane & 15) >> 2)) * kVStride + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  // staging by DMA: the 256 threads of group 0 copy K blocks, those of group 1 V blocks.
  // Round p, thread st covers cell 256p + st of the slot; st_goff is its source offset
  // from the block's first key (pad cells copy column 0 of their row).  Waves whose cells
  // of a round lie past the end of the slot skip that round (a wave-uniform test).
  const int st = tid & 255;
  const bool stage_k = (grp == 0);
  const int wq = wave & 3;
  const int st_cells = stage_k ? kKCells : kVCells;
  uint32_t st_goff[kRounds];
#pragma unroll
  for (int p = 0; p < kRounds; ++p) {
    const int cell = 256 * p + st;
    if (stage_k) {
      const int row = (cell / kKSpr) & (kBlk - 1), col = cell % kKSpr;
      st_goff[p] = ((row & ~31) | key_perm_bf16(row & 31)) * krs + 16 * (col < L::kKCols ? col : 0);
    } else {
      const int row = (cell / kVSpr) & (kBlk - 1), col = cell % kVSpr;
      st_goff[p] = row * vrs + 16 * (col < 16 ? col : 0);
    }
  }
  const int st_lds = 16 * 64 * wq + (stage_k ? 0 : kVBase);
  const v16f zero16 = {};
  const float cp = a.cp;

  // (b, h, j) of the workgroup's first item; later items follow by scalar increments, so the
  // loop holds no division (whose reciprocals the compiler would keep in vector registers)
  int b, h, j;
  decode_item(work.first, sch.HS, sch.P, b, h, j);
  h *= hstep;
  int hk = h / a.G, hg = h - hk * a.G;  // key/value head of query head h, and h's place in its group
  // the item after (b, h, j): work.step items on
  auto next_item = [&](int& b_, int& h_, int& hk_, int& hg_, int& j_) {
    j_ += work.step;
    while (j_ >= sch.P) {
      j_ -= sch.P;
      hg_ += hstep;
      if (hg_ == a.G) {
        hg_ = 0;
        ++hk_;
      }
      h_ += hstep;
      if (h_ == H) {
        h_ = hg_ = hk_ = 0;
        ++b_;
      }
    }
  };
  // Q^T operand (lane holds Q[qrow][16m + 8hh .. +8]) of a tile: the first tile's here, every
  // later one's at the start of the epilogue before it, so the load overlaps that epilogue
  v4i qop[QM];
  auto load_q = [&](int b_, int h_, int tile_) {
    const uint8_t* qh = (const uint8_t*)a.q + b_ * a.mq.sb + (h_ + (pair ? grp : 0)) * a.mq.sh;
    const int ln = lane_now();
    const uint8_t* qp = qh + (int64_t)(tile_ * trows + wrow * kWaveRows + (ln & 31)) * a.mq.ss + 16 * (ln >> 5);
#pragma unroll
    for (int mm = 0; mm < QM; ++mm) qop[mm] = *(const v4i*)(qp + 32 * mm);
  };
  // item indices fit in 32 bits (B H S is below 2^31 / d_qk); a 32-bit loop bound stays scalar
  const int wfirst = (int)work.first, wend = (int)work.end;
  if (wfirst < wend) load_q(b, h, sch.T - 1 - j);
  for (int item = wfirst; item < wend; item += work.step) {
    const int hw = h + (pair ? grp : 0);  // the wave's query head
    const uint8_t* st_head = stage_k ? (const uint8_t*)a.k + b * a.mk.sb + hk * a.mk.sh
                                     : (const uint8_t*)a.v + b * a.mv.sb + hk * a.mv.sh;
    const int st_rs = stage_k ? krs : vrs;

    for (int pass = 0; pass < 2; ++pass) {
      // the long tile of the pair first: the workgroups of one XCD then start on key block 0
      // together and read the same K/V blocks from its L2 for most of that tile
      const int tile = pass == 0 ? sch.T - 1 - j : j;
      if (pass == 1 && tile == sch.T - 1 - j) break;
      const int row0 = tile * trows + wrow * kWaveRows;
      const int qrow = row0 + l32;
      const int nb = (tile + 1) * (trows / kBlk);  // key blocks

      // DMA of block blk: K into slot blk % 2, V into slot blk % kVS.  stage() goes through a
      // scalar base (copy_round: no per-lane 64-bit addresses, which the compiler would keep,
      // spill and reload at every tile start, and no vector instructions to form them): the
      // prologue uses it, and so does the loop at d_qk = 128, where group 1 issues its V copies
      // inside the softmax phase and the address arithmetic of the builtin competed with the
      // softmax (4.5% at 16K-32K).  With 64-key blocks (d_qk = 192) the loop keeps the builtin,
      // whose per-lane address cost less there than the asm round's wait states and M0 handling.
      auto stage = [&](int blk) {
        const uint64_t gs = (uint64_t)(uintptr_t)(st_head + (int64_t)(blk * kBlk) * st_rs);  // wave-uniform
        const uint32_t mb = __builtin_amdgcn_readfirstlane(
            lds_addr(smem) + st_lds + (stage_k ? (blk & 1) * kKSlot : (blk % kVS) * kVSlot));
#pragma unroll
        for (int p = 0; p < kRounds; ++p)
          if (256 * p + 64 * wq < st_cells) copy_round(gs, mb + 4096 * p, st_goff[p]);
      };
      auto stage_loop = [&](int blk) {
        const uint8_t* src = st_head + (int64_t)(blk * kBlk) * st_rs;
        uint8_t* dst = smem + st_lds + (stage_k ? (blk & 1) * kKSlot : (blk % kVS) * kVSlot);
#pragma unroll
        for (int p = 0; p < kRounds; ++p)
          if (256 * p + 64 * wq < st_cells) dma16(src + st_goff[p], dst + 4096 * p);
      };

      v16f oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = zero16;
      v16f sacc[NU];  // scores of the next block (32-key sub-tiles)
      v4i pb[NM];     // P^T operand per 16-key step
      float m = 0.f, l = 0.f;

      auto live = [&](int blk) { return blk * kBlk <= row0 + kWaveRows - 1; };
      // S^T(blk) = K(blk) Q^T.  The two sub-tiles alternate, so consecutive MFMAs are
      // independent, and each MFMA's operand is read one MFMA ahead.
      auto qk = [&](int blk) {
        const uint8_t* sk = smem + (blk & 1) * kKSlot + k_rd;
        auto kread = [&](int t) { return *(const v4i*)(sk + 32 * (t % NU) * kKStride + 32 * (t / NU)); };
        constexpr int D = 3;        // operand reads in flight ahead of the MFMAs
        constexpr int N = NU * QM;  // MFMAs
        v4i kop[D + 1];
#pragma unroll
        for (int t = 0; t < D; ++t) kop[t] = kread(t);
#pragma unroll
        for (int t = 0; t < N; ++t) {
          const int u = t % NU, mm = t / NU;
          if (t + D < N) kop[(t + D) % (D + 1)] = kread(t + D);
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kop[t % (D + 1)]), as_bf(qop[mm]),
                                                            mm == 0 ? zero16 : sacc[u], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
#pragma unroll
        for (int t = 0; t < N - D; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, D, 0);
      };
      // causal mask (lane half hh, sub-tile u, register r holds key key0+32u+16(r/8)+8hh+r%8),
      // running max and the lazy decision
      auto max_step = [&](int blk, bool first) {
        const int key0 = blk * kBlk;
        if (key0 + kBlk - 1 > row0) {
#pragma unroll
          for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (key0 + 32 * u + 16 * (r >> 3) + 8 * hh + (r & 7) > qrow) sacc[u][r] = -INFINITY;
        }
        // v_max3 tree over the lane's scores of the block
        float x[NU * 16];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[16 * u + r] = sacc[u][r];
        const float y = max_tree<NU * 16>(x);
        const uint32_t yu = __float_as_uint(y);
        const auto sw = __builtin_amdgcn_permlane32_swap(yu, yu, false, false);
        const float tmax = max2(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cp;
        if (first) {
          m = tmax;
        } else {
          const float M = fmaxf(m, tmax);
          if (__any((M - m) >= kTau)) {  // O and l hold blocks <= blk-1
            const float f = __builtin_amdgcn_exp2f(m - M);
            l *= f;
            m = M;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) oacc[dt] *= f;
          }
        }
      };
      auto probs = [&]() {
        const float nm = -m;
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) {
          const int u = mm >> 1, r0 = 8 * (mm & 1);
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[u][r0 + e], cp, nm));
          l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[mm][e] = (int)cvt_pk_bf16(p[2 * e], p[2 * e + 1]);
        }
      };
      // Operand stream of a matrix phase: the 16 PV MFMAs (O^T += V^T P^T) of block blk, then
      // the 2 QM QK MFMAs of block blk+1.  Operand t is read kDist MFMAs ahead of its MFMA
      // through the ring opb; the first kDist (V operands) are read by preload().
      constexpr int kDist = 3;
      constexpr int NQ = NU * QM;
      v4i opb[kDist + 1];
      // lane: V^T operand d = 32dt + l32 over keys 16mm + 8hh + 0..7 (two transpose reads);
      // K operand as in qk()
      auto opread = [&](int blk, int t) -> v4i {
        if (t < 4 * NM) {
          const uint8_t* sv = smem + (blk % kVS) * kVSlot + v_tr;
          const int dt = t & 3, mm = t >> 2;
          const v2i r0 = lds_tr16(sv + (16 * mm) * kVStride + 64 * dt);
          const v2i r1 = lds_tr16(sv + (16 * mm + 4) * kVStride + 64 * dt);
          return (v4i){r0[0], r0[1], r1[0], r1[1]};
        }
        const int tq = t - 4 * NM;
        const uint8_t* sk = smem + ((blk + 1) & 1) * kKSlot + k_rd;
        return *(const v4i*)(sk + 32 * (tq % NU) * kKStride + 32 * (tq / NU));
      };
      auto preload = [&](int blk) {
#pragma unroll
        for (int t = 0; t < kDist; ++t) opb[t] = opread(blk, t);
      };
      auto stream = [&](int blk) {
        constexpr int N = 4 * NM + NQ;
#pragma unroll
        for (int t = 0; t < N; ++t) {
          if (t + kDist < N) opb[(t + kDist) % (kDist + 1)] = opread(blk, t + kDist);
          const v4i op = opb[t % (kDist + 1)];
          if (t < 4 * NM) {
            const int dt = t & 3, mm = t >> 2;
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(op), as_bf(pb[mm]), oacc[dt], 0, 0, 0);
          } else {
            const int tq = t - 4 * NM, u = tq % NU, mm = tq / NU;
            sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(op), as_bf(qop[mm]), mm == 0 ? zero16 : sacc[u],
                                                              0, 0, 0);
          }
        }
        // issue order: each MFMA, then the reads of the operand kDist MFMAs ahead of it
#pragma unroll
        for (int t = 0; t < N; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          const int nr = t + kDist < N ? (t + kDist < 4 * NM ? 2 : 1) : 0;
          if (nr == 2)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          else if (nr == 1)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      };

      // prologue: only the Q rows and block 0 are waited for before the first barrier; block 1
      // streams in under the first two phases, each wave waiting for its share at the end of
      // its S_pro (K(1) is first read in M_0, V(1) in S_0).  Tile 0 of the head-pair mode at
      // d_qk = 128 has one block; its block 1 (keys 128-255, present since S >= 256) is copied
      // unused.
      stage(0);
      wait_dma();
      lds_barrier();
      stage(1);
      if (grp == 1) lds_barrier();

      if (live(0)) qk(0);
      lds_barrier();
      if (live(0)) {
        max_step(0, true);
        probs();
        preload(0);
      }
      wait_dma();
      lds_barrier();

      for (int i = 0; i < nb; ++i) {
        // -------------------------------------------------------------- M_i
        __builtin_amdgcn_s_setprio(1);
        const bool live_i = live(i), live_n = (i + 1 < nb) && live(i + 1);
        if (live_i) stream(i);
        // after this phase's last operand read: K(i+2) by group 0 into the slot of K(i), and with
        // three V slots V(i+2) by group 1 into the slot of V(i-1); waited for at the end of S_i
        if (i + 2 < nb && (stage_k || kVS == 3)) {
          if constexpr (kVS == 2)
            stage(i + 2);
          else
            stage_loop(i + 2);
        }
        lds_barrier();
        // -------------------------------------------------------------- S_i
        __builtin_amdgcn_s_setprio(0);
        // with two V slots, V(i+2) goes into the slot of V(i), which this group read in M_i and
        // the other group a phase earlier: free only after the barrier just passed
        if (kVS == 2 && !stage_k && i + 2 < nb) stage(i + 2);  // through the scalar base
        if (live_n) {
          max_step(i + 1, false);
          probs();
        }
        if (i + 2 < nb) wait_dma();
        // V(i+1): its copy was waited for at least one phase ago, and its slot is next written
        // at the start of the other group's S_{i+1} (two V slots) or in M_{i+2} (three), after
        // this wave's M_{i+1} has used the reads, so they may complete after the barrier
        if (live_n) preload(i + 1);
        barrier_reads_in_flight();
      }
      if (grp == 0) lds_barrier();

      // epilogue: O through a per-wave LDS staging area, stored as whole 256-byte rows (the
      // barrier at the end keeps the next tile's copies out until every wave has read its area)
      if (pass == 0 && j != sch.T - 1 - j) {
        load_q(b, h, j);
      } else if (item + work.step < wend) {
        int b1 = b, h1 = h, hk1 = hk, hg1 = hg, j1 = j;
        next_item(b1, h1, hk1, hg1, j1);
        load_q(b1, h1, sch.T - 1 - j1);
      }
      const float lt = sum_with_partner(l);
      const float inv = 1.0f / lt;
      uint8_t* stg = smem + wave * kStgWave;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hh;
          uint2 w;
          w.x = cvt_pk_bf16(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
          w.y = cvt_pk_bf16(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
          *(uint2*)(stg + l32 * kStgPitch + 2 * d0) = w;
        }
      {
        uint8_t* orow = (uint8_t*)a.out + b * a.mo.sb + hw * a.mo.sh + (int64_t)row0 * a.mo.ss;
        const int ln = lane_now();
        const int sr = ln >> 4, sc = 16 * (ln & 15);
#pragma unroll
        for (int s4 = 0; s4 < kWaveRows / 4; ++s4) {
          const int r = 4 * s4 + sr;
          *(v4i*)(orow + (int64_t)r * a.mo.ss + sc) = *(const v4i*)(stg + r * kStgPitch + sc);
        }
      }
      if (a.lse != nullptr && hh == 0) a.lse[(int64_t)(b * H + hw) * S + qrow] = kLn2 * (m + __log2f(lt));
      lds_barrier();
    }
    // the workgroup's next item, work.step items on
    if (item + work.step >= wend) break;
    next_item(b, h, hk, hg, j);
  }
}

}  // namespace

hipError_t launch_bf16(const Bf16Args& a, int dqk, int grid, hipStream_t stream) {
  if (dqk == 128)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<192>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cfa
