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
//                      MFMA phase and a softmax phase, with a workgroup barrier per phase.
//                      The matrix phase is one block of hand-ordered instructions and, as
//                      the paper's MFMA wave does, takes the block maxima of the next block
//                      between its PV MFMAs.
//
// Schedule per tile (256 rows of one head, or in the head-pair mode 128 rows of each of two
// heads that share a key/value head) with nb 128-key blocks.  Group g = wave / 4 (one wave
// of each group per SIMD).  Group 1 runs one phase behind group 0:
//   group 0:  M_pro S_pro M_0 S_0 M_1 S_1 ... M_{nb-1} S_{nb-1} idle
//   group 1:  idle  M_pro S_pro M_0 S_0 ... M_{nb-1} S_{nb-1}
// M_i (matrix phase): row sums of P(i); S(i+1) = K(i+1) Q^T; O += V(i)^T P(i); l update;
//      the block maxima of S(i+1) (the softmax phase redoes them with the causal mask on the
//      blocks that cross a wave's diagonal).
// S_i (softmax phase): the masked block maxima on the diagonal, lazy decision (and the rare
//      rescale of O and l), o(i+1), P(i+1).
// Staging by DMA (global_load_lds, no registers): at the end of M_i, after its last
// operand read, group 0 copies K(i+2) into the slot of K(i) (two K slots) and group 1
// copies V(i+2) into the slot of V(i-1) (three V slots); each wave waits for its copies at
// the end of S_i.  Every target slot was last read in an earlier phase, every copy
// completes at least one phase before its first read, and the softmax phase reads no
// LDS, so nothing waits on a copy early.  Every step copies: in a tile's last two steps,
// which have no block i+2, the wave copies the tile's last block again into the slot the
// schedule frees.
// Epilogue: after the tile's last barrier no wave reads K or V, so each wave first requests
// the Q rows of its next tile (the operand registers are free now), then writes its 32 rows
// of bf16 O into a staging area of its own at the start of LDS and stores them as whole
// 256-byte rows; a barrier keeps the next tile's copies out until every wave has read its
// area.
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

// LDS: two K slots then three V slots, each a run of 16-byte cells written by DMA (lane L
// of a wave writes cell base + L).  Pad cells receive a copy of a data cell of the same row
// (no per-lane masking) and are never read.
//   K slot: row 32*(key/32) + kinv(key%32) holds key `key` (kKCols data cells + 1 pad cell
//           per row), so lane i of a wave reads row 32u + i, which holds key
//           32u + key_perm_fp8(i).
//   V slot: 32 groups, each of four 128-byte rows (8 data cells each) and one pad cell, so
//           row r starts at byte 128 r + 16 (r/4); then 32 spare cells (1088 cells, 17 DMA
//           instructions of 64 cells).  Key 32a + 8b + c (c < 8) of the block lives in row
//           32a + 8 (c%4) + c/4 + 2b.  The PV operand V^T comes from ds_read_b64_tr_b8: each
//           instruction reads 8 consecutive keys, which this placement spreads over rows
//           whose 16-byte cells fall in distinct bank groups (measured on gfx950: 192 bytes
//           per clock and CU, against 178 for a uniform 160-byte row stride).
// V slot placement: row of key k of the block, and its inverse
__host__ __device__ constexpr int v_row_of_key(int k) {
  return 32 * (k >> 5) + 8 * (k & 3) + ((k & 7) >> 2) + 2 * ((k >> 3) & 3);
}
__host__ __device__ constexpr int v_key_of_row(int r) {
  return 32 * (r >> 5) + 8 * ((r & 7) >> 1) + ((r & 31) >> 3) + 4 * (r & 1);
}
__host__ __device__ constexpr int v_row_offset(int r) { return 128 * r + 16 * (r >> 2); }
// Key-contiguous V (V^T rows: one row of S key bytes per channel d): the slot holds the 128
// channels as rows of 8 data cells and one pad cell (144 bytes, the K row pitch), so a PV
// operand is one 32-byte read per lane, conflict-free like the K reads.  Within each 64-key
// scale block the four 16-key cells are stored in the order 0, 2, 1, 3, so that lane half hh
// finds its keys 16 hh + 0..15 and 32 + 16 hh + 0..15 (the key order of the P operand)
// together at byte 32 hh of the block.
__host__ __device__ constexpr int vt_cell_src(int c) { return (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1); }

template <int DQK, bool VT = false>
struct Fp8Lds {
  static constexpr int kKCols = DQK / 16;
  static constexpr int kKSpr = kKCols + 1;  // cells per K row
  static constexpr int kKStride = 16 * kKSpr;
  static constexpr int kKCells = 128 * kKSpr;
  static constexpr int kKSlot = 16 * kKCells;
  static constexpr int kVGroupCells = 33;  // 4 rows of 8 cells + 1 pad cell
  static constexpr int kVtSpr = 9;         // key-contiguous V: cells per channel row
  // 32 groups + 32 spare cells (a whole last DMA instruction); or 128 channel rows
  static constexpr int kVCells = VT ? 128 * kVtSpr : 1088;
  static constexpr int kVSlot = 16 * kVCells;
  // byte offsets of the transpose reads (see v_row_of_key): the 64 keys of scale block n start
  // 8448 n bytes in; the four 8-key pieces of a lane half at keys +0, +8, +32, +40 lie 0, 256,
  // 4224 and 4480 bytes from the first.  The matrix-phase assembly writes these offsets as
  // literals; the asserts below tie them to the placement.
  static constexpr int kVHalf = 8448, kVPc8 = 256, kVPc32 = 4224, kVPc40 = 4480;
  static_assert(v_row_offset(v_row_of_key(64)) == kVHalf && v_row_offset(v_row_of_key(8)) == kVPc8 &&
                    v_row_offset(v_row_of_key(32)) == kVPc32 && v_row_offset(v_row_of_key(40)) == kVPc40 &&
                    v_row_offset(v_row_of_key(0)) == 0,
                "transpose-read offsets of the matrix-phase assembly do not match the V placement");
  static constexpr int kVBase = 2 * kKSlot;
  static constexpr int kBytes = 2 * kKSlot + 3 * kVSlot;
  static constexpr int kRounds = ((kKCells > kVCells ? kKCells : kVCells) + 255) / 256;  // DMA rounds, 256 threads
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

// O staging for the epilogue: a 32-row area per wave with a 272-byte row pitch, so the
// 16-byte pieces that 16 consecutive rows write at one column fall on distinct banks
constexpr int kStgPitch = 272;
constexpr int kStgWave = kWaveRows * kStgPitch;
static_assert(kThreads / 64 * kStgWave <= Fp8Lds<128>::kBytes, "O staging exceeds the LDS of the kernel");

template <int DQK, bool EXACT_P, bool DEBUG, bool VT>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(Fp8Args a) {
  using L = Fp8Lds<DQK, VT>;
  constexpr int KC = DQK / 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  const int S = a.S, H = a.H;
  // head-pair mode: a tile is 128 rows of each of the heads h (waves 0-3) and h+1 (waves 4-7)
  const bool pair = a.pair_heads != 0;
  const Schedule sch = make_schedule(a.B, H, S, pair);
  const int hstep = pair ? 2 : 1;
  const int trows = pair ? kPairTileRows : kTileRows;
  const int wrow = pair ? (wave & 3) : wave;  // the wave's 32-row slot in the tile
  const ItemRange work = xcd_items(blockIdx.x, gridDim.x, sch.items);

  // key row stride in bytes; value row stride (key-major V) or channel row stride (VT)
  const int krs = a.mk.ss, vrs = a.mv.ss;

  // per-lane LDS read bases
  const int k_rd = l32 * L::kKStride + 32 * hh;
  // V^T operand by transpose reads: within each 16-lane group, source lane s points at key
  // (piece base) + s/2, bytes d0 + 8 (s%2) .. +7 with d0 = 32 dt + 16 ((lane/16) % 2); the
  // reading lane then holds d = 32 dt + lane%32 for 8 consecutive keys.  The four pieces of
  // a 64-key block n are keys 64n + 16 hh + {0, 8, 32, 40} + 0..7 (Sec. IV-A layout of P).
  // source lane s of a 16-lane group reads key 16hh + s/2 (+ the piece and block offsets), in
  // row v_row_of_key(16hh + s/2), bytes 16 ((lane/16) % 2) + 8 (s%2) of column group dt
  // channel-major V: lane l32 of lane half hh reads channel row 32 dt + l32 at byte 32 hh of the
  // 64-key scale block (two 16-byte reads per operand)
  const int vt_rd = L::kVBase + l32 * (16 * L::kVtSpr) + 32 * hh;
  const int v_tr = L::kVBase + v_row_offset(v_row_of_key(16 * hh + ((lane & 15) >> 1))) + 16 * ((lane >> 4) & 1) +
                   8 * (lane & 1);

  // DMA assignments: the 256 threads of group 0 copy K blocks, those of group 1 V blocks.
  // Round p, thread st covers cell 256p + st of the slot; st_goff is its source offset
  // from the block's first key (pad cells copy column 0 of their row).  Waves whose cells
  // of a round lie past the end of the slot skip that round (a wave-uniform test).
  constexpr int NR = L::kRounds;
  const int st = tid & 255;
  const bool stage_k = (grp == 0);
  const int wq = wave & 3;  // wave index within its group
  const int st_cells = stage_k ? L::kKCells : L::kVCells;
  uint32_t st_goff[NR];
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    const int cell = 256 * p + st;
    if (stage_k) {
      const int row = (cell / L::kKSpr) & 127, col = cell % L::kKSpr;
      st_goff[p] = ((row & ~31) | key_perm_fp8(row & 31)) * krs + 16 * (col < L::kKCols ? col : 0);
    } else if constexpr (VT) {  // pad cells copy the row's first 16 bytes
      const int row = (cell / L::kVtSpr) & 127, col = cell % L::kVtSpr;
      st_goff[p] = row * vrs + 16 * (col < 8 ? vt_cell_src(col) : 0);
    } else {  // pad and spare cells copy the block's first 16 bytes
      const int g = cell / L::kVGroupCells, w = cell % L::kVGroupCells;
      const bool data = g < 32 && w < 32;
      st_goff[p] = data ? v_key_of_row(4 * g + w / 8) * vrs + 16 * (w % 8) : 0;
    }
  }
  const int st_lds = 16 * 64 * wq + (stage_k ? 0 : L::kVBase);
  // copy rounds of this wave: those of its 64-cell shares 256 p + 64 wq inside the slot
  const uint32_t nrounds = (uint32_t)(st_cells - 64 * wq + 255) >> 8;

  // row-sum selector (Sec. IV-B3): lane L of the 16x16x128 A operand is all ones
  // iff (L/16)%2 == ((L%16)/4)%2, so every lane receives the sum of its own query.
  const int sel_on = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1));
  const int selw = sel_on ? 0x38383838 : 0;
  const v8i selv = {selw, selw, selw, selw, selw, selw, selw, selw};
  const v16f zero16 = {};

  const float cp = a.cp;
  const float cp8 = 8.0f * cp;

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
  // Q rows of a tile into the MFMA operand registers: the first tile's here, every later one's
  // at the start of the epilogue before it, so the load overlaps that epilogue
  v8i qop[KC];
  auto load_q = [&](int b_, int h_, int tile_) {
    const uint8_t* qh = a.q + b_ * a.mq.sb + (h_ + (pair ? grp : 0)) * a.mq.sh;
    const int ln = lane_now();
    const uint8_t* qp = qh + (int64_t)(tile_ * trows + wrow * kWaveRows + (ln & 31)) * a.mq.ss + 32 * (ln >> 5);
#pragma unroll
    for (int c = 0; c < KC; ++c) qop[c] = *(const v8i*)(qp + 64 * c);
  };
  // item indices fit in 32 bits (B H S is below 2^31 / d_qk); a 32-bit loop bound stays scalar
  const int wfirst = (int)work.first, wend = (int)work.end;
  if (wfirst < wend) load_q(b, h, sch.T - 1 - j);
  for (int item = wfirst; item < wend; item += work.step) {
    const int hw = h + (pair ? grp : 0);  // the wave's query head
    const uint8_t* st_head = stage_k ? a.k + b * a.mk.sb + hk * a.mk.sh : a.v + b * a.mv.sb + hk * a.mv.sh;
    // bytes from one 128-key block to the next in the staged tensor
    const int64_t st_bstep = stage_k || !VT ? (int64_t)kBlockKeys * (stage_k ? krs : vrs) : kBlockKeys;

    for (int pass = 0; pass < 2; ++pass) {
      // the long tile of the pair first: the workgroups of one XCD then start on key block 0
      // together and read the same K/V blocks from its L2 for most of that tile
      const int tile = pass == 0 ? sch.T - 1 - j : j;
      if (pass == 1 && tile == sch.T - 1 - j) break;
      const int row0 = tile * trows + wrow * kWaveRows;  // first query row of this wave
      const int qrow = row0 + l32;
      const int nb = pair ? tile + 1 : 2 * tile + 2;       // 128-key blocks

      // DMA of block blk: K by group 0 into slot blk % 2, V by group 1 into slot blk % 3
      auto stage = [&](int blk) {
        const uint64_t gs = (uint64_t)(uintptr_t)(st_head + blk * st_bstep);  // wave-uniform
        const uint32_t mb = __builtin_amdgcn_readfirstlane(
            lds_addr(smem) + st_lds + (stage_k ? (blk & 1) * L::kKSlot : (blk % 3) * L::kVSlot));
#pragma unroll
        for (int p = 0; p < NR; ++p)
          if (256 * p + 64 * wq < st_cells) copy_round(gs, mb + 4096 * p, st_goff[p]);
      };

      // ---------------------------------------------------------------- per-wave state
      v16f oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = zero16;
      v16f sacc[4];  // scores of the next block
      v8i pb[2];     // codes of the current block, per 64-key scale block
      float m = 0.f, l = 0.f;
      int o_cur[2] = {0, 0}, o_nxt[2] = {0, 0};

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
      // The matrix phase, as one block of hand-ordered instructions that every step of every
      // wave runs: the row sums of P(i), S^T(i+1) = K Q^T (8 MFMAs at d_qk = 128, 12 at 192),
      // O^T += V^T(i) P^T(i) (8 MFMAs), and between the PV MFMAs the maxima of the two
      // 64-key blocks of S(i+1) (the paper's MFMA wave computes them too, Sec. IV-C; the softmax
      // phase then only takes the lazy decision, o and the codes), then the wave's copies of
      // block i+2.  The first K operand read goes out before the row-sum MFMAs, each later
      // operand read two MFMAs ahead of its MFMA, the first two V^T operands during the last two
      // QK^T MFMAs; every read is waited for inside the block.  A V^T operand is four
      // transpose reads from key-major V, or two 16-byte reads from channel-major V (the
      // assembler's .if on the vt operand picks one).  K and V^T operands pass through
      // two fixed 8-register groups (v240-v255), the 0/1 row-sum selector is an input that stays
      // in registers across the loop, and the scores sit in v176-v239 so that the maxima can
      // name them.  Copies go through a scalar base and the per-lane 32-bit offsets, with M0
      // saved and restored.  Wait states: five at the top, before the first copy may read the
      // scalar base (a compiler reload of it may come just before the block) and before the
      // row-sum MFMAs read the selector and the codes, two after the permlane operands are
      // written, one after each M0 write; the instructions after the last PV MFMA cover the 20
      // that a VALU read of its results needs.
      // the assembly below writes the LDS strides as literal offsets: 32 K rows (one sub-tile)
      // are 4608 bytes at d_qk = 128 and 6656 at 192, 32 channel rows of channel-major V 4608
      static_assert(32 * L::kKStride == (DQK == 128 ? 4608 : 6656), "K sub-tile stride of the matrix-phase assembly");
      static_assert(32 * 16 * L::kVtSpr == 4608, "channel-row stride of the matrix-phase assembly");
      float bmx[2] = {0.f, 0.f};  // block maxima of the next block from the hand-ordered matrix phase
      float bm[2];
      auto mphase_asm = [&](int i) -> v2f {
        const uint32_t kb = lds_addr(smem) + ((i + 1) & 1) * L::kKSlot + k_rd;
        const uint32_t vb = lds_addr(smem) + (i % 3) * L::kVSlot + (VT ? vt_rd : v_tr);
        const int sc0 = 127 - o_cur[0], sc1 = 127 - o_cur[1], one = 127;
        // in a tile's last two steps there is no block i+2: the wave then copies the tile's last
        // block again into the slot the schedule frees (no wave reads it before it is written
        // again), so every step runs the same instructions; the copies are waited for as usual
        const int blk = i + 2 < nb ? i + 2 : nb - 1;
        const uint8_t* src = st_head + blk * st_bstep;
        const uint32_t mb = __builtin_amdgcn_readfirstlane(
            lds_addr(smem) + st_lds + (stage_k ? ((i + 2) & 1) * L::kKSlot : ((i + 2) % 3) * L::kVSlot));
        const uint64_t gs = (uint64_t)(uintptr_t)src;  // wave-uniform: scalar base of the copies
        int m0s;
        float xt0, xt1;
        v4f b0, b1;
        v8i g0, g1;  // the operand groups, clobbered
        if constexpr (DQK == 128) {
        asm volatile(
            // wait states before the first copy's scalar base (a compiler reload of it may precede)
            "s_nop 4\n\t"
            "s_mov_b32 %[m0s], m0\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            // row sums of P(i) against the 0/1 selector; the first K operand read in group 0
            "ds_read_b128 v[240:243], %[kb]\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:16\n\t"
            "v_mfma_scale_f32_16x16x128_f8f6f4 %[b0], %[sel], %[p0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "v_mfma_scale_f32_16x16x128_f8f6f4 %[b1], %[sel], %[p1], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            // S^T(i+1) = K Q^T: sub-tile u, 64-wide chunk c, chunk-outer; each operand read two MFMAs ahead
            "ds_read_b128 v[248:251], %[kb] offset:4608\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:4624\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[176:191], v[240:247], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:9216\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:9232\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[192:207], v[248:255], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:13824\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:13840\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[208:223], v[240:247], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:64\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:80\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[224:239], v[248:255], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:4672\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:4688\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[176:191], v[240:247], %[q1], v[176:191], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:9280\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:9296\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[192:207], v[248:255], %[q1], v[192:207], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:13888\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:13904\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[208:223], v[240:247], %[q1], v[208:223], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            // the first two V^T operands of PV(i), four transpose reads each
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb]\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:16\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb]\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:256\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:4224\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:4480\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[224:239], v[248:255], %[q1], v[224:239], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:4608\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:4624\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:32\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:288\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:4256\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:4512\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            // O^T += V^T(i) P^T(i) with the 2^-o scale of each 64-key block; between these MFMAs the maxima
            // of the two 64-key blocks of S(i+1), each a v_max3 chain over a lane's 32 scores of the block
            // (the scores were written five or more MFMAs earlier)
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o0], v[240:247], %[p0], %[o0], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:9216\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:9232\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:64\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:320\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:4288\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:4544\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o1], v[248:255], %[p0], %[o1], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:13824\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:13840\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:96\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:352\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:4320\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:4576\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], v176, v177, v178\n\t"
            "v_max3_f32 %[t0], %[t0], v179, v180\n\t"
            "v_max3_f32 %[t0], %[t0], v181, v182\n\t"
            "v_max3_f32 %[t0], %[t0], v183, v184\n\t"
            "v_max3_f32 %[t0], %[t0], v185, v186\n\t"
            "v_max3_f32 %[t0], %[t0], v187, v188\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o2], v[240:247], %[p0], %[o2], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:64\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:80\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:8448\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:8704\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:12672\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:12928\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], %[t0], v189, v190\n\t"
            "v_max3_f32 %[t0], %[t0], v191, v192\n\t"
            "v_max3_f32 %[t0], %[t0], v193, v194\n\t"
            "v_max3_f32 %[t0], %[t0], v195, v196\n\t"
            "v_max3_f32 %[t0], %[t0], v197, v198\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o3], v[248:255], %[p0], %[o3], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:4672\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:4688\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:8480\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:8736\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:12704\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:12960\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], %[t0], v199, v200\n\t"
            "v_max3_f32 %[t0], %[t0], v201, v202\n\t"
            "v_max3_f32 %[t0], %[t0], v203, v204\n\t"
            "v_max3_f32 %[t0], %[t0], v205, v206\n\t"
            "v_max_f32 %[t0], %[t0], v207\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o0], v[240:247], %[p1], %[o0], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:9280\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:9296\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:8512\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:8768\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:12736\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:12992\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t1], v208, v209, v210\n\t"
            "v_max3_f32 %[t1], %[t1], v211, v212\n\t"
            "v_max3_f32 %[t1], %[t1], v213, v214\n\t"
            "v_max3_f32 %[t1], %[t1], v215, v216\n\t"
            "v_max3_f32 %[t1], %[t1], v217, v218\n\t"
            "v_max3_f32 %[t1], %[t1], v219, v220\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o1], v[248:255], %[p1], %[o1], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:13888\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:13904\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:8544\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:8800\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:12768\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:13024\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t1], %[t1], v221, v222\n\t"
            "v_max3_f32 %[t1], %[t1], v223, v224\n\t"
            "v_max3_f32 %[t1], %[t1], v225, v226\n\t"
            "v_max3_f32 %[t1], %[t1], v227, v228\n\t"
            "v_max3_f32 %[t1], %[t1], v229, v230\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o2], v[240:247], %[p1], %[o2], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            "v_max3_f32 %[t1], %[t1], v231, v232\n\t"
            "v_max3_f32 %[t1], %[t1], v233, v234\n\t"
            "v_max3_f32 %[t1], %[t1], v235, v236\n\t"
            "v_max3_f32 %[t1], %[t1], v237, v238\n\t"
            "v_max_f32 %[t1], %[t1], v239\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o3], v[248:255], %[p1], %[o3], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            // the two lanes of a query hold keys 16 hh + r: combine them, then scale to base-2 units
            "v_mov_b32 %[x0], %[t0]\n\t"
            "v_mov_b32 %[x1], %[t1]\n\t"
            "s_nop 1\n\t"
            "v_permlane32_swap_b32 %[t0], %[x0]\n\t"
            "v_permlane32_swap_b32 %[t1], %[x1]\n\t"
            "s_nop 1\n\t"
            "v_max_f32 %[t0], %[t0], %[x0]\n\t"
            "v_mul_f32 %[t0], %[cp], %[t0]\n\t"
            "v_max_f32 %[t1], %[t1], %[x1]\n\t"
            "v_mul_f32 %[t1], %[cp], %[t1]\n\t"
            // the wave's copies of block i+2: four 64-cell rounds, and up to 1 more for the waves
            // whose slot share has them (%[nr] rounds in all); these instructions also cover the wait
            // states a VALU read of the last PV results needs
            "s_mov_b32 m0, %[mb]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a0], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 4096\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a1], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 8192\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a2], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 12288\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a3], %[gs]\n\t"
            "s_cmp_le_u32 %[nr], 4\n\t"
            "s_cbranch_scc1 1f\n\t"
            "s_add_u32 m0, %[mb], 16384\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a4], %[gs]\n\t"
            "1:\n\t"
            "s_mov_b32 m0, %[m0s]\n\t"
            : "=&{v[176:191]}"(sacc[0]), "=&{v[192:207]}"(sacc[1]), "=&{v[208:223]}"(sacc[2]),
              "=&{v[224:239]}"(sacc[3]), [t0] "=&v"(bmx[0]), [t1] "=&v"(bmx[1]), [x0] "=&v"(xt0), [x1] "=&v"(xt1),
              [o0] "+v"(oacc[0]), [o1] "+v"(oacc[1]), [o2] "+v"(oacc[2]), [o3] "+v"(oacc[3]),
              [b0] "=&v"(b0), [b1] "=&v"(b1), "=&{v[240:247]}"(g0), "=&{v[248:255]}"(g1), [m0s] "=&s"(m0s)
            : [kb] "v"(kb), [vb] "v"(vb), [q0] "v"(qop[0]), [q1] "v"(qop[1]), [p0] "v"(pb[0]), [p1] "v"(pb[1]),
              [sel] "v"(selv), [one] "v"(one), [c0] "v"(sc0), [c1] "v"(sc1), [mb] "s"(mb), [gs] "s"(gs),
              [a0] "v"(st_goff[0]), [a1] "v"(st_goff[1]), [a2] "v"(st_goff[2]), [a3] "v"(st_goff[3]),
              [a4] "v"(st_goff[4]), [nr] "s"(nrounds), [cp] "s"(cp), [vt] "n"(VT ? 1 : 0)
            : "memory", "scc");
        } else {
        asm volatile(
            // wait states before the first copy's scalar base (a compiler reload of it may precede)
            "s_nop 4\n\t"
            "s_mov_b32 %[m0s], m0\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            // row sums of P(i) against the 0/1 selector; the first K operand read in group 0
            "ds_read_b128 v[240:243], %[kb]\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:16\n\t"
            "v_mfma_scale_f32_16x16x128_f8f6f4 %[b0], %[sel], %[p0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "v_mfma_scale_f32_16x16x128_f8f6f4 %[b1], %[sel], %[p1], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            // S^T(i+1) = K Q^T: sub-tile u, 64-wide chunk c, chunk-outer; each operand read two MFMAs ahead
            "ds_read_b128 v[248:251], %[kb] offset:6656\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:6672\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[176:191], v[240:247], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:13312\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:13328\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[192:207], v[248:255], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:19968\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:19984\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[208:223], v[240:247], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:64\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:80\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[224:239], v[248:255], %[q0], 0, %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:6720\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:6736\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[176:191], v[240:247], %[q1], v[176:191], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:13376\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:13392\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[192:207], v[248:255], %[q1], v[192:207], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:20032\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:20048\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[208:223], v[240:247], %[q1], v[208:223], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:128\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:144\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[224:239], v[248:255], %[q1], v[224:239], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:6784\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:6800\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[176:191], v[240:247], %[q2], v[176:191], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[240:243], %[kb] offset:13440\n\t"
            "ds_read_b128 v[244:247], %[kb] offset:13456\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[192:207], v[248:255], %[q2], v[192:207], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            "ds_read_b128 v[248:251], %[kb] offset:20096\n\t"
            "ds_read_b128 v[252:255], %[kb] offset:20112\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[208:223], v[240:247], %[q2], v[208:223], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            // the first two V^T operands of PV(i), four transpose reads each
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb]\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:16\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb]\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:256\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:4224\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:4480\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 v[224:239], v[248:255], %[q2], v[224:239], %[one], %[one] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:4608\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:4624\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:32\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:288\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:4256\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:4512\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            // O^T += V^T(i) P^T(i) with the 2^-o scale of each 64-key block; between these MFMAs the maxima
            // of the two 64-key blocks of S(i+1), each a v_max3 chain over a lane's 32 scores of the block
            // (the scores were written five or more MFMAs earlier)
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o0], v[240:247], %[p0], %[o0], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:9216\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:9232\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:64\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:320\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:4288\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:4544\n\t"
            ".endif\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o1], v[248:255], %[p0], %[o1], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:13824\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:13840\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:96\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:352\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:4320\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:4576\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], v176, v177, v178\n\t"
            "v_max3_f32 %[t0], %[t0], v179, v180\n\t"
            "v_max3_f32 %[t0], %[t0], v181, v182\n\t"
            "v_max3_f32 %[t0], %[t0], v183, v184\n\t"
            "v_max3_f32 %[t0], %[t0], v185, v186\n\t"
            "v_max3_f32 %[t0], %[t0], v187, v188\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o2], v[240:247], %[p0], %[o2], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:64\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:80\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:8448\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:8704\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:12672\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:12928\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], %[t0], v189, v190\n\t"
            "v_max3_f32 %[t0], %[t0], v191, v192\n\t"
            "v_max3_f32 %[t0], %[t0], v193, v194\n\t"
            "v_max3_f32 %[t0], %[t0], v195, v196\n\t"
            "v_max3_f32 %[t0], %[t0], v197, v198\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o3], v[248:255], %[p0], %[o3], %[one], %[c0] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:4672\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:4688\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:8480\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:8736\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:12704\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:12960\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t0], %[t0], v199, v200\n\t"
            "v_max3_f32 %[t0], %[t0], v201, v202\n\t"
            "v_max3_f32 %[t0], %[t0], v203, v204\n\t"
            "v_max3_f32 %[t0], %[t0], v205, v206\n\t"
            "v_max_f32 %[t0], %[t0], v207\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o0], v[240:247], %[p1], %[o0], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[240:243], %[vb] offset:9280\n\t"
            "ds_read_b128 v[244:247], %[vb] offset:9296\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[240:241], %[vb] offset:8512\n\t"
            "ds_read_b64_tr_b8 v[242:243], %[vb] offset:8768\n\t"
            "ds_read_b64_tr_b8 v[244:245], %[vb] offset:12736\n\t"
            "ds_read_b64_tr_b8 v[246:247], %[vb] offset:12992\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t1], v208, v209, v210\n\t"
            "v_max3_f32 %[t1], %[t1], v211, v212\n\t"
            "v_max3_f32 %[t1], %[t1], v213, v214\n\t"
            "v_max3_f32 %[t1], %[t1], v215, v216\n\t"
            "v_max3_f32 %[t1], %[t1], v217, v218\n\t"
            "v_max3_f32 %[t1], %[t1], v219, v220\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o1], v[248:255], %[p1], %[o1], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            ".if %[vt]\n\t"
            "ds_read_b128 v[248:251], %[vb] offset:13888\n\t"
            "ds_read_b128 v[252:255], %[vb] offset:13904\n\t"
            ".else\n\t"
            "ds_read_b64_tr_b8 v[248:249], %[vb] offset:8544\n\t"
            "ds_read_b64_tr_b8 v[250:251], %[vb] offset:8800\n\t"
            "ds_read_b64_tr_b8 v[252:253], %[vb] offset:12768\n\t"
            "ds_read_b64_tr_b8 v[254:255], %[vb] offset:13024\n\t"
            ".endif\n\t"
            "v_max3_f32 %[t1], %[t1], v221, v222\n\t"
            "v_max3_f32 %[t1], %[t1], v223, v224\n\t"
            "v_max3_f32 %[t1], %[t1], v225, v226\n\t"
            "v_max3_f32 %[t1], %[t1], v227, v228\n\t"
            "v_max3_f32 %[t1], %[t1], v229, v230\n\t"
            ".if %[vt]\n\t"
            "s_waitcnt lgkmcnt(2)\n\t"
            ".else\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            ".endif\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o2], v[240:247], %[p1], %[o2], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            "v_max3_f32 %[t1], %[t1], v231, v232\n\t"
            "v_max3_f32 %[t1], %[t1], v233, v234\n\t"
            "v_max3_f32 %[t1], %[t1], v235, v236\n\t"
            "v_max3_f32 %[t1], %[t1], v237, v238\n\t"
            "v_max_f32 %[t1], %[t1], v239\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            "v_mfma_scale_f32_32x32x64_f8f6f4 %[o3], v[248:255], %[p1], %[o3], %[one], %[c1] op_sel_hi:[0,0,0]\n\t"
            // the two lanes of a query hold keys 16 hh + r: combine them, then scale to base-2 units
            "v_mov_b32 %[x0], %[t0]\n\t"
            "v_mov_b32 %[x1], %[t1]\n\t"
            "s_nop 1\n\t"
            "v_permlane32_swap_b32 %[t0], %[x0]\n\t"
            "v_permlane32_swap_b32 %[t1], %[x1]\n\t"
            "s_nop 1\n\t"
            "v_max_f32 %[t0], %[t0], %[x0]\n\t"
            "v_mul_f32 %[t0], %[cp], %[t0]\n\t"
            "v_max_f32 %[t1], %[t1], %[x1]\n\t"
            "v_mul_f32 %[t1], %[cp], %[t1]\n\t"
            // the wave's copies of block i+2: four 64-cell rounds, and up to 3 more for the waves
            // whose slot share has them (%[nr] rounds in all); these instructions also cover the wait
            // states a VALU read of the last PV results needs
            "s_mov_b32 m0, %[mb]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a0], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 4096\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a1], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 8192\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a2], %[gs]\n\t"
            "s_add_u32 m0, %[mb], 12288\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a3], %[gs]\n\t"
            "s_cmp_le_u32 %[nr], 4\n\t"
            "s_cbranch_scc1 1f\n\t"
            "s_add_u32 m0, %[mb], 16384\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a4], %[gs]\n\t"
            "1:\n\t"
            "s_cmp_le_u32 %[nr], 5\n\t"
            "s_cbranch_scc1 1f\n\t"
            "s_add_u32 m0, %[mb], 20480\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a5], %[gs]\n\t"
            "1:\n\t"
            "s_cmp_le_u32 %[nr], 6\n\t"
            "s_cbranch_scc1 1f\n\t"
            "s_add_u32 m0, %[mb], 24576\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[a6], %[gs]\n\t"
            "1:\n\t"
            "s_mov_b32 m0, %[m0s]\n\t"
            : "=&{v[176:191]}"(sacc[0]), "=&{v[192:207]}"(sacc[1]), "=&{v[208:223]}"(sacc[2]),
              "=&{v[224:239]}"(sacc[3]), [t0] "=&v"(bmx[0]), [t1] "=&v"(bmx[1]), [x0] "=&v"(xt0), [x1] "=&v"(xt1),
              [o0] "+v"(oacc[0]), [o1] "+v"(oacc[1]), [o2] "+v"(oacc[2]), [o3] "+v"(oacc[3]),
              [b0] "=&v"(b0), [b1] "=&v"(b1), "=&{v[240:247]}"(g0), "=&{v[248:255]}"(g1), [m0s] "=&s"(m0s)
            : [kb] "v"(kb), [vb] "v"(vb), [q0] "v"(qop[0]), [q1] "v"(qop[1]), [q2] "v"(qop[KC - 1]),
              [p0] "v"(pb[0]), [p1] "v"(pb[1]), [sel] "v"(selv), [one] "v"(one), [c0] "v"(sc0), [c1] "v"(sc1),
              [mb] "s"(mb), [gs] "s"(gs), [a0] "v"(st_goff[0]), [a1] "v"(st_goff[1]), [a2] "v"(st_goff[2]),
              [a3] "v"(st_goff[3]), [a4] "v"(st_goff[4]), [a5] "v"(st_goff[NR > 5 ? 5 : 4]),
              [a6] "v"(st_goff[NR > 6 ? 6 : 4]), [nr] "s"(nrounds), [cp] "s"(cp), [vt] "n"(VT ? 1 : 0)
            : "memory", "scc");
        }
        (void)g0;
        (void)g1;
        (void)xt0;
        (void)xt1;
        return (v2f){b0[0], b1[0]};
      };
      // causal mask, block maxima (v_max3 tree), running max with the lazy decision (the
      // rare rescale of O and l happens here, in the softmax phase), exponents o for blk
      auto dump_scores = [&](int blk) {
        const int key0 = blk * kBlockKeys;
        if constexpr (DEBUG) {  // raw scores as the MFMA left them, before the mask
          if (a.dbg_scores != nullptr) {
            float* srow = a.dbg_scores + ((int64_t)(b * H + hw) * S + qrow) * S + key0 + 16 * hh;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int r = 0; r < 16; r += 4)
                *(v4f*)(srow + 32 * u + r) = (v4f){sacc[u][r], sacc[u][r + 1], sacc[u][r + 2], sacc[u][r + 3]};
          }
        }
      };
      auto block_max = [&](int blk) {
        const int key0 = blk * kBlockKeys;
        if (key0 + kBlockKeys - 1 > row0) {  // diagonal block: key key0+32u+16hh+r
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (key0 + 32 * u + 16 * hh + r > qrow) sacc[u][r] = -INFINITY;
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float x[11];
#pragma unroll
          for (int k = 0; k < 5; ++k) x[k] = fmax3(sacc[2 * n][3 * k], sacc[2 * n][3 * k + 1], sacc[2 * n][3 * k + 2]);
          x[5] = fmax3(sacc[2 * n][15], sacc[2 * n + 1][0], sacc[2 * n + 1][1]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            x[6 + k] = fmax3(sacc[2 * n + 1][2 + 3 * k], sacc[2 * n + 1][3 + 3 * k], sacc[2 * n + 1][4 + 3 * k]);
          x[10] = max2(sacc[2 * n + 1][14], sacc[2 * n + 1][15]);
          const float y = fmax3(fmax3(x[0], x[1], x[2]), fmax3(x[3], x[4], x[5]),
                                fmax3(fmax3(x[6], x[7], x[8]), x[9], x[10]));
          const uint32_t yu = __float_as_uint(y);
          const auto sw = __builtin_amdgcn_permlane32_swap(yu, yu, false, false);
          const float ya = __uint_as_float(sw[0]), yb = __uint_as_float(sw[1]);
          bm[n] = max2(ya, yb) * cp;
        }
      };
      auto decide = [&](bool first) {
        if (first) {
          m = fmaxf(bm[0], bm[1]);
        } else {
          const float M = fmax3(m, bm[0], bm[1]);
          if (__any((M - m) >= kTauFp8)) {
            const float f = __builtin_amdgcn_exp2f(m - M);
            m = M;
            l *= f;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) oacc[dt] *= f;
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
          uint8_t* orow = a.dbg_o + ((int64_t)(b * H + hw) * S + qrow) * (S / 64);
          uint8_t* crow = a.dbg_codes + ((int64_t)(b * H + hw) * S + qrow) * S;
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

      // ---------------------------------------------------------------- prologue
      // K(0), K(1) by group 0 and V(0), V(1) by group 1.  Only the Q rows and block 0 are
      // waited for here: block 1 streams in under the first two phases and each wave waits
      // for its share at the end of its S_pro (K(1) is first read in M_0, V(1) in M_1), so a
      // tile starts after one block's copies instead of two.  Tile 0 of the head-pair mode
      // has one block; its block 1 (keys 128-255, present since S >= 256) is copied unused.
      stage(0);
      wait_dma();
      lds_barrier();
      stage(1);
      if (grp == 1) lds_barrier();  // group 1 runs one phase behind

      // M_pro
      if (live(0)) qk(0);
      lds_barrier();
      // S_pro
      if (live(0)) {
        dump_scores(0);
        block_max(0);
        decide(true);
        codes(0);
      }
      wait_dma();
      lds_barrier();

      for (int i = 0; i < nb; ++i) {
        // -------------------------------------------------------------- M_i
        __builtin_amdgcn_s_setprio(1);
        const bool live_n = (i + 1 < nb) && live(i + 1);
        // every wave runs the whole stream: a block the causal mask hides from all rows of the
        // wave has zero codes (set in the softmax phase), so its PV and row sums add 0, and the
        // scores of a dead or missing next block (its K slot holds an earlier block, in bounds)
        // are never read
        {
          const v2f bsum = mphase_asm(i);
          l = fmaf(bsum[1], __int_as_float((127 - o_cur[1]) << 23), fmaf(bsum[0], __int_as_float((127 - o_cur[0]) << 23), l));
        }
        lds_barrier();
        // -------------------------------------------------------------- S_i
        __builtin_amdgcn_s_setprio(0);
        if (live_n) {
          dump_scores(i + 1);
          if ((i + 1) * kBlockKeys + kBlockKeys - 1 <= row0) {
            // below the diagonal for every row of the wave: the matrix phase took the maxima
            bm[0] = bmx[0];
            bm[1] = bmx[1];
          } else {
            block_max(i + 1);
          }
          decide(false);
          codes(i + 1);
        } else {
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            pb[n] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
            o_cur[n] = 0;
          }
        }
        wait_dma();
        lds_barrier();
      }
      if (grp == 0) lds_barrier();

      // ---------------------------------------------------------------- epilogue
      // O goes through LDS so that the stores are whole rows: each wave writes its 32 rows
      // of bf16 O into a staging area of its own, then 16 lanes store each 256-byte row.
      // Every operand read of the tile completed at the last barrier; the barrier after the
      // stores keeps the next tile's copies out of LDS until every wave has read its area.
      if (pass == 0 && j != sch.T - 1 - j) {
        load_q(b, h, j);
      } else if (item + work.step < wend) {
        int b1 = b, h1 = h, hk1 = hk, hg1 = hg, j1 = j;
        next_item(b1, h1, hk1, hg1, j1);
        load_q(b1, h1, sch.T - 1 - j1);
      }
      const float inv = a.v_descale / l;
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
      if (a.lse != nullptr && hh == 0)
        a.lse[(int64_t)(b * H + hw) * S + qrow] = kLn2 * (m + __log2f(l) - (float)kSigma);
      lds_barrier();
    }
    // the workgroup's next item, work.step items on
    if (item + work.step >= wend) break;
    next_item(b, h, hk, hg, j);
  }
}

}  // namespace

template <bool VT>
void launch_fp8_layout(const Fp8Args& a, int dqk, bool exact_p, dim3 g, dim3 t, hipStream_t stream) {
  if (dqk == 128) {
    if (exact_p)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true, false, VT>), g, t, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false, false, VT>), g, t, 0, stream, a);
  } else {
    if (exact_p)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, true, false, VT>), g, t, 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, false, false, VT>), g, t, 0, stream, a);
  }
}

hipError_t launch_fp8(const Fp8Args& a, int dqk, bool exact_p, bool debug, bool v_channel_major, int grid,
                      hipStream_t stream) {
  const dim3 g(grid), t(kThreads);
  if (debug) {  // the test hooks: either P mode at either head dimension, key-major V
    if (dqk == 128) {
      if (exact_p)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true, true, false>), g, t, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false, true, false>), g, t, 0, stream, a);
    } else {
      if (exact_p)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, true, true, false>), g, t, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<192, false, true, false>), g, t, 0, stream, a);
    }
  } else if (v_channel_major) {
    launch_fp8_layout<true>(a, dqk, exact_p, g, t, stream);
  } else {
    launch_fp8_layout<false>(a, dqk, exact_p, g, t, stream);
  }
  return hipGetLastError();
}

}  // namespace cfa
