// Shared pieces of the causal attention forward kernels for gfx950 (CDNA4).
//
// Work decomposition, LDS layouts and MFMA operand types.  The method follows
// "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4" (Anthony et al.):
// Sec. II-B (tiled causal attention), Sec. IV-A (workgroup structure, KQ^T
// orientation, causal pairing, persistent grid, chiplet placement).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// A workgroup owns a tile of 256 query rows; each of its 8 waves owns 32 rows
// (two waves per SIMD).  Keys stream through LDS in blocks of 128 (FP8 and BF16 at
// d_qk = 128) or 64 (BF16 at d_qk = 192).  In the head-pair mode (grouped-query
// attention with an even group) a tile is 128 rows of each of two query heads that share
// one key/value head: waves 0-3 take the first head, waves 4-7 the second.
constexpr int kTileRows = 256;
constexpr int kPairTileRows = 128;
constexpr int kWaves = 8;
constexpr int kWaveRows = 32;
constexpr int kThreads = 512;
constexpr int kBlockKeys = 128;
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// Work decomposition (Sec. IV-A, "Causal pairing" and "Chiplet placement").
// Per (b, h) there are T = S / 256 query tiles.  Work item j of a head runs tile
// T-1-j and then tile j, so every item covers T+1 key steps of 256; when T is odd
// the middle tile runs alone.  The long tile comes first, so that the workgroups of an
// XCD, which start together on neighbouring items of one head, read the same K/V blocks
// at about the same time for most of it.  Items are numbered head-major, pairs contiguous:
//   item = (b * H + h) * P + j,  P = ceil(T / 2).
// A persistent grid of G workgroups covers the N items.  The hardware dispatches
// workgroup i to XCD i mod 8; XCD x, with n_x = G/8 + (x < G%8) workgroups, owns the
// contiguous item range [N p_x / G, N (p_x + n_x) / G), where p_x counts the workgroups
// of the XCDs below x, and its w-th workgroup takes items first + w, first + w + n_x, ...
// So the workgroups of one XCD always work on neighbouring items, the tile pairs of one
// or two heads, whose K and V blocks then stream through that XCD's L2 once.  The ranges
// follow the workgroup counts, so no workgroup gets more than ceil(N / G) items.
//
// Head-pair mode (Sec. IV-A: with grouped-query attention and an even group size a pair
// covers two query heads with tiles of half the size).  The heads 2u and 2u+1, which share
// a key/value head, form head pair u; its tiles have 128 rows of each head, T = S / 128,
// and the items are numbered as above with H/2 head pairs in place of H heads.  Every K/V
// block a workgroup stages then feeds 256 query rows of two heads, and a tile has one
// diagonal block instead of two, so a pair takes S/128 + 1 block steps instead of S/128 + 2.
struct Schedule {
  int T;          // tiles per head (per head pair in the head-pair mode)
  int P;          // items per head (per head pair)
  int HS;         // heads (head pairs) the items run over
  int64_t items;  // B * HS * P
};

// pair_heads: the head-pair mode, for H / H_kv even
__host__ __device__ inline Schedule make_schedule(int B, int H, int S, bool pair_heads) {
  Schedule s;
  s.T = S / (pair_heads ? kPairTileRows : kTileRows);
  s.P = (s.T + 1) / 2;
  s.HS = pair_heads ? H / 2 : H;
  s.items = (int64_t)B * s.HS * s.P;
  return s;
}

// the items of workgroup bid of a grid of G: first, first + step, ... below end
struct ItemRange {
  int64_t first, end;
  int step;
};

__host__ __device__ inline ItemRange xcd_items(int bid, int grid, int64_t items) {
  const int per = grid / kXcds, rem = grid % kXcds;
  const int x = bid % kXcds, w = bid / kXcds;
  const int n = per + (x < rem ? 1 : 0);
  const int64_t p0 = (int64_t)x * per + (x < rem ? x : rem);
  ItemRange r;
  const uint64_t a = (uint64_t)items * (uint64_t)p0, b = (uint64_t)items * (uint64_t)(p0 + n);
  if (b < (UINT64_C(1) << 32)) {  // the usual case: 32-bit divisions (a 64-bit one is slow on the GPU)
    r.first = (uint32_t)a / (uint32_t)grid;
    r.end = (uint32_t)b / (uint32_t)grid;
  } else {
    r.first = (int64_t)(a / (uint64_t)grid);
    r.end = (int64_t)(b / (uint64_t)grid);
  }
  r.first += w;
  r.step = n;
  return r;
}

// (b, head or head pair u, j) of an item, for HS heads (head pairs) and P items per head
__host__ __device__ inline void decode_item(int64_t item, int H, int P, int& b, int& h, int& j) {
  const int64_t bh = item / P;
  j = (int)(item - bh * P);
  b = (int)(bh / H);
  h = (int)(bh - (int64_t)b * H);
}

// ---------------------------------------------------------------------------
// Key order inside a 32-key sub-tile.  The score MFMA computes S^T = K Q^T, so
// lane l of a wave holds the scores of query l%32 (Sec. IV-A: max and sum need
// one exchange between the two lanes of a query, the rescale one scalar per
// lane).  Row i of the K operand is loaded from key pi(i) of the sub-tile; with
// that order, lane half hh = l/32 holds keys 16*hh + r (r = 0..15) of each FP8
// sub-tile in accumulator order, which is exactly the byte order the PV MFMA
// needs for the probabilities, and the matching V^T operand is two contiguous
// 16-byte LDS reads.
__host__ __device__ constexpr int key_perm_fp8(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// BF16 (32x32x16 MFMA, 8 keys per lane half): lane half hh holds keys
// 16*(r/8) + 8*hh + r%8.
__host__ __device__ constexpr int key_perm_bf16(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}

// global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane L of
// the wave writes lds_wave_base + 16 L, whatever its source address.  Completion is
// tracked by the issuing wave's vmcnt.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// One 64-cell copy round from global memory into LDS (lane L writes cell base + L), in the form
// the FP8 kernel's hand-ordered matrix phase also uses: a wave-uniform 64-bit base in scalar
// registers plus each lane's 32-bit offset, with M0 = the round's LDS base (saved and
// restored).  With a per-lane 64-bit address (the builtin's form) the compiler keeps one
// address pair per round, spills them, and reloads them with a wait for every load in flight.  Five wait states come first in case the compiler
// has just written a scalar operand from a vector instruction (a spill reload), and one after
// the M0 write.
__device__ __forceinline__ void copy_round(uint64_t gs, uint32_t m, uint32_t off) {
  int t;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %[t], m0\n\t"
      "s_mov_b32 m0, %[m]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o], %[gs]\n\t"
      "s_mov_b32 m0, %[t]"
      : [t] "=&s"(t)
      : [m] "s"(m), [o] "v"(off), [gs] "s"(gs)
      : "memory");
}

// The lane index, read afresh at its point of use.  Per-lane address offsets computed from it
// inside the tile loop then live only there: computed once at the top of the kernel, the
// compiler keeps them (widened to 64 bits) across the whole kernel, spills them, and reloads them
// at every work item with a wait for every memory access in flight.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt at their maxima), issued as the
// builtin so the compiler's own wait insertion knows the counter is drained afterwards
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS transpose reads (gfx950).  Within each 16-lane group of a wave:
//   tr8:  output lane 8a+e receives byte e of the 8 bytes at the addresses of
//         source lanes a, a+2, ..., a+14;
//   tr16: output lane 4a+e receives element e of the 4 bf16 at the addresses of
//         source lanes a, a+4, a+8, a+12.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}
__device__ __forceinline__ v2i lds_tr16(const uint8_t* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p));
}

// byte permute: result byte k = sel byte k indexing {lo bytes 0-3, hi bytes 4-7}
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4x4 byte transpose: r[i] holds bytes (key i; d 0..3) -> s[e] holds (d e; keys 0..3).
__device__ __forceinline__ void transpose4x4_u8(const uint32_t r[4], uint32_t s[4]) {
  const uint32_t t0 = perm(r[1], r[0], 0x05010400u);
  const uint32_t t1 = perm(r[1], r[0], 0x07030602u);
  const uint32_t t2 = perm(r[3], r[2], 0x05010400u);
  const uint32_t t3 = perm(r[3], r[2], 0x07030602u);
  s[0] = perm(t2, t0, 0x05040100u);
  s[1] = perm(t2, t0, 0x07060302u);
  s[2] = perm(t3, t1, 0x05040100u);
  s[3] = perm(t3, t1, 0x07060302u);
}

// value exchange between lane l and lane l^32 (gfx950 v_permlane32_swap).
__device__ __forceinline__ float max_with_partner(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Per-tensor power-of-two e4m3 scale: the largest 2^k with amax * 2^k <= 448 (nothing
// saturates), k clamped to [-126, 126], k = 0 for amax = 0 (Sec. V-E, footnote 17).
__device__ __forceinline__ int pow2_exponent_e4m3(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float f = frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1); 448 = 0.875 2^9
  int k = (f <= 0.875f) ? 9 - e : 8 - e;
  k = k > 126 ? 126 : (k < -126 ? -126 : k);
  return k;
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// two fp32 values to packed bf16 (lo in the low half), rounded to nearest even: the compiler
// lowers the conversion to one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}


}  // namespace cfa
