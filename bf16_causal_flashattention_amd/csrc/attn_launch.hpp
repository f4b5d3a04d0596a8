// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfa {

// Byte strides of one attention tensor: element (b, s, h, d) of it sits at
// base + b * sb + h * sh + s * ss + d * (element size); the head dimension is contiguous.
struct TensorMap {
  int64_t sb;  // batch stride
  int64_t sh;  // head stride
  int ss;      // sequence (row) stride; 128 rows of it fit in 31 bits
};

struct Fp8Args {
  const uint8_t* q;  // e4m3 codes, [B][S][H][d_qk] through mq
  const uint8_t* k;  // e4m3 codes, [B][S][H_kv][d_qk] through mk
  const uint8_t* v;  // e4m3 codes, [B][S][H_kv][128] through mv; channel-major V: [B][H_kv][128][S]
                     // with mv.ss the stride between channel rows (keys contiguous)
  uint16_t* out;     // bf16 bits, [B][S][H][128] through mo
  float* lse;        // [B][H][S] (contiguous) or null
  float cp;          // fp32(softmax_scale * q_descale * k_descale * log2 e)
  float v_descale;
  int B, H, S;
  int G;             // query heads per key/value head (H / H_kv): head h reads key/value head h / G
  int pair_heads;    // 1: head-pair mode (G even), a tile is 128 rows of heads 2u and 2u+1
  TensorMap mq, mk, mv, mo;
  uint8_t* dbg_o;      // debug build only: [B*H*S][S/64] block exponents
  uint8_t* dbg_codes;  // debug build only: [B*H*S][S] probability codes
  float* dbg_scores;   // debug build only, may be null: [B*H*S][S] raw fp32 scores (MFMA sums)
};

struct Bf16Args {
  const uint16_t* q;  // bf16 bits, [B][S][H][d_qk] through mq (d_qk = 128 or 192)
  const uint16_t* k;  // [B][S][H_kv][d_qk] through mk
  const uint16_t* v;  // [B][S][H_kv][128] through mv
  uint16_t* out;      // [B][S][H][128] through mo
  float* lse;
  float cp;  // fp32(softmax_scale * log2 e)
  int B, H, S;
  int G;
  int pair_heads;  // as in Fp8Args
  TensorMap mq, mk, mv, mo;
};

hipError_t launch_fp8(const Fp8Args& a, int dqk, bool exact_p, bool debug, bool v_channel_major, int grid,
                      hipStream_t stream);
hipError_t launch_bf16(const Bf16Args& a, int dqk, int grid, hipStream_t stream);
hipError_t launch_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* ws,
                                hipStream_t stream);
hipError_t launch_round_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t stream);
int64_t key_mean_workspace_bytes(int B, int S, int H, int D);
// size of the file-scope partial-sum array of the allocation-free key mean
constexpr int64_t kKeyMeanScratchBytes = INT64_C(4) << 20;
// the key mean with its partial sums in that array (per device; calls on one GPU must not
// overlap); B * H * ceil(S / 1024) * D * 8 bytes must not exceed kKeyMeanScratchBytes
hipError_t launch_key_mean_noalloc(const float* k, int B, int S, int H, int D, float* mean, hipStream_t stream);
hipError_t launch_key_mean(const float* k, int B, int S, int H, int D, float* mean, void* ws, hipStream_t stream);
// static_scale / is_static: one pass with the given power-of-two scale (saturating at 448)
// instead of the two-pass maximum-derived scale (descale and ws unused then).
hipError_t launch_rotate_quantize(const float* x, const float* mean, const float* signs, int B, int S, int H,
                                  int D, const float c3[9], uint8_t* codes, float* descale, uint32_t* ws,
                                  float static_scale, bool is_static, hipStream_t stream);
hipError_t launch_quantize_e4m3_static(const float* x, int64_t n, float scale, uint8_t* codes, hipStream_t stream);

}  // namespace cfa
