// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfa {

struct Fp8Args {
  const uint8_t* q;  // e4m3 codes, BSHD [B][S][H][d_qk]
  const uint8_t* k;  // e4m3 codes, BSHD [B][S][H][d_qk]
  const uint8_t* v;  // e4m3 codes, BSHD [B][S][H][128]
  uint16_t* out;     // bf16 bits, BSHD [B][S][H][128]
  float* lse;        // [B][H][S] or null
  float cp;          // fp32(softmax_scale * q_descale * k_descale * log2 e)
  float v_descale;
  int B, H, S;
  uint8_t* dbg_o;      // debug build only: [B*H*S][S/64] block exponents
  uint8_t* dbg_codes;  // debug build only: [B*H*S][S] probability codes
};

struct Bf16Args {
  const uint16_t* q;  // bf16 bits, BSHD [B][S][H][128]
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  float cp;  // fp32(softmax_scale * log2 e)
  int B, H, S;
};

hipError_t launch_fp8(const Fp8Args& a, int dqk, bool debug, int grid, hipStream_t stream);
hipError_t launch_bf16(const Bf16Args& a, int grid, hipStream_t stream);
hipError_t launch_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* ws,
                                hipStream_t stream);
hipError_t launch_round_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t stream);

}  // namespace cfa
