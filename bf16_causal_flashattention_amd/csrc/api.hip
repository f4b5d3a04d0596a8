// C ABI of libattn_fwd_causal.so: argument validation (host only, before any
// device call), grid selection and launch.  Declarations and contracts are in
// include/attn_fwd_causal.h.
#include <math.h>
#include <stdint.h>

#include "attn_common.hpp"
#include "attn_fwd_causal.h"
#include "attn_launch.hpp"

namespace {

constexpr double kLog2e = 1.4426950408889634074;
constexpr int kMaxDevices = 64;
int g_num_cu[kMaxDevices];  // cached compute-unit count per device (0 = unknown)

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

// common checks of the attention entry points; returns ATTN_OK or an error
int check_attn(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int S,
               int d_qk, int d_v, int want_qk, int want_v, int elem) {
  if (B < 0 || H < 0 || S < 0) return ATTN_ERR_SHAPE;
  if (d_qk != want_qk || d_v != want_v) return ATTN_ERR_SHAPE;
  if (B == 0 || H == 0 || S == 0) return 1;  // empty problem: nothing to do
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (S % cfa::kTileRows != 0) return ATTN_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  // every tensor must hold fewer than 2^31 elements (B, S, H < 2^31, so no overflow below)
  const int64_t dmax = d_qk > d_v ? d_qk : d_v;
  const int64_t lim = INT64_C(1) << 31;
  const int64_t bs = (int64_t)B * S;
  if (bs >= lim || bs * H >= lim || bs * H * dmax >= lim) return ATTN_ERR_RANGE;
  (void)elem;
  return ATTN_OK;
}

int device_cu_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices && g_num_cu[dev] > 0) {
    *n = g_num_cu[dev];
    return ATTN_OK;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices) g_num_cu[dev] = cu;
  *n = cu;
  return ATTN_OK;
}

int grid_for(int B, int H, int S, int num_cu) {
  const cfa::Schedule s = cfa::make_schedule(B, H, S);
  return (int)(s.items < num_cu ? s.items : num_cu);
}

int run_fp8(const void* q, const void* k, const void* v, void* out, float* lse, float qd, float kd, float vd,
            float sm, int B, int H, int S, int dqk, int dv, uint8_t* dbg_o, uint8_t* dbg_c, bool debug,
            void* stream) {
  int rc = check_attn(q, k, v, out, lse, B, H, S, dqk, dv, dqk == 192 ? 192 : 128, 128, 1);
  if (rc == 1) return ATTN_OK;
  if (rc != ATTN_OK) return rc;
  if (!good_scale(qd) || !good_scale(kd) || !good_scale(vd) || !good_scale(sm)) return ATTN_ERR_ARG;
  if (debug) {
    if (!dbg_o || !dbg_c) return ATTN_ERR_NULL;
    if ((int64_t)B * H * S * S > (INT64_C(1) << 28)) return ATTN_ERR_RANGE;
  }
  const float cp = (float)((double)sm * (double)qd * (double)kd * kLog2e);
  if (!isfinite(cp) || !(cp > 0.0f)) return ATTN_ERR_ARG;
  int ncu = 0;
  if ((rc = device_cu_count(&ncu)) != ATTN_OK) return rc;
  cfa::Fp8Args a;
  a.q = (const uint8_t*)q;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.cp = cp;
  a.v_descale = vd;
  a.B = B;
  a.H = H;
  a.S = S;
  a.dbg_o = dbg_o;
  a.dbg_codes = dbg_c;
  const hipError_t e = cfa::launch_fp8(a, dqk, debug, grid_for(B, H, S, ncu), (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_fwd_causal_fp8(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream) {
  if (d_qk != 128) return ATTN_ERR_SHAPE;
  return run_fp8(q, k, v, out, lse, q_descale, k_descale, v_descale, softmax_scale, B, H, S, d_qk, d_v, nullptr,
                 nullptr, false, stream);
}

int attn_fwd_causal_mla(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream) {
  if (d_qk != 192) return ATTN_ERR_SHAPE;
  return run_fp8(q, k, v, out, lse, q_descale, k_descale, v_descale, softmax_scale, B, H, S, d_qk, d_v, nullptr,
                 nullptr, false, stream);
}

int attn_fwd_causal_fp8_debug(const void* q, const void* k, const void* v, void* out, float* lse,
                              float q_descale, float k_descale, float v_descale, float softmax_scale, int B,
                              int H, int S, int d_qk, int d_v, uint8_t* dbg_o, uint8_t* dbg_codes,
                              void* stream) {
  if (d_qk != 128 && d_qk != 192) return ATTN_ERR_SHAPE;
  return run_fp8(q, k, v, out, lse, q_descale, k_descale, v_descale, softmax_scale, B, H, S, d_qk, d_v, dbg_o,
                 dbg_codes, true, stream);
}

int attn_fwd_causal_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                         float softmax_scale, int B, int H, int S, int d_qk, int d_v, void* stream) {
  int rc = check_attn(q, k, v, out, lse, B, H, S, d_qk, d_v, 128, 128, 2);
  if (rc == 1) return ATTN_OK;
  if (rc != ATTN_OK) return rc;
  if (!good_scale(softmax_scale)) return ATTN_ERR_ARG;
  const float cp = (float)((double)softmax_scale * kLog2e);
  if (!isfinite(cp) || !(cp > 0.0f)) return ATTN_ERR_ARG;
  int ncu = 0;
  if ((rc = device_cu_count(&ncu)) != ATTN_OK) return rc;
  cfa::Bf16Args a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.cp = cp;
  a.B = B;
  a.H = H;
  a.S = S;
  const hipError_t e = cfa::launch_bf16(a, grid_for(B, H, S, ncu), (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* workspace,
                       void* stream) {
  if (n < 0) return ATTN_ERR_ARG;
  if (!descale || !workspace) return ATTN_ERR_NULL;
  if (n > 0 && (!x || !codes)) return ATTN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(descale, 4) || !aligned(workspace, 4))
    return ATTN_ERR_ALIGN;
  const hipError_t e = cfa::launch_quantize_e4m3(x, n, codes, descale, workspace, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_round_bf16(const float* x, int64_t n, uint16_t* out, void* stream) {
  if (n < 0) return ATTN_ERR_ARG;
  if (n == 0) return ATTN_OK;
  if (!x || !out) return ATTN_ERR_NULL;
  if (!aligned(x, 4) || !aligned(out, 2)) return ATTN_ERR_ALIGN;
  const hipError_t e = cfa::launch_round_bf16(x, n, out, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_default_grid(int B, int H, int S, int num_cu) {
  if (B <= 0 || H <= 0 || S <= 0 || S % cfa::kTileRows != 0 || num_cu <= 0) return ATTN_ERR_SHAPE;
  return grid_for(B, H, S, num_cu);
}

int64_t attn_schedule(int B, int H, int S, int grid, int32_t* records, int64_t cap) {
  if (B <= 0 || H <= 0 || S <= 0 || S % cfa::kTileRows != 0 || grid <= 0) return ATTN_ERR_SHAPE;
  const cfa::Schedule s = cfa::make_schedule(B, H, S);
  const int64_t need = (int64_t)B * H * s.T;
  if (!records || cap < need) return ATTN_ERR_ARG;
  int64_t n = 0;
  for (int bid = 0; bid < grid; ++bid) {
    const int logical = cfa::xcd_logical(bid, grid);
    for (int64_t item = logical; item < s.items; item += grid) {
      int b, h, j;
      cfa::decode_item(item, H, s.P, b, h, j);
      for (int pass = 0; pass < 2; ++pass) {
        const int tile = pass == 0 ? j : s.T - 1 - j;
        if (pass == 1 && tile == j) break;
        if (n >= need) return ATTN_ERR_ARG;  // would mean a tile is visited twice
        records[4 * n + 0] = bid;
        records[4 * n + 1] = b;
        records[4 * n + 2] = h;
        records[4 * n + 3] = tile;
        ++n;
      }
    }
  }
  return n;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "unsupported shape (S must be a positive multiple of 256; check head dims)";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_RANGE: return "tensor too large (2^31 elements or more)";
    case ATTN_ERR_ARG: return "invalid argument (scales must be finite and positive)";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

}  // extern "C"
