// C ABI of libattn_fwd_causal.so: argument validation (host only, before any
// device call), grid selection and launch.  Declarations and contracts are in
// include/attn_fwd_causal.h.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "attn_common.hpp"
#include "attn_fwd_causal.h"
#include "attn_launch.hpp"

namespace {

constexpr double kLog2e = 1.4426950408889634074;
constexpr int kMaxDevices = 64;
// cached compute-unit count per device (0 = unknown); atomic because the entry points may be
// called from several host threads at once
std::atomic<int> g_num_cu[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

// Problem description shared by the attention entry points (element strides).
struct Problem {
  const void *q, *k, *v;
  void* out;
  float* lse;
  int B, H, Hkv, S, dqk, dv;
  attn_strides sq, sk, sv, so;
  bool v_channel_major;  // v is [B][H_kv][d_v][S]: sv.seq is the channel row stride
};

attn_strides bshd(int S, int H, int d) {
  attn_strides t;
  t.batch = (int64_t)S * H * d;
  t.head = d;
  t.seq = (int64_t)H * d;
  return t;
}

// one tensor: strides non-negative, byte strides multiples of 16 (16-byte rows and cells),
// every element offset below 2^31, and 128 rows of the row stride below 2^31 bytes
int check_tensor(const attn_strides& t, int B, int S, int heads, int d, int elem) {
  if (t.batch < 0 || t.head < 0 || t.seq < 0) return ATTN_ERR_ARG;
  if ((t.batch * elem) % 16 || (t.head * elem) % 16 || (t.seq * elem) % 16) return ATTN_ERR_ALIGN;
  const int64_t lim = INT64_C(1) << 31;
  if (t.batch >= lim || t.head >= lim || t.seq * elem * cfa::kBlockKeys >= lim) return ATTN_ERR_RANGE;
  const int64_t last = (int64_t)(B - 1) * t.batch + (int64_t)(heads - 1) * t.head + (int64_t)(S - 1) * t.seq + d;
  if (last >= lim) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

// The output's (b, h, s) rows must not overlap, or several workgroups would write the same
// bytes.  Sufficient test: with the levels of extent > 1 sorted by stride, each stride is at
// least the span that the levels below it cover (d elements to begin with).  Rejects zero
// strides (expanded views) and interleaved rows.
int check_no_overlap(const attn_strides& t, int B, int S, int heads, int d) {
  int64_t st[3] = {t.batch, t.head, t.seq}, n[3] = {B, heads, S};
  for (int i = 0; i < 3; ++i)  // sort the three levels by stride
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        const int64_t a = st[i], c = n[i];
        st[i] = st[j];
        n[i] = n[j];
        st[j] = a;
        n[j] = c;
      }
  int64_t span = d;
  for (int i = 0; i < 3; ++i) {
    if (n[i] <= 1) continue;
    if (st[i] < span) return ATTN_ERR_ARG;
    span += (n[i] - 1) * st[i];
  }
  return ATTN_OK;
}

// common checks of the attention entry points; returns ATTN_OK, 1 for an empty problem,
// or an error
int check_attn(const Problem& p, int elem) {
  if (p.B < 0 || p.H < 0 || p.S < 0 || p.Hkv < 0) return ATTN_ERR_SHAPE;
  if (p.B == 0 || p.H == 0 || p.S == 0) return 1;  // empty problem: nothing to do
  if (p.Hkv < 1 || p.H % p.Hkv != 0) return ATTN_ERR_SHAPE;
  if (!p.q || !p.k || !p.v || !p.out) return ATTN_ERR_NULL;
  if (p.S % cfa::kTileRows != 0) return ATTN_ERR_SHAPE;
  if (!aligned(p.q, 16) || !aligned(p.k, 16) || !aligned(p.v, 16) || !aligned(p.out, 16)) return ATTN_ERR_ALIGN;
  if (p.lse && !aligned(p.lse, 4)) return ATTN_ERR_ALIGN;
  const int64_t lim = INT64_C(1) << 31;
  if ((int64_t)p.B * p.H * p.S >= lim) return ATTN_ERR_RANGE;  // lse, and the schedule's counts
  int rc;
  if ((rc = check_tensor(p.sq, p.B, p.S, p.H, p.dqk, elem)) != ATTN_OK) return rc;
  if ((rc = check_tensor(p.sk, p.B, p.S, p.Hkv, p.dqk, elem)) != ATTN_OK) return rc;
  if (p.v_channel_major) {  // d_v rows of S contiguous keys: the same rules with rows and columns swapped
    if ((rc = check_tensor(p.sv, p.B, p.dv, p.Hkv, p.S, elem)) != ATTN_OK) return rc;
  } else if ((rc = check_tensor(p.sv, p.B, p.S, p.Hkv, p.dv, elem)) != ATTN_OK) {
    return rc;
  }
  if ((rc = check_tensor(p.so, p.B, p.S, p.H, p.dv, 2)) != ATTN_OK) return rc;
  if ((rc = check_no_overlap(p.so, p.B, p.S, p.H, p.dv)) != ATTN_OK) return rc;
  return ATTN_OK;
}

cfa::TensorMap tmap(const attn_strides& t, int elem) {
  cfa::TensorMap m;
  m.sb = t.batch * elem;
  m.sh = t.head * elem;
  m.ss = (int)(t.seq * elem);
  return m;
}

Problem make_problem(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                     int S, int dqk, int dv, const attn_strides* sq, const attn_strides* sk,
                     const attn_strides* sv, const attn_strides* so) {
  Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.S = S;
  p.dqk = dqk;
  p.dv = dv;
  const int hk = Hkv > 0 ? Hkv : 1;
  p.sq = sq ? *sq : bshd(S, H, dqk);
  p.sk = sk ? *sk : bshd(S, hk, dqk);
  p.sv = sv ? *sv : bshd(S, hk, dv);
  p.so = so ? *so : bshd(S, H, dv);
  p.v_channel_major = false;
  return p;
}

int device_cu_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices && g_num_cu[dev].load(std::memory_order_relaxed) > 0) {
    *n = g_num_cu[dev].load(std::memory_order_relaxed);
    return ATTN_OK;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices) g_num_cu[dev].store(cu, std::memory_order_relaxed);
  *n = cu;
  return ATTN_OK;
}

// the head-pair mode (Sec. IV-A): grouped-query attention with an even number of query
// heads per key/value head
bool pair_heads(int H, int Hkv) { return Hkv > 0 && H % Hkv == 0 && (H / Hkv) % 2 == 0; }

int grid_for(int B, int H, int Hkv, int S, int num_cu) {
  const cfa::Schedule s = cfa::make_schedule(B, H, S, pair_heads(H, Hkv));
  return (int)(s.items < num_cu ? s.items : num_cu);
}

int run_fp8(const Problem& p, float qd, float kd, float vd, float sm, int p_mode, uint8_t* dbg_o, uint8_t* dbg_c,
            float* dbg_s, bool debug, void* stream) {
  if (p.dqk != 128 && p.dqk != 192) return ATTN_ERR_SHAPE;
  if (p.dv != 128) return ATTN_ERR_SHAPE;
  if (p_mode != ATTN_P_DEFAULT && p_mode != ATTN_P_LEAN && p_mode != ATTN_P_EXACT) return ATTN_ERR_ARG;
  int rc = check_attn(p, 1);
  if (rc == 1) return ATTN_OK;
  if (rc != ATTN_OK) return rc;
  if (!good_scale(qd) || !good_scale(kd) || !good_scale(vd) || !good_scale(sm)) return ATTN_ERR_ARG;
  if (debug) {
    if (!dbg_o || !dbg_c) return ATTN_ERR_NULL;
    if ((int64_t)p.B * p.H * p.S * p.S > (INT64_C(1) << 28)) return ATTN_ERR_RANGE;
    if (dbg_s && !aligned(dbg_s, 16)) return ATTN_ERR_ALIGN;
  }
  const float cp = (float)((double)sm * (double)qd * (double)kd * kLog2e);
  if (!isfinite(cp) || !(cp > 0.0f)) return ATTN_ERR_ARG;
  int ncu = 0;
  if ((rc = device_cu_count(&ncu)) != ATTN_OK) return rc;
  cfa::Fp8Args a;
  a.q = (const uint8_t*)p.q;
  a.k = (const uint8_t*)p.k;
  a.v = (const uint8_t*)p.v;
  a.out = (uint16_t*)p.out;
  a.lse = p.lse;
  a.cp = cp;
  a.v_descale = vd;
  a.B = p.B;
  a.H = p.H;
  a.S = p.S;
  a.G = p.H / p.Hkv;
  a.pair_heads = pair_heads(p.H, p.Hkv) ? 1 : 0;
  a.mq = tmap(p.sq, 1);
  a.mk = tmap(p.sk, 1);
  a.mv = tmap(p.sv, 1);
  a.mo = tmap(p.so, 2);
  a.dbg_o = dbg_o;
  a.dbg_codes = dbg_c;
  a.dbg_scores = dbg_s;
  const bool exact = p_mode == ATTN_P_EXACT || (p_mode == ATTN_P_DEFAULT && p.dqk == 192);
  const hipError_t e =
      cfa::launch_fp8(a, p.dqk, exact, debug, p.v_channel_major, grid_for(p.B, p.H, p.Hkv, p.S, ncu), (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int run_bf16(const Problem& p, float sm, void* stream) {
  if ((p.dqk != 128 && p.dqk != 192) || p.dv != 128) return ATTN_ERR_SHAPE;
  int rc = check_attn(p, 2);
  if (rc == 1) return ATTN_OK;
  if (rc != ATTN_OK) return rc;
  if (!good_scale(sm)) return ATTN_ERR_ARG;
  const float cp = (float)((double)sm * kLog2e);
  if (!isfinite(cp) || !(cp > 0.0f)) return ATTN_ERR_ARG;
  int ncu = 0;
  if ((rc = device_cu_count(&ncu)) != ATTN_OK) return rc;
  cfa::Bf16Args a;
  a.q = (const uint16_t*)p.q;
  a.k = (const uint16_t*)p.k;
  a.v = (const uint16_t*)p.v;
  a.out = (uint16_t*)p.out;
  a.lse = p.lse;
  a.cp = cp;
  a.B = p.B;
  a.H = p.H;
  a.S = p.S;
  a.G = p.H / p.Hkv;
  a.pair_heads = pair_heads(p.H, p.Hkv) ? 1 : 0;
  a.mq = tmap(p.sq, 2);
  a.mk = tmap(p.sk, 2);
  a.mv = tmap(p.sv, 2);
  a.mo = tmap(p.so, 2);
  const hipError_t e = cfa::launch_bf16(a, p.dqk, grid_for(p.B, p.H, p.Hkv, p.S, ncu), (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Power-of-two descale in [2^-126, 2^126] -> the scale 2^k that multiplies x; 0 if invalid.
float static_scale_of(float descale) {
  int e;
  const float m = frexpf(descale, &e);  // descale = m 2^e; a power of two has m = 0.5
  if (!(m == 0.5f) || e - 1 < -126 || e - 1 > 126) return 0.f;
  return ldexpf(1.f, 1 - e);
}

int check_rotate(const float* x, const float* mean, const float* signs, int B, int S, int H, int D,
                 const uint8_t* codes) {
  if (B < 0 || S < 0 || H < 0 || (D != 128 && D != 192)) return ATTN_ERR_SHAPE;
  if (!signs) return ATTN_ERR_NULL;
  const int64_t n = (int64_t)B * S * H * D;
  if (n > 0 && (!x || !codes)) return ATTN_ERR_NULL;
  if (!aligned(x, 4) || !aligned(signs, 4) || !aligned(mean, 4)) return ATTN_ERR_ALIGN;
  if (n >= (INT64_C(1) << 31)) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

// orthonormal DCT-II of size 3 (the C_m factor at D = 192): C[k][n] = a_k cos(pi (2n+1) k / 6)
void dct3(float c3[9]) {
  for (int kk = 0; kk < 3; ++kk)
    for (int nn = 0; nn < 3; ++nn)
      c3[3 * kk + nn] = (float)((kk == 0 ? sqrt(1.0 / 3.0) : sqrt(2.0 / 3.0)) * cos(M_PI * (2 * nn + 1) * kk / 6.0));
}

}  // namespace

extern "C" {

int attn_fwd_causal_fp8(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream) {
  if (d_qk != 128) return ATTN_ERR_SHAPE;
  const Problem p = make_problem(q, k, v, out, lse, B, H, H, S, d_qk, d_v, nullptr, nullptr, nullptr, nullptr);
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, ATTN_P_LEAN, nullptr, nullptr, nullptr, false,
                 stream);
}

int attn_fwd_causal_mla(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream) {
  if (d_qk != 192) return ATTN_ERR_SHAPE;
  const Problem p = make_problem(q, k, v, out, lse, B, H, H, S, d_qk, d_v, nullptr, nullptr, nullptr, nullptr);
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, ATTN_P_EXACT, nullptr, nullptr, nullptr, false,
                 stream);
}

int attn_fwd_causal_fp8_ex(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                           float k_descale, float v_descale, float softmax_scale, int B, int H, int H_kv, int S,
                           int d_qk, int d_v, const attn_strides* q_strides, const attn_strides* k_strides,
                           const attn_strides* v_strides, const attn_strides* out_strides, int p_mode,
                           void* stream) {
  const Problem p = make_problem(q, k, v, out, lse, B, H, H_kv, S, d_qk, d_v, q_strides, k_strides, v_strides,
                                 out_strides);
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, p_mode, nullptr, nullptr, nullptr, false,
                 stream);
}

int attn_fwd_causal_fp8_vt(const void* q, const void* k, const void* vt, void* out, float* lse, float q_descale,
                           float k_descale, float v_descale, float softmax_scale, int B, int H, int H_kv, int S,
                           int d_qk, int d_v, const attn_strides* q_strides, const attn_strides* k_strides,
                           const attn_strides* vt_strides, const attn_strides* out_strides, int p_mode,
                           void* stream) {
  Problem p = make_problem(q, k, vt, out, lse, B, H, H_kv, S, d_qk, d_v, q_strides, k_strides, nullptr,
                           out_strides);
  if (vt_strides) {
    p.sv = *vt_strides;
  } else {  // dense [B][H_kv][d_v][S]
    const int64_t hk = H_kv > 0 ? H_kv : 1;
    p.sv.batch = hk * d_v * S;
    p.sv.head = (int64_t)d_v * S;
    p.sv.seq = S;
  }
  p.v_channel_major = true;
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, p_mode, nullptr, nullptr, nullptr, false,
                 stream);
}

int attn_fwd_causal_fp8_debug(const void* q, const void* k, const void* v, void* out, float* lse,
                              float q_descale, float k_descale, float v_descale, float softmax_scale, int B,
                              int H, int S, int d_qk, int d_v, uint8_t* dbg_o, uint8_t* dbg_codes,
                              void* stream) {
  const Problem p = make_problem(q, k, v, out, lse, B, H, H, S, d_qk, d_v, nullptr, nullptr, nullptr, nullptr);
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, ATTN_P_DEFAULT, dbg_o, dbg_codes, nullptr,
                 true, stream);
}

int attn_fwd_causal_fp8_debug_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                                 float q_descale, float k_descale, float v_descale, float softmax_scale, int B,
                                 int H, int H_kv, int S, int d_qk, int d_v, const attn_strides* q_strides,
                                 const attn_strides* k_strides, const attn_strides* v_strides,
                                 const attn_strides* out_strides, int p_mode, uint8_t* dbg_o, uint8_t* dbg_codes,
                                 float* dbg_scores, void* stream) {
  const Problem p = make_problem(q, k, v, out, lse, B, H, H_kv, S, d_qk, d_v, q_strides, k_strides, v_strides,
                                 out_strides);
  return run_fp8(p, q_descale, k_descale, v_descale, softmax_scale, p_mode, dbg_o, dbg_codes, dbg_scores, true,
                 stream);
}

int attn_fwd_causal_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                         float softmax_scale, int B, int H, int S, int d_qk, int d_v, void* stream) {
  if (d_qk != 128) return ATTN_ERR_SHAPE;
  const Problem p = make_problem(q, k, v, out, lse, B, H, H, S, d_qk, d_v, nullptr, nullptr, nullptr, nullptr);
  return run_bf16(p, softmax_scale, stream);
}

int attn_fwd_causal_bf16_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                            float softmax_scale, int B, int H, int H_kv, int S, int d_qk, int d_v,
                            const attn_strides* q_strides, const attn_strides* k_strides,
                            const attn_strides* v_strides, const attn_strides* out_strides, void* stream) {
  const Problem p = make_problem(q, k, v, out, lse, B, H, H_kv, S, d_qk, d_v, q_strides, k_strides, v_strides,
                                 out_strides);
  return run_bf16(p, softmax_scale, stream);
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

int64_t attn_key_mean_workspace(int B, int S, int H, int D) {
  if (B < 0 || S < 0 || H < 0 || (D != 128 && D != 192)) return ATTN_ERR_SHAPE;
  return cfa::key_mean_workspace_bytes(B, S, H, D);
}

int attn_key_mean(const float* k, int B, int S, int H, int D, float* mean, void* workspace, void* stream) {
  if (B < 0 || S < 0 || H < 0 || (D != 128 && D != 192)) return ATTN_ERR_SHAPE;
  if (B == 0 || H == 0) return ATTN_OK;
  if (S == 0) return ATTN_ERR_SHAPE;  // the mean of no keys is undefined
  if (!k || !mean || !workspace) return ATTN_ERR_NULL;
  if (!aligned(k, 4) || !aligned(mean, 4) || !aligned(workspace, 8)) return ATTN_ERR_ALIGN;
  if ((int64_t)B * S * H * D >= (INT64_C(1) << 31) || (int64_t)B * H >= 65536) return ATTN_ERR_RANGE;
  const hipError_t e = cfa::launch_key_mean(k, B, S, H, D, mean, workspace, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_key_mean_noalloc(const float* k, int B, int S, int H, int D, float* mean, void* stream) {
  if (B < 0 || S < 0 || H < 0 || (D != 128 && D != 192)) return ATTN_ERR_SHAPE;
  if (B == 0 || H == 0) return ATTN_OK;
  if (S == 0) return ATTN_ERR_SHAPE;
  if (!k || !mean) return ATTN_ERR_NULL;
  if (!aligned(k, 4) || !aligned(mean, 4)) return ATTN_ERR_ALIGN;
  if ((int64_t)B * S * H * D >= (INT64_C(1) << 31) || (int64_t)B * H >= 65536) return ATTN_ERR_RANGE;
  if (cfa::key_mean_workspace_bytes(B, S, H, D) > cfa::kKeyMeanScratchBytes) return ATTN_ERR_SCRATCH;
  const hipError_t e = cfa::launch_key_mean_noalloc(k, B, S, H, D, mean, (hipStream_t)stream);
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice) return ATTN_ERR_DEVICE;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_rotate_quantize_e4m3(const float* x, const float* mean, const float* signs, int B, int S, int H, int D,
                              uint8_t* codes, float* descale, uint32_t* workspace, void* stream) {
  const int rc = check_rotate(x, mean, signs, B, S, H, D, codes);
  if (rc != ATTN_OK) return rc;
  if (!descale || !workspace) return ATTN_ERR_NULL;
  if (!aligned(descale, 4) || !aligned(workspace, 4)) return ATTN_ERR_ALIGN;
  float c3[9];
  dct3(c3);
  const hipError_t e = cfa::launch_rotate_quantize(x, mean, signs, B, S, H, D, c3, codes, descale, workspace, 1.f,
                                                   false, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_rotate_quantize_e4m3_static(const float* x, const float* mean, const float* signs, int B, int S, int H,
                                     int D, float descale, uint8_t* codes, void* stream) {
  const int rc = check_rotate(x, mean, signs, B, S, H, D, codes);
  if (rc != ATTN_OK) return rc;
  const float scale = static_scale_of(descale);
  if (scale == 0.f) return ATTN_ERR_ARG;
  if ((int64_t)B * S * H == 0) return ATTN_OK;
  float c3[9];
  dct3(c3);
  const hipError_t e = cfa::launch_rotate_quantize(x, mean, signs, B, S, H, D, c3, codes, nullptr, nullptr, scale,
                                                   true, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_quantize_e4m3_static(const float* x, int64_t n, float descale, uint8_t* codes, void* stream) {
  if (n < 0) return ATTN_ERR_ARG;
  const float scale = static_scale_of(descale);
  if (scale == 0.f) return ATTN_ERR_ARG;
  if (n == 0) return ATTN_OK;
  if (!x || !codes) return ATTN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 4)) return ATTN_ERR_ALIGN;
  const hipError_t e = cfa::launch_quantize_e4m3_static(x, n, scale, codes, (hipStream_t)stream);
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

int attn_default_grid(int B, int H, int H_kv, int S, int num_cu) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || S <= 0 || S % cfa::kTileRows != 0 || num_cu <= 0)
    return ATTN_ERR_SHAPE;
  return grid_for(B, H, H_kv, S, num_cu);
}

int64_t attn_schedule(int B, int H, int H_kv, int S, int grid, int32_t* records, int64_t cap) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || S <= 0 || S % cfa::kTileRows != 0 || grid <= 0)
    return ATTN_ERR_SHAPE;
  const bool pair = pair_heads(H, H_kv);
  const cfa::Schedule s = cfa::make_schedule(B, H, S, pair);
  const int rows = pair ? cfa::kPairTileRows : cfa::kTileRows, hstep = pair ? 2 : 1;
  const int64_t need = (int64_t)B * H * (S / rows);
  if (!records || cap < need) return ATTN_ERR_ARG;
  int64_t n = 0;
  for (int bid = 0; bid < grid; ++bid) {
    const cfa::ItemRange work = cfa::xcd_items(bid, grid, s.items);
    for (int64_t item = work.first; item < work.end; item += work.step) {
      int b, u, j;
      cfa::decode_item(item, s.HS, s.P, b, u, j);
      for (int pass = 0; pass < 2; ++pass) {
        const int tile = pass == 0 ? s.T - 1 - j : j;
        if (pass == 1 && tile == s.T - 1 - j) break;
        for (int e = 0; e < hstep; ++e) {
          if (n >= need) return ATTN_ERR_ARG;  // would mean a tile is visited twice
          int32_t* r = records + 5 * n;
          r[0] = bid;
          r[1] = b;
          r[2] = hstep * u + e;
          r[3] = tile * rows;
          r[4] = rows;
          ++n;
        }
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
    case ATTN_ERR_SCRATCH:
      return "problem needs more scratch memory than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

}  // extern "C"
