/*
 * attn_fwd_causal.h -- C ABI of the causal attention forward (prefill) library for
 * AMD Instinct MI355X (gfx950, CDNA4): libattn_fwd_causal.so.
 *
 * The operation is causal softmax attention, "ZYFA: Speed and Accuracy of FP8
 * FlashAttention on AMD CDNA4" (Anthony, Bikshandi, Medepalli, Ebert), Sec. II-B:
 *     O = softmax(c Q K^T + M) V,   M the causal mask (query i sees keys 0..i),
 * with the log-sum-exp of every row of scores, for one (batch, head) at a time over
 * B batches and H heads.  Supported configurations follow the paper's Table VI:
 * causal forward only, equal query and key lengths S (a multiple of 256),
 * multi-head attention, BF16 or e4m3 operands with one fp32 scale per tensor,
 * BF16 output and fp32 LSE.
 *
 * Layout of the basic entry points (all tensors dense, row-major):
 *   q, k : [B][S][H][d_qk]   (BSHD, the (batch, seqlen, heads, headdim) order)
 *   v    : [B][S][H][d_v]
 *   out  : [B][S][H][d_v]    bf16
 * The *_ex entry points take any strided layout (BSHD, BHSD, ...) and grouped-query
 * attention (H query heads over H_kv key/value heads; Table VI lists both).
 *   lse  : [B][H][S]         fp32, natural log of sum_j exp(c q_i.k_j) over visible
 *                            keys (for FP8, of the rounded probabilities; Sec. IV-B3)
 * e4m3 is the OCP "fn" variant (bias 7, max 448, no infinities), not FNUZ.
 *
 * Memory and ownership: every pointer is a device pointer owned by the caller;
 * the library allocates nothing and keeps no pointer after a call returns.
 * q, k, v, out must be 16-byte aligned, lse 4-byte aligned.
 *
 * Execution: calls are asynchronous on `stream` (a hipStream_t; NULL = the
 * default stream) and never synchronise.  All functions are reentrant.  The
 * attention kernels use a static work partition and no atomics, so results are
 * bitwise identical from run to run (Sec. VI-B, Table XII property).
 *
 * Errors: arguments are validated on the host before any device call, and
 * nothing is launched when a check fails.  A call with B, H or S equal to zero
 * is a no-op that returns ATTN_OK.  Launch failures map to ATTN_ERR_LAUNCH.
 * NaN or infinite inputs are not errors but are unsupported (outputs undefined).
 */
#ifndef ATTN_FWD_CAUSAL_H
#define ATTN_FWD_CAUSAL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,   /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,  /* negative size, S not a multiple of 256, or wrong head dims */
  ATTN_ERR_ALIGN = -3,  /* pointer misaligned */
  ATTN_ERR_RANGE = -4,  /* a tensor has 2^31 elements or more */
  ATTN_ERR_ARG = -5,    /* a scale is not finite and positive, or a bad size argument */
  ATTN_ERR_LAUNCH = -6, /* the kernel launch failed (hipGetLastError) */
  ATTN_ERR_DEVICE = -7, /* no usable device / device query failed */
  ATTN_ERR_SCRATCH = -8 /* the allocation-free entry point's scratch array is too small */
} attn_status;

/* Element strides of one attention tensor for the *_ex entry points: element
 * (b, s, h, d) sits at base + b*batch + h*head + s*seq + d (the head dimension is
 * contiguous).  BSHD [B][S][H][D] is {S*H*D, D, H*D}; BHSD [B][H][S][D] is {H*S*D, S*D, D}.
 * Every stride must be >= 0 and a multiple of 16 bytes, every element offset below 2^31,
 * and 128 rows of the seq stride below 2^31 bytes; tensors must not overlap `out`.
 * The rows of `out` must not overlap one another: sorted by stride, the levels with more
 * than one entry must each have a stride at least the span of the levels below them (so
 * zero strides and interleaved rows are refused with ATTN_ERR_ARG). */
typedef struct {
  int64_t batch;
  int64_t head;
  int64_t seq;
} attn_strides;

/* FP8 probability mode (paper Sec. IV-B1): lean P forms each e4m3 code with one
 * multiply-add and an integer conversion; exact P rounds 2^x to e4m3.  DEFAULT is the
 * paper's choice per shape: lean P at d_qk = 128, exact P at d_qk = 192. */
enum { ATTN_P_DEFAULT = -1, ATTN_P_LEAN = 0, ATTN_P_EXACT = 1 };

/* FP8 causal attention at head dimension 128 with lean P.
 * Paper Sec. IV-B1 (Eq. 2: each probability's e4m3 code from one multiply-add and
 * an integer conversion), Sec. IV-B2 (per-64-key-block power-of-two scaling undone
 * by the scaled PV MFMA), Sec. IV-B3 (row sum of the rounded probabilities),
 * Sec. II-C (per-tensor scales folded into the score scale and the output).
 * q, k, v: e4m3 codes; *_descale: the fp32 factors that map codes back to values
 * (value = decoded code * descale); softmax_scale: c (e.g. 1/sqrt(128)).
 * d_qk and d_v must both be 128. */
int attn_fwd_causal_fp8(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream);

/* BF16 causal attention at head dimension 128 (paper Sec. II-B, Sec. IV-A and
 * IV-D: BF16 operands, fp32 softmax with the scale applied to the fp32 scores).
 * q, k, v: bf16 bit patterns.  d_qk and d_v must both be 128. */
int attn_fwd_causal_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                         float softmax_scale, int B, int H, int S, int d_qk, int d_v, void* stream);

/* FP8 causal attention at the MLA prefill shape, d_qk = 192 and d_v = 128, with
 * exact P (paper Sec. IV-B1: the exponential and an e4m3 conversion per
 * probability; Sec. IV intro: the MLA-shaped kernel keeps exact P), plus the
 * block scaling and rounded-sum normaliser of Sec. IV-B2/B3.  Arguments as for
 * attn_fwd_causal_fp8; d_qk must be 192 and d_v 128. */
int attn_fwd_causal_mla(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                        float k_descale, float v_descale, float softmax_scale, int B, int H, int S, int d_qk,
                        int d_v, void* stream);

/* General FP8 entry point: d_qk in {128, 192}, d_v = 128, H query heads and H_kv
 * key/value heads (H a multiple of H_kv; query head h reads key/value head
 * h / (H / H_kv), the grouped-query attention of paper Table VI), per-tensor strides
 * (NULL = dense BSHD with H heads for q/out and H_kv heads for k/v), and the P mode
 * (ATTN_P_*).  lse stays dense [B][H][S].  Other arguments and errors as for
 * attn_fwd_causal_fp8; ATTN_ERR_ARG for an unknown p_mode or a negative stride,
 * ATTN_ERR_ALIGN for a stride that is not a multiple of 16 bytes, ATTN_ERR_SHAPE when
 * H_kv does not divide H. */
int attn_fwd_causal_fp8_ex(const void* q, const void* k, const void* v, void* out, float* lse, float q_descale,
                           float k_descale, float v_descale, float softmax_scale, int B, int H, int H_kv, int S,
                           int d_qk, int d_v, const attn_strides* q_strides, const attn_strides* k_strides,
                           const attn_strides* v_strides, const attn_strides* out_strides, int p_mode,
                           void* stream);

/* attn_fwd_causal_fp8_ex with V given channel-major: vt holds, per batch and key/value
 * head, d_v = 128 rows of S contiguous e4m3 key codes (vt[b][g][d][s] = v[b][s][g][d]),
 * the layout in which the PV product (paper Sec. IV-A, O^T = V^T P^T) reads its operand
 * directly.  vt_strides: batch, head and, in its seq field, the stride between channel
 * rows, in bytes (NULL = dense [B][H_kv][128][S]); the same rules as the other strides
 * (multiples of 16 bytes, non-negative, offsets below 2^31).  Results are bit-identical
 * to attn_fwd_causal_fp8_ex on the same values.  Other arguments and errors as for
 * attn_fwd_causal_fp8_ex. */
int attn_fwd_causal_fp8_vt(const void* q, const void* k, const void* vt, void* out, float* lse, float q_descale,
                           float k_descale, float v_descale, float softmax_scale, int B, int H, int H_kv, int S,
                           int d_qk, int d_v, const attn_strides* q_strides, const attn_strides* k_strides,
                           const attn_strides* vt_strides, const attn_strides* out_strides, int p_mode,
                           void* stream);

/* General BF16 entry point: d_qk = 128, or the MLA shape d_qk = 192, with d_v = 128;
 * grouped-query heads and strides as for attn_fwd_causal_fp8_ex (strides in bf16
 * elements).  At d_qk = 192 the lazy-rescale threshold is 8 binades, as in the paper's
 * BF16 MLA kernel (Sec. IV-A). */
int attn_fwd_causal_bf16_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                            float softmax_scale, int B, int H, int H_kv, int S, int d_qk, int d_v,
                            const attn_strides* q_strides, const attn_strides* k_strides,
                            const attn_strides* v_strides, const attn_strides* out_strides, void* stream);

/* Per-tensor power-of-two e4m3 quantiser (paper Sec. V-E, footnote 17): finds
 * amax = max |x|, takes the largest 2^k with amax * 2^k <= 448 (k clamped to
 * [-126, 126], k = 0 when amax = 0), writes codes[i] = e4m3_rne(x[i] * 2^k) and
 * *descale = 2^-k.  x: n fp32 values (16-byte aligned); codes: n bytes (4-byte
 * aligned); descale: one device float; workspace: one device uint32 that the
 * call overwrites (do not share it between concurrent calls).  n >= 0. */
int attn_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, float* descale, uint32_t* workspace,
                       void* stream);

/* K smoothing for the quantisation pre-pass (paper Sec. V-E, "Rotation and K smoothing":
 * the mean key of each head over the sequence is subtracted before the rotation).
 * k: dense fp32 [B][S][H][D] (4-byte aligned), D in {128, 192}, S > 0;
 * mean: [B][H][D] fp32, mean[b][h][d] = (1/S) sum_s k[b][s][h][d], summed in fp64 in a
 * fixed order (chunks of 1024 keys, then the chunks in sequence) and rounded once to fp32,
 * so repeat calls give identical results and identical keys give their own value;
 * workspace: attn_key_mean_workspace(B, S, H, D) bytes of device memory (8-byte
 * aligned), overwritten.  B*H < 65536 and B*S*H*D < 2^31 (else ATTN_ERR_RANGE).
 * B = 0 or H = 0 is a no-op. */
int64_t attn_key_mean_workspace(int B, int S, int H, int D);
int attn_key_mean(const float* k, int B, int S, int H, int D, float* mean, void* workspace, void* stream);

/* attn_key_mean for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results, with the fp64 partial sums in a static 4 MiB device array of the library instead
 * of a caller workspace.  The call allocates nothing.  Each GPU it runs on holds its own
 * copy of the array until the process ends.  Needs B*H*ceil(S/1024)*D*8 <= 4 MiB
 * (B*H*ceil(S/1024)*D <= 524288, e.g. B = 1, H = 32, S = 131072, D = 128), else
 * ATTN_ERR_SCRATCH and nothing is launched.  Every call on one GPU uses that GPU's array:
 * calls that overlap on one GPU (other streams or host threads) race and must be
 * serialised by the caller.  Other arguments and errors as for attn_key_mean. */
int attn_key_mean_noalloc(const float* k, int B, int S, int H, int D, float* mean, void* stream);

/* Quantisation pre-pass with rotation (paper Sec. V-E, "Rotation and K smoothing", and
 * Table XIII): y = (x - mean[b][h]) R with R = diag(signs) (C_m kron H_{D/m}), H the
 * normalised Sylvester-Hadamard matrix, C_m the orthonormal DCT-II, m = 1 at D = 128 and
 * 3 at D = 192 (element (a, b) -> (a', b') of the Kronecker product is C[a][a'] H[b][b'],
 * index a*(D/m) + b), computed in fp32; then the per-tensor power-of-two e4m3 quantiser
 * of attn_quantize_e4m3 with the scale taken from max |y|.  R is orthogonal, so
 * (QR)(KR)^T = QK^T: rotate q and k with the same signs (k with its mean for K smoothing,
 * q without), leave v unrotated, and call the attention entry points as usual.
 * x: dense fp32 [B][S][H][D]; mean: [B][H][D] fp32, or NULL for no smoothing; signs: D
 * fp32 values, each +1 or -1, drawn by the caller (other values do not give an orthogonal
 * transform); codes: [B][S][H][D] bytes; descale and workspace as for attn_quantize_e4m3.
 * B*S*H*D < 2^31.  y is computed twice (for the maximum, then for the codes) and never
 * stored. */
int attn_rotate_quantize_e4m3(const float* x, const float* mean, const float* signs, int B, int S, int H, int D,
                              uint8_t* codes, float* descale, uint32_t* workspace, void* stream);

/* Static-scale quantisers (paper Sec. V-E: the fused quantisation pass uses a static
 * power-of-two scale, set per tensor from calibration, so it needs no pass for the
 * maximum).  descale: a host float, a power of two in [2^-126, 2^126] (else ATTN_ERR_ARG);
 * codes[i] = e4m3_rne(x[i] / descale), and scaled values beyond +-448 saturate to +-448.
 * attn_quantize_e4m3_static: n fp32 values (x 16-byte aligned, codes 4-byte aligned).
 * attn_rotate_quantize_e4m3_static: the rotation of attn_rotate_quantize_e4m3 (same
 * arguments and layout) followed by this quantiser; one read of x, one write of codes. */
int attn_quantize_e4m3_static(const float* x, int64_t n, float descale, uint8_t* codes, void* stream);
int attn_rotate_quantize_e4m3_static(const float* x, const float* mean, const float* signs, int B, int S, int H,
                                     int D, float descale, uint8_t* codes, void* stream);

/* fp32 -> bf16 rounding to nearest even (the BF16 operands of the paper's Sec. V-D
 * error measurement are the inputs rounded to BF16).  out: n uint16 bit patterns. */
int attn_round_bf16(const float* x, int64_t n, uint16_t* out, void* stream);

/* Test hooks.  Same computation as attn_fwd_causal_fp8 / attn_fwd_causal_mla (dense
 * BSHD, H_kv = H, the default P mode of the head dimension), and
 * in addition the kernel writes, for every (b, h, query row) and every block it
 * processes, the block-scale exponent o of each 64-key block (dbg_o, [B*H*S][S/64]
 * bytes) and the e4m3 code of every probability it forms (dbg_codes, [B*H*S][S]
 * bytes; masked keys get code 0).  Entries of blocks the kernel skips are left
 * untouched.  Limited to B*H*S*S <= 2^28. */
int attn_fwd_causal_fp8_debug(const void* q, const void* k, const void* v, void* out, float* lse,
                              float q_descale, float k_descale, float v_descale, float softmax_scale, int B,
                              int H, int S, int d_qk, int d_v, uint8_t* dbg_o, uint8_t* dbg_codes, void* stream);

/* Test hook with the arguments of attn_fwd_causal_fp8_ex (key-major V, either P mode at
 * either head dimension) and the dumps of attn_fwd_causal_fp8_debug, plus, when dbg_scores
 * is not NULL, the raw fp32 score s of every (b, h, query row, key) of every block the
 * kernel processes, as the score MFMA left it and before the causal mask
 * (dbg_scores: [B*H*S][S] floats, 16-byte aligned; entries of skipped blocks are left
 * untouched).  These are the kernel's inputs to the decisions of paper Sec. IV-A (running
 * maximum, lazy rescale), Sec. IV-B1 (the codes) and Sec. IV-B2 (the exponents o), so a
 * test can re-run those decisions on them.  The outputs equal attn_fwd_causal_fp8_ex's
 * bit for bit.  Limited to B*H*S*S <= 2^28. */
int attn_fwd_causal_fp8_debug_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                                 float q_descale, float k_descale, float v_descale, float softmax_scale, int B,
                                 int H, int H_kv, int S, int d_qk, int d_v, const attn_strides* q_strides,
                                 const attn_strides* k_strides, const attn_strides* v_strides,
                                 const attn_strides* out_strides, int p_mode, uint8_t* dbg_o, uint8_t* dbg_codes,
                                 float* dbg_scores, void* stream);

/* Host-only helpers (no device call), for schedule inspection and tests (ZYFA paper,
 * Sec. IV-A: causal pairing, persistent grid, chiplet placement).
 * attn_default_grid: the persistent grid the attention entry points launch for a
 *   problem with H query and H_kv key/value heads on a device with num_cu compute
 *   units: min(num_cu, work items).
 * attn_schedule: writes, in execution order, one (workgroup, b, h, first query row,
 *   rows) record of five int32 per query tile and head that the grid of `grid`
 *   workgroups processes.  When H / H_kv is even the kernels run the head-pair mode
 *   (Sec. IV-A: a pair covers two query heads with tiles of half the size): a tile is
 *   128 rows of heads 2u and 2u+1, recorded as two consecutive records; otherwise a
 *   tile is 256 rows of one head.  Returns the number of records (B*H*S/rows), or a
 *   negative attn_status if `cap` records do not fit or the sizes are invalid. */
int attn_default_grid(int B, int H, int H_kv, int S, int num_cu);
int64_t attn_schedule(int B, int H, int H_kv, int S, int grid, int32_t* records, int64_t cap);

/* Human-readable name of a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_CAUSAL_H */
