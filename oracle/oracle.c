/*
 * CPU oracle for causal attention forward (prefill) with FP8 e4m3 or BF16 operands.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or constant with the GPU library; both are written independently from the
 * same source: "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4"
 * (Anthony, Bikshandi, Medepalli, Ebert; arXiv:2611.07496).
 *
 * Plain, slow and obviously correct: scalar loops, fp64 wherever the paper leaves
 * the precision free, and fp32 (with fmaf) exactly where the emulation mirrors the
 * fp32 arithmetic of the kernel it checks.  Build with -O2 -ffp-contract=off and
 * without -ffast-math.  OpenMP only distributes independent rows / row groups.
 *
 * Contents
 *   orc_e4m3_value      decode one e4m3 (OCP "fn") code          paper Sec. II-C, fn 5
 *   orc_e4m3_rne        round a real to e4m3, nearest-even, saturating to +-448
 *   orc_bf16_rne        round an fp32 to bf16, nearest-even
 *   orc_quantize_e4m3   per-tensor power-of-two scaled quantiser   paper Sec. V-E, fn 17
 *   orc_quantize_e4m3_f64  the same quantiser on fp64 inputs (rotated Q, K; Sec. V-E)
 *   orc_leanp_code      lean-P code of x = log2 p (ideal, fp64)    paper Sec. IV-B1, Eq. 2
 *   orc_exactp_code     exact-P code of x (round 2^(x+sigma))      paper Sec. IV-B1
 *   orc_attn_exact      exact causal softmax attention in fp64     paper Sec. II-B (definition)
 *   orc_emulate_fp8     step-by-step emulation of the FP8 scheme   paper Sec. IV-A/IV-B
 *   orc_emulate_fp8_scores  the same scheme from given fp32 scores (checks of a kernel's
 *                       decisions given its own scores; not a parity reference)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_LOG2E 1.4426950408889634074
#define ORC_LN2 0.69314718055994530942

/* ------------------------------------------------------------------------- */
/* e4m3 (OCP "fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities; the two codes with all exponent and mantissa bits set are
 * NaN; the largest finite magnitude is 448 (paper Sec. II-C).  A normal value is
 * (1 + F/8) 2^(E-7); exponent field 0 holds the subnormals (F/8) 2^-6, spaced 2^-9
 * apart (paper Sec. II-C, footnote 5).                                       */
double orc_e4m3_value(int code) {
  code &= 0xFF;
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int f = code & 0x7;
  double mag;
  if (e == 0xF && f == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)f / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)f / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Round a real number to the nearest e4m3 value; ties go to the code with an even
 * mantissa (the default IEEE rounding).  Magnitudes beyond the largest finite value
 * saturate to 448.  Written as a search over the ordered positive codes so that it
 * follows the definition rather than any bit trick.  NaN maps to 0x7F.          */
int orc_e4m3_rne(double x) {
  if (isnan(x)) return 0x7F;
  int neg = signbit(x) ? 1 : 0;
  double a = fabs(x);
  int lo = 0; /* largest code with value <= a, codes 0..126 are increasing */
  for (int c = 1; c <= 126; ++c) {
    if (orc_e4m3_value(c) <= a) lo = c; else break;
  }
  int code;
  if (lo == 126) {
    code = 126; /* saturate */
  } else {
    double vlo = orc_e4m3_value(lo), vhi = orc_e4m3_value(lo + 1);
    double dlo = a - vlo, dhi = vhi - a; /* exact: all values are dyadic with few bits */
    if (dlo < dhi) code = lo;
    else if (dhi < dlo) code = lo + 1;
    else code = (lo % 2 == 0) ? lo : lo + 1;
  }
  return code | (neg << 7);
}

/* fp32 -> bf16 (upper 16 bits of the fp32 pattern), nearest-even on the dropped
 * 16 bits.  Defined by comparing the two neighbouring bf16 values in fp64.      */
uint16_t orc_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lo_bits = u & 0xFFFF0000u;
  if (lo_bits == u) return (uint16_t)(u >> 16);
  uint32_t hi_bits = lo_bits + 0x10000u; /* next bf16 away from zero */
  float flo, fhi;
  memcpy(&flo, &lo_bits, 4);
  memcpy(&fhi, &hi_bits, 4);
  double dlo = fabs((double)x - (double)flo), dhi = fabs((double)fhi - (double)x);
  if (isinf(fhi)) dhi = INFINITY; /* only reachable at the very top of the range */
  if (dlo < dhi) return (uint16_t)(lo_bits >> 16);
  if (dhi < dlo) return (uint16_t)(hi_bits >> 16);
  return (uint16_t)((((lo_bits >> 16) & 1u) == 0) ? (lo_bits >> 16) : (hi_bits >> 16));
}

double orc_bf16_value(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Per-tensor power-of-two quantiser (paper Sec. V-E with footnote 17: per-call
 * scales from the absolute maximum, power-of-two descales).  Reading: the scale is
 * the largest power of two 2^k with amax * 2^k <= 448, so nothing saturates; k is
 * clamped to [-126, 126] so that the fp32 descale 2^-k is a normal number; an
 * all-zero tensor gets k = 0.  Returns the descale 2^-k (exact in fp32).       */
static int orc_pow2_exponent(double amax) {
  int k = 0;
  if (amax > 0.0) {
    k = (int)floor(log2(448.0 / amax));
    while (ldexp(amax, k) > 448.0) --k;       /* make sure nothing saturates */
    while (ldexp(amax, k + 1) <= 448.0) ++k;  /* and that 2^k is the largest such */
    if (k > 126) k = 126;
    if (k < -126) k = -126;
  }
  return k;
}

float orc_quantize_e4m3(const float* x, int64_t n, uint8_t* codes) {
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  const int k = orc_pow2_exponent(amax);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_rne(ldexp((double)x[i], k));
  return (float)ldexp(1.0, -k);
}

/* The same quantiser applied to fp64 values, for inputs the oracle itself computes in
 * fp64 (the rotated Q and K of paper Sec. V-E, "Rotation and K smoothing", whose FP8
 * scales come after the rotation). */
float orc_quantize_e4m3_f64(const double* x, int64_t n, uint8_t* codes) {
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double a = fabs(x[i]);
    if (a > amax) amax = a;
  }
  const int k = orc_pow2_exponent(amax);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_rne(ldexp(x[i], k));
  return (float)ldexp(1.0, -k);
}

/* Lean P on the ideal (fp64) path, paper Sec. IV-B1, Eq. 2: y = 8 (x + sigma + 7)
 * - beta, rounded to the nearest integer and clamped to [0, 255]; the integer is
 * used directly as the e4m3 code.  x = log2 p relative to the (scaled) maximum. */
int orc_leanp_code(double x, int sigma, double beta) {
  double y = 8.0 * (x + sigma + 7.0) - beta;
  double r = nearbyint(y); /* default rounding mode: nearest, ties to even */
  if (!(r >= 0.0)) r = 0.0;  /* negative and NaN clamp to 0 */
  if (r > 255.0) r = 255.0;
  return (int)r;
}

/* Exact P, paper Sec. IV-B1: evaluate 2^(x + sigma) and round it to e4m3. */
int orc_exactp_code(double x, int sigma) { return orc_e4m3_rne(exp2(x + (double)sigma)); }

/* ------------------------------------------------------------------------- */
/* Input element access.  Layout BSHD: element (b, s, h, d) of a tensor with
 * head dimension D sits at ((b*S + s)*H + h)*D + d.  dtype 0 = e4m3 codes
 * (value = decoded code * descale), dtype 1 = bf16 bit patterns.           */
static double g_e4m3[256];
static int g_e4m3_ready = 0;
static void orc_init_tables(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 256; ++c) g_e4m3[c] = orc_e4m3_value(c);
  g_e4m3_ready = 1;
}

static inline double elem(int dtype, const void* base, int64_t idx) {
  if (dtype == 0) return g_e4m3[((const uint8_t*)base)[idx]];
  return orc_bf16_value(((const uint16_t*)base)[idx]);
}

static inline int64_t bshd(int b, int s, int h, int d, int S, int H, int D) {
  return (((int64_t)b * S + s) * H + h) * (int64_t)D + d;
}

/* Exact causal softmax attention for selected rows, paper Sec. II-B:
 *   O_i = sum_{j<=i} exp(c q_i.k_j - M_i) v_j / sum_{j<=i} exp(c q_i.k_j - M_i)
 *   LSE_i = M_i + ln sum_{j<=i} exp(c q_i.k_j - M_i),  M_i = max_{j<=i} c q_i.k_j
 * all in fp64, on the values the kernel receives (decoded e4m3 times the
 * per-tensor descale, or bf16).  rows holds n_rows triples (b, h, i).
 * out: n_rows x dv (fp64, not rounded); lse: n_rows (natural log units).    */
int orc_attn_exact(int dtype, const void* q, const void* k, const void* v, double dq, double dk,
                   double dvs, double c, int B, int H, int S, int dqk, int dv, const int64_t* rows,
                   int64_t n_rows, double* out, double* lse) {
  orc_init_tables();
  if (dtype != 0) { dq = dk = dvs = 1.0; }
  int bad = 0;
#pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)S);
    double* qi = (double*)malloc(sizeof(double) * (size_t)dqk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
      if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      for (int d = 0; d < dqk; ++d) qi[d] = elem(dtype, q, bshd(b, i, h, d, S, H, dqk)) * dq;
      double mx = -INFINITY;
      for (int j = 0; j <= i; ++j) {
        double dot = 0.0;
        for (int d = 0; d < dqk; ++d) dot += qi[d] * (elem(dtype, k, bshd(b, j, h, d, S, H, dqk)) * dk);
        sc[j] = c * dot;
        if (sc[j] > mx) mx = sc[j];
      }
      double l = 0.0;
      for (int d = 0; d < dv; ++d) acc[d] = 0.0;
      for (int j = 0; j <= i; ++j) {
        double w = exp(sc[j] - mx);
        l += w;
        for (int d = 0; d < dv; ++d) acc[d] += w * (elem(dtype, v, bshd(b, j, h, d, S, H, dv)) * dvs);
      }
      for (int d = 0; d < dv; ++d) out[r * dv + d] = acc[d] / l;
      lse[r] = mx + log(l);
    }
    free(sc); free(qi); free(acc);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Step-by-step emulation of the FP8 scheme (paper Sec. IV-A lazy rescaling,
 * Sec. IV-B1 lean/exact P, Sec. IV-B2 per-64-key-block power-of-two scaling,
 * Sec. IV-B3 row sum of the rounded probabilities), for groups of consecutive
 * query rows.
 *
 * mirror mode (ideal == 0) repeats the fp32 decisions of a kernel that
 *   - computes raw fp32 scores s (the exact e4m3 dot product rounded once),
 *   - works in base-2 units t = s * cp, cp = fp32(c * dq * dk * log2 e),
 *   - visits keys from 0 upward in tiles of n_tile keys, and in each tile takes the
 *     new maximum M = max(m, max t); the first tile sets m = M; afterwards it keeps
 *     the stale m unless some row of the group grows by at least tau, in which case
 *     every row takes m = M and rescales acc and l by 2^(m_old - M);
 *   - per 64-key block: b = max visible t, o = clamp(floor(m - b), 0, 127);
 *   - lean P:  y = fmaf(s, 8 cp, 8 (sigma + 7 + o - m) - beta), code = rne(y) in
 *     [0, 255]; exact P: x = fmaf(s, cp, (sigma + o) - m), code = e4m3(2^x);
 *   - l += 2^-o sum p, acc += 2^-o sum p v  (fp64 here);
 *   - O = bf16(dv * acc / l), LSE = ln2 (m + log2 l - sigma).
 * ideal mode (ideal == 1) uses the exact final row maximum (no lazy trajectory)
 * and fp64 for t, m, b and y ("emulated with the exact row maximum", Sec. V-E).
 *
 * Options for the variants the paper contrasts (used by tests):
 *   scale_blocks == 0: no per-block scaling (o = 0 everywhere);
 *   rounded_sum  == 0: l sums the unrounded probabilities (exact 2^(x+sigma))
 *                      while the numerator uses the rounded ones.
 *
 * groups: n_groups triples (b, h, r0): rows r0 .. r0+group-1 (clipped to S).
 * out: n_groups*group*dv doubles (O before bf16 rounding, already * dv);
 * out_bf16: same count of bf16 patterns (may be NULL); lse: n_groups*group.
 * Optional debug (all may be NULL): o_dbg (n_groups*group*ceil(S/64) bytes, 255 for
 * blocks the row does not see), code_dbg (n_groups*group*S bytes, codes of visible
 * keys, 0 for masked), ymargin (n_groups*group*S floats: distance of the rounded
 * quantity from its rounding boundary), omargin (per (row, block): distance of
 * m - b from the nearest integer), lazy_margin (n_groups*ntiles: min over rows of
 * |(M - m) - tau| at each decision).                                          */
typedef struct {
  int n_tile;        /* keys per max update (128) */
  int group;         /* rows that share one lazy-rescale decision (32) */
  float tau;         /* lazy-rescale threshold, base-2 units */
  int sigma;         /* probability shift (6) */
  float beta;        /* lean-P bias (0.35) */
  int block;         /* keys per scale block (64) */
  int exact_p;       /* 0 lean P, 1 exact P */
  int ideal;         /* 0 mirror, 1 ideal */
  int scale_blocks;  /* 1 per-block scaling on */
  int rounded_sum;   /* 1 l from rounded probabilities */
} orc_fp8_params;

/* The walk itself; scores_in == NULL computes the raw scores from q and k (step 1 of the
 * scheme), otherwise row i of head (b, h) reads them from
 * scores_in[((b*H + h)*S + i)*S + j] (and q, k are not read).                 */
static int emulate_walk(const float* scores_in, const uint8_t* q, const uint8_t* k, const uint8_t* v,
                        float dq, float dk, float dvs, float c, int B, int H, int S, int dqk, int dv,
                        const orc_fp8_params* prm, const int64_t* groups, int64_t n_groups,
                        double* out, uint16_t* out_bf16, double* lse, uint8_t* o_dbg,
                        uint8_t* code_dbg, float* ymargin, float* omargin, float* lazy_margin) {
  orc_init_tables();
  const int G = prm->group, NT = prm->n_tile, BK = prm->block;
  const int nblk = (S + BK - 1) / BK;
  const int ntile = (S + NT - 1) / NT;
  if (NT % BK != 0 || G <= 0) return -3;
  /* fp32 constants of the mirrored arithmetic */
  const float cp = (float)((double)c * (double)dq * (double)dk * ORC_LOG2E);
  const float cp8 = 8.0f * cp;
  const double cp_d = (double)c * (double)dq * (double)dk * ORC_LOG2E;
  int bad = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)G * S);     /* exact raw scores */
    double* acc = (double*)malloc(sizeof(double) * (size_t)G * dv);
    double* l = (double*)malloc(sizeof(double) * (size_t)G);
    double* m = (double*)malloc(sizeof(double) * (size_t)G);      /* fp32 values in mirror */
    double* Mn = (double*)malloc(sizeof(double) * (size_t)G);
    double* qrow = (double*)malloc(sizeof(double) * (size_t)dqk);
    double* pv = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
    for (int64_t gi = 0; gi < n_groups; ++gi) {
      int b = (int)groups[3 * gi], h = (int)groups[3 * gi + 1], r0 = (int)groups[3 * gi + 2];
      if (b < 0 || b >= B || h < 0 || h >= H || r0 < 0 || r0 >= S) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int nr = G;
      if (r0 + nr > S) nr = S - r0;
      int last = r0 + nr - 1; /* last row of the group */
      /* raw scores: exact dot products of decoded codes (fits in fp64 exactly), or the
       * given fp32 scores */
      for (int r = 0; r < nr; ++r) {
        int i = r0 + r;
        if (scores_in) {
          const float* srow = scores_in + (((int64_t)b * H + h) * S + i) * (int64_t)S;
          for (int j = 0; j <= i; ++j) s[(size_t)r * S + j] = (double)srow[j];
        } else {
          for (int d = 0; d < dqk; ++d) qrow[d] = g_e4m3[q[bshd(b, i, h, d, S, H, dqk)]];
          for (int j = 0; j <= i; ++j) {
            double dot = 0.0;
            for (int d = 0; d < dqk; ++d) dot += qrow[d] * g_e4m3[k[bshd(b, j, h, d, S, H, dqk)]];
            s[(size_t)r * S + j] = dot;
          }
        }
        for (int d = 0; d < dv; ++d) acc[(size_t)r * dv + d] = 0.0;
        l[r] = 0.0;
      }
      /* ideal mode: exact final row maximum in base-2 units */
      if (prm->ideal) {
        for (int r = 0; r < nr; ++r) {
          int i = r0 + r;
          double mx = -INFINITY;
          for (int j = 0; j <= i; ++j) {
            double t = s[(size_t)r * S + j] * cp_d;
            if (t > mx) mx = t;
          }
          m[r] = mx;
        }
      }
      for (int ti = 0; ti * NT <= last; ++ti) {
        int k0 = ti * NT, k1 = k0 + NT; /* keys [k0, k1) */
        if (!prm->ideal) {
          /* new maximum per row over the visible keys of this tile (fp32) */
          for (int r = 0; r < nr; ++r) {
            int i = r0 + r;
            float M = (ti == 0) ? -INFINITY : (float)m[r];
            for (int j = k0; j < k1 && j <= i; ++j) {
              float t = (float)s[(size_t)r * S + j] * cp; /* fl32(fl32(s) * cp) */
              if (t > M) M = t;
            }
            Mn[r] = M;
          }
          if (ti == 0) {
            for (int r = 0; r < nr; ++r) m[r] = Mn[r];
          } else {
            int grow = 0;
            float minmargin = INFINITY;
            for (int r = 0; r < nr; ++r) {
              float dlt = (float)Mn[r] - (float)m[r];
              if (dlt >= prm->tau) grow = 1;
              float mg = fabsf(dlt - prm->tau);
              if (mg < minmargin) minmargin = mg;
            }
            if (lazy_margin) lazy_margin[gi * ntile + ti] = minmargin;
            if (grow) {
              for (int r = 0; r < nr; ++r) {
                double f = exp2((double)((float)m[r] - (float)Mn[r]));
                for (int d = 0; d < dv; ++d) acc[(size_t)r * dv + d] *= f;
                l[r] *= f;
                m[r] = Mn[r];
              }
            }
          }
        }
        /* the 64-key scale blocks of the tile */
        for (int kb = k0; kb < k1; kb += BK) {
          int blk = kb / BK;
          for (int r = 0; r < nr; ++r) {
            int i = r0 + r;
            int row = (int)(gi * G + r);
            if (o_dbg) o_dbg[(size_t)row * nblk + blk] = 255;
            if (kb > i) continue; /* no visible key: the block is skipped */
            int ke = kb + BK;
            if (ke > i + 1) ke = i + 1;
            int o = 0;
            if (prm->ideal) {
              double bmax = -INFINITY;
              for (int j = kb; j < ke; ++j) {
                double t = s[(size_t)r * S + j] * cp_d;
                if (t > bmax) bmax = t;
              }
              if (prm->scale_blocks) {
                double fo = floor(m[r] - bmax);
                o = fo < 0 ? 0 : (fo > 127 ? 127 : (int)fo);
                if (omargin) omargin[(size_t)row * nblk + blk] = (float)fabs((m[r] - bmax) - nearbyint(m[r] - bmax));
              }
            } else {
              float bmax = -INFINITY;
              for (int j = kb; j < ke; ++j) {
                float t = (float)s[(size_t)r * S + j] * cp;
                if (t > bmax) bmax = t;
              }
              if (prm->scale_blocks) {
                float dlt = (float)m[r] - bmax;
                float fo = floorf(dlt);
                o = fo < 0.0f ? 0 : (fo > 127.0f ? 127 : (int)fo);
                if (omargin) omargin[(size_t)row * nblk + blk] = fabsf(dlt - nearbyintf(dlt));
              }
            }
            if (o_dbg) o_dbg[(size_t)row * nblk + blk] = (uint8_t)o;
            double bs = 0.0, bs_unrounded = 0.0;
            for (int d = 0; d < dv; ++d) pv[d] = 0.0;
            for (int j = kb; j < ke; ++j) {
              int code;
              double mg;
              double xexact; /* log2 of the scaled probability, for the unrounded sum */
              if (prm->ideal) {
                double x = s[(size_t)r * S + j] * cp_d - m[r] + (double)o;
                xexact = x + prm->sigma;
                if (prm->exact_p) {
                  code = orc_exactp_code(x, prm->sigma);
                  mg = 0.0;
                } else {
                  double y = 8.0 * (x + prm->sigma + 7.0) - (double)prm->beta;
                  code = orc_leanp_code(x, prm->sigma, (double)prm->beta);
                  mg = fabs(y - floor(y) - 0.5);
                }
              } else {
                float sf = (float)s[(size_t)r * S + j];
                if (prm->exact_p) {
                  float cst = (float)(prm->sigma + o) - (float)m[r];
                  float x = fmaf(sf, cp, cst);
                  xexact = (double)x;
                  double p = exp2((double)x);
                  code = orc_e4m3_rne(p);
                  /* distance of p from the nearest e4m3 rounding boundary, relative */
                  double lo = orc_e4m3_value(code & 0x7F), nb;
                  nb = (p >= lo) ? orc_e4m3_value((code & 0x7F) + 1) : orc_e4m3_value((code & 0x7F) - 1);
                  mg = fabs(p - 0.5 * (lo + nb)) / (p > 0 ? p : 1.0);
                } else {
                  float cst = 8.0f * ((float)(prm->sigma + 7 + o) - (float)m[r]) - prm->beta;
                  float y = fmaf(sf, cp8, cst);
                  xexact = ((double)y + (double)prm->beta) / 8.0 - 7.0;
                  double rr = nearbyint((double)y);
                  if (!(rr >= 0.0)) rr = 0.0;
                  if (rr > 255.0) rr = 255.0;
                  code = (int)rr;
                  mg = fabs((double)y - floor((double)y) - 0.5);
                }
              }
              if (code >= 127) {
#pragma omp atomic write
                bad = 2; /* would be NaN or negative: impossible by construction */
              }
              if (code_dbg) code_dbg[(size_t)row * S + j] = (uint8_t)code;
              if (ymargin) ymargin[(size_t)row * S + j] = (float)mg;
              double p = g_e4m3[code];
              bs += p;
              bs_unrounded += exp2(xexact);
              for (int d = 0; d < dv; ++d) pv[d] += p * g_e4m3[v[bshd(b, j, h, d, S, H, dv)]];
            }
            double sc = ldexp(1.0, -o);
            l[r] += sc * (prm->rounded_sum ? bs : bs_unrounded);
            for (int d = 0; d < dv; ++d) acc[(size_t)r * dv + d] += sc * pv[d];
          }
        }
      }
      for (int r = 0; r < nr; ++r) {
        int64_t row = gi * G + r;
        for (int d = 0; d < dv; ++d) {
          double o_val = (double)dvs * acc[(size_t)r * dv + d] / l[r];
          out[row * dv + d] = o_val;
          if (out_bf16) out_bf16[row * dv + d] = orc_bf16_rne((float)o_val);
        }
        lse[row] = ORC_LN2 * (m[r] + log2(l[r]) - (double)prm->sigma);
      }
      for (int r = nr; r < G; ++r) {
        int64_t row = gi * G + r;
        for (int d = 0; d < dv; ++d) {
          out[row * dv + d] = NAN;
          if (out_bf16) out_bf16[row * dv + d] = 0x7FC0;
        }
        lse[row] = NAN;
      }
    }
    free(s); free(acc); free(l); free(m); free(Mn); free(qrow); free(pv);
  }
  return bad ? -bad : 0;
}

int orc_emulate_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, float dq, float dk,
                    float dvs, float c, int B, int H, int S, int dqk, int dv,
                    const orc_fp8_params* prm, const int64_t* groups, int64_t n_groups,
                    double* out, uint16_t* out_bf16, double* lse, uint8_t* o_dbg,
                    uint8_t* code_dbg, float* ymargin, float* omargin, float* lazy_margin) {
  return emulate_walk(NULL, q, k, v, dq, dk, dvs, c, B, H, S, dqk, dv, prm, groups, n_groups, out,
                      out_bf16, lse, o_dbg, code_dbg, ymargin, omargin, lazy_margin);
}

/* The same scheme from given raw fp32 scores instead of the exact dot products: steps
 * 2-6 (running maximum and lazy rescale, Sec. IV-A; o, Sec. IV-B2; codes, Sec. IV-B1;
 * rounded sums, Sec. IV-B3) on scores [B*H*S][S] (row (b*H + h)*S + i, only j <= i
 * read).  For checking a kernel's decisions given the scores it computed; the parity
 * gates use orc_emulate_fp8, whose scores are exact.                          */
int orc_emulate_fp8_scores(const float* scores, const uint8_t* v, float dq, float dk, float dvs,
                           float c, int B, int H, int S, int dv, const orc_fp8_params* prm,
                           const int64_t* groups, int64_t n_groups, double* out, uint16_t* out_bf16,
                           double* lse, uint8_t* o_dbg, uint8_t* code_dbg, float* ymargin,
                           float* omargin, float* lazy_margin) {
  if (!scores) return -4;
  return emulate_walk(scores, NULL, NULL, v, dq, dk, dvs, c, B, H, S, 0, dv, prm, groups, n_groups,
                      out, out_bf16, lse, o_dbg, code_dbg, ymargin, omargin, lazy_margin);
}

/* Bulk helpers used by tests. */
void orc_e4m3_rne_array(const double* x, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_rne(x[i]);
}
void orc_bf16_rne_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}
