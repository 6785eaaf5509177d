/*
 * Exact CPU re-quantizer NVFP4 -> sign-symmetric 2-bit planes (TEST INFRASTRUCTURE ONLY: used
 * by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg; never by the product).
 *
 * What it computes ("The v0.24.0 port", section "Our hooks", modelopt.py bullet; README opening
 * paragraph; plain readings where the pages are silent):
 *   x = e2m1 * e4m3[block of 16] * scale_2, exact (every factor is exactly representable and the
 *   product has at most 30 significant bits, so the f64 product the pages describe is exact).
 *   For every 32-element block along a row: choose the UE8M0 exponent e (2^e, e in -127..127) and
 *   for each element the magnitude q in {1, 4} that minimise the squared error
 *       SSE(e) = sum_i (|x_i| - q_i 2^e)^2 .
 *   For a fixed e each q_i is chosen independently: q_i = 4 iff |x_i| > 2.5 * 2^e (equal -> 1).
 *   Among exponents with equal SSE the lower one wins. The code is then
 *       negative x (sign bit set, -0 included): q=4 -> 0, q=1 -> 1;  otherwise q=1 -> 2, q=4 -> 3
 *   (code order {0,1,2,3} -> {-4,-1,1,4}), and the scale byte is e + 127.
 *
 * Exactness. |x_i| = N_i * 2^P_i with N_i = m2_i * S_j * F < 2^32 (m2 = twice the e2m1
 * magnitude, S_j the e4m3 significand, F the fp32 significand). Since sum |x_i|^2 does not depend
 * on e, SSE(e) is compared through
 *       D(e) = SSE(e) - sum |x_i|^2 = Q(e) 2^(2e) - 2^(e+1) A(e),
 *       Q(e) = sum q_i^2,   A(e) = sum q_i |x_i| ,
 * evaluated in 768-bit two's-complement integers after scaling by a power of two common to all
 * candidates, so every comparison is exact.
 *
 * Modes: window = 0 scans all 255 exponents; window = 1 scans only [top-6, top] (top =
 * ceil(log2 max|x|), clamped to -127..127). The tests check that both agree.
 */
#include <stdint.h>
#include <string.h>

#define NL 12 /* 64-bit limbs: 768 bits */

typedef struct { uint64_t w[NL]; } big_t; /* two's complement, little-endian limbs */

static void big_zero(big_t* a) { memset(a, 0, sizeof(*a)); }

/* a = v << s (v < 2^64, 0 <= s, result must fit) */
static void big_from_shifted(big_t* a, uint64_t v, int s) {
  big_zero(a);
  int limb = s / 64, bit = s % 64;
  if (limb < NL) a->w[limb] = v << bit;
  if (bit && limb + 1 < NL) a->w[limb + 1] = v >> (64 - bit);
}

static void big_add(big_t* r, const big_t* a, const big_t* b) {
  unsigned __int128 c = 0;
  for (int i = 0; i < NL; ++i) {
    c += (unsigned __int128)a->w[i] + b->w[i];
    r->w[i] = (uint64_t)c;
    c >>= 64;
  }
}

static void big_sub(big_t* r, const big_t* a, const big_t* b) {
  uint64_t borrow = 0;
  for (int i = 0; i < NL; ++i) {
    uint64_t ai = a->w[i], bi = b->w[i];
    uint64_t d = ai - bi - borrow;
    borrow = (ai < bi) || (ai - bi < borrow) ? 1 : 0;
    r->w[i] = d;
  }
}

/* signed compare: -1, 0, 1 */
static int big_cmp(const big_t* a, const big_t* b) {
  int sa = (int)(a->w[NL - 1] >> 63), sb = (int)(b->w[NL - 1] >> 63);
  if (sa != sb) return sa ? -1 : 1;
  for (int i = NL - 1; i >= 0; --i) {
    if (a->w[i] != b->w[i]) return a->w[i] < b->w[i] ? -1 : 1;
  }
  return 0;
}

static const int E2M1_TWICE_MAG[8] = {0, 1, 2, 3, 4, 6, 8, 12};

/* E4M3FN byte -> value = S * 2^P (S integer <= 15); returns -1 on NaN */
static int decode_e4m3(uint8_t b, uint64_t* S, int* P, int* neg) {
  int e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return -1;
  *neg = b >> 7;
  if (e == 0) { *S = (uint64_t)m; *P = -9; }      /* (m/8) 2^-6 */
  else { *S = (uint64_t)(8 + m); *P = e - 10; }   /* (1+m/8) 2^(e-7) */
  return 0;
}

/* fp32 -> value = F * 2^G; returns -1 on NaN/Inf */
static int decode_f32(float f, uint64_t* F, int* G, int* neg) {
  uint32_t u;
  memcpy(&u, &f, 4);
  int e = (u >> 23) & 255;
  uint32_t m = u & 0x7fffff;
  *neg = (int)(u >> 31);
  if (e == 255) return -1;
  if (e == 0) { *F = m; *G = -149; }
  else { *F = m | 0x800000u; *G = e - 150; }
  return 0;
}

/* N * 2^d > 5 for integer N >= 0 (exact) */
static int gt_five(uint64_t N, int d) {
  if (N == 0) return 0;
  if (d >= 3) return 1;               /* N*8 >= 8 > 5 */
  if (d >= 0) return (N << d) > 5;    /* N < 2^32 */
  if (d <= -40) return 0;             /* 5*2^40 > N */
  return N > ((uint64_t)5 << (-d));
}

/* floor(log2 v) for v > 0 */
static int ilog2(uint64_t v) { int r = -1; while (v) { v >>= 1; ++r; } return r; }

/*
 * The exact search of one 32-element block whose elements are |x_k| = N[k] * 2^P[k] (N < 2^32)
 * with sign flags neg[k]. Writes 8 canonical code bytes and the scale byte. Shared by every input
 * format: the format only decides how N, P and the sign come out of its bytes.
 */
static void requant_elems(const uint64_t* N, const int* P, const int* neg, int window, uint8_t* codes_out,
                          uint8_t* scale_out) {
  /* max |x| and top = ceil(log2 max|x|) */
  int any = 0, top = 0;
  for (int k = 0; k < 32; ++k) {
    if (!N[k]) continue;
    int l = ilog2(N[k]);
    int c = P[k] + l + ((N[k] & (N[k] - 1)) ? 1 : 0);   /* ceil(log2(N 2^P)) */
    if (!any || c > top) top = c;
    any = 1;
  }
  int best_e;
  if (!any) {
    best_e = -127; /* SSE = 32 * 4^e, strictly increasing in e */
  } else {
    int lo = -127, hi = 127;
    if (window) {
      lo = top - 6; hi = top;
      if (lo < -127) lo = -127;
      if (lo > 127) lo = 127;
      if (hi < -127) hi = -127;
      if (hi > 127) hi = 127;
    }
    /* common scale: D(e) * 2^-Z with Z below every term's exponent */
    int Pmin = P[0];
    for (int k = 1; k < 32; ++k) if (P[k] < Pmin) Pmin = P[k];
    int Z = -254;
    if (Pmin - 126 < Z) Z = Pmin - 126;
    big_t best, cur, t1, t2, acc;
    int have = 0;
    best_e = lo;
    for (int e = lo; e <= hi; ++e) {
      /* A(e) 2^-(Pmin) as a big integer, Q(e) as an integer */
      big_zero(&acc);
      uint64_t Q = 0;
      for (int k = 0; k < 32; ++k) {
        int q = gt_five(N[k], P[k] - e + 1) ? 4 : 1;
        Q += (uint64_t)(q * q);
        big_from_shifted(&t1, N[k] * (uint64_t)q, P[k] - Pmin);
        big_add(&acc, &acc, &t1);
      }
      /* term1 = Q 2^(2e - Z); term2 = A' 2^(e + 1 + Pmin - Z) with A' = acc */
      big_from_shifted(&t1, Q, 2 * e - Z);
      int s2 = e + 1 + Pmin - Z;
      /* shift acc left by s2 */
      big_zero(&t2);
      {
        int limb = s2 / 64, bit = s2 % 64;
        for (int i = NL - 1; i >= 0; --i) {
          uint64_t v = 0;
          int src = i - limb;
          if (src >= 0) v = acc.w[src] << bit;
          if (bit && src - 1 >= 0) v |= acc.w[src - 1] >> (64 - bit);
          t2.w[i] = v;
        }
      }
      big_sub(&cur, &t1, &t2);
      if (!have || big_cmp(&cur, &best) < 0) { best = cur; best_e = e; have = 1; }
    }
  }
  memset(codes_out, 0, 8);
  for (int k = 0; k < 32; ++k) {
    int q4 = gt_five(N[k], P[k] - best_e + 1);
    int c = neg[k] ? (q4 ? 0 : 1) : (q4 ? 3 : 2);
    codes_out[k / 4] |= (uint8_t)(c << (2 * (k % 4)));
  }
  *scale_out = (uint8_t)(best_e + 127);
}

/*
 * One NVFP4 block. e2m1: 16 bytes (low nibble = even element), e4m3: 2 bytes (one per 16
 * elements), scale2 decoded as F * 2^G with sign neg2.
 */
static int requant_block(const uint8_t* e2m1, const uint8_t* e4m3, uint64_t F, int G, int neg2,
                         int window, uint8_t* codes_out, uint8_t* scale_out) {
  uint64_t N[32];
  int P[32], neg[32];
  for (int j = 0; j < 2; ++j) {
    uint64_t S; int Pe, negs;
    if (decode_e4m3(e4m3[j], &S, &Pe, &negs)) return -1;
    for (int i = 0; i < 16; ++i) {
      int k = 16 * j + i;
      int nib = (e2m1[k / 2] >> (4 * (k & 1))) & 15;
      N[k] = (uint64_t)E2M1_TWICE_MAG[nib & 7] * S * F;   /* < 12*15*2^24 < 2^32 */
      P[k] = Pe + G - 1;                                    /* the -1 undoes the doubling */
      neg[k] = ((nib >> 3) & 1) ^ negs ^ neg2;
    }
  }
  requant_elems(N, P, neg, window, codes_out, scale_out);
  return 0;
}

/*
 * FP8 block-quant input ("The v0.24.0 port", section "Our hooks", fp8.py bullet: fp8 weights
 * with fp32 scales per 128 x 128 block, re-quantized in float64 math): x = e4m3 * scale, exact
 * (4 + 24 significant bits). One 32-element block of a row: 32 e4m3 bytes and the fp32 scale of
 * its 128 x 128 block.
 */
static int requant_block_fp8(const uint8_t* e4m3, float scale, int window, uint8_t* codes_out, uint8_t* scale_out) {
  uint64_t F; int G, negs;
  if (decode_f32(scale, &F, &G, &negs)) return -1;
  uint64_t N[32];
  int P[32], neg[32];
  for (int k = 0; k < 32; ++k) {
    uint64_t S; int Pe, ne;
    if (decode_e4m3(e4m3[k], &S, &Pe, &ne)) return -1;
    N[k] = S * F;            /* < 15 * 2^24 */
    P[k] = Pe + G;
    neg[k] = ne ^ negs;
  }
  requant_elems(N, P, neg, window, codes_out, scale_out);
  return 0;
}

/*
 * MXFP4 input (the FP4 checkpoints' experts; README: "FP4 experts ... codes remap"): x = e2m1 *
 * 2^(b-127) with one UE8M0 byte b per 32 elements, exact. Byte 255 (NaN) is rejected.
 */
static int requant_block_mxfp4(const uint8_t* e2m1, uint8_t b, int window, uint8_t* codes_out, uint8_t* scale_out) {
  if (b == 255) return -1;
  uint64_t N[32];
  int P[32], neg[32];
  for (int k = 0; k < 32; ++k) {
    int nib = (e2m1[k / 2] >> (4 * (k & 1))) & 15;
    N[k] = (uint64_t)E2M1_TWICE_MAG[nib & 7];
    P[k] = (int)b - 127 - 1;
    neg[k] = (nib >> 3) & 1;
  }
  requant_elems(N, P, neg, window, codes_out, scale_out);
  return 0;
}

/* fp8 block-quant rows of one tensor: e4m3 [nrows][C], scales [nrows/128][C/128] (fp32) ->
   codes [nrows][C/4], scales_out [nrows][C/32] */
int oracle_fp8_block128_rows(int64_t nrows, int64_t C, int64_t row0, const uint8_t* e4m3, const float* scales,
                             uint8_t* codes, uint8_t* scales_out, int window, int nthreads) {
  if (C % 128) return -2;
  int64_t nb = nrows * (C / 32);
  int err = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(|:err)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t r = b / (C / 32), c32 = b % (C / 32);
    float sc = scales[((row0 + r) / 128) * (C / 128) + (32 * c32) / 128];
    err |= requant_block_fp8(e4m3 + 32 * b, sc, window, codes + 8 * b, scales_out + b) ? 1 : 0;
  }
  return err ? -1 : 0;
}

/* MXFP4 rows: e2m1 [nrows][C/2], ue8m0 [nrows][C/32] -> codes [nrows][C/4], scales_out [nrows][C/32] */
int oracle_mxfp4_rows(int64_t nrows, int64_t C, const uint8_t* e2m1, const uint8_t* ue8m0, uint8_t* codes,
                      uint8_t* scales_out, int window, int nthreads) {
  if (C % 32) return -2;
  int64_t nb = nrows * (C / 32);
  int err = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(|:err)
  for (int64_t b = 0; b < nb; ++b)
    err |= requant_block_mxfp4(e2m1 + 16 * b, ue8m0[b], window, codes + 8 * b, scales_out + b) ? 1 : 0;
  return err ? -1 : 0;
}

int oracle_requant_block(const uint8_t* e2m1_16, const uint8_t* e4m3_2, float scale2,
                         uint8_t* codes_8, uint8_t* scale_byte, int window) {
  uint64_t F; int G, neg2;
  if (decode_f32(scale2, &F, &G, &neg2)) return -1;
  return requant_block(e2m1_16, e4m3_2, F, G, neg2, window, codes_8, scale_byte);
}

/* rows of one tensor: e2m1 [nrows][C/2], e4m3 [nrows][C/16] -> codes [nrows][C/4], scales [nrows][C/32] */
int oracle_requant_rows(int64_t nrows, int64_t C, const uint8_t* e2m1, const uint8_t* e4m3,
                        float scale2, uint8_t* codes, uint8_t* scales, int window, int nthreads) {
  if (C % 32) return -2;
  uint64_t F; int G, neg2;
  if (decode_f32(scale2, &F, &G, &neg2)) return -1;
  int64_t nb = nrows * (C / 32);
  int err = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(|:err)
  for (int64_t b = 0; b < nb; ++b) {
    err |= requant_block(e2m1 + 16 * b, e4m3 + 2 * b, F, G, neg2, window, codes + 8 * b, scales + b) ? 1 : 0;
  }
  return err ? -1 : 0;
}
