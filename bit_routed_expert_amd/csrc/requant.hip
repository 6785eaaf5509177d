// nvfp4_to_w2: load-time re-quantizer NVFP4 -> sign-symmetric 2-bit planes.
//
// "The v0.24.0 port", section "Our hooks", modelopt.py bullet: modelopt NVFP4 experts (e2m1
// codes, f8e4m3 scales per 16 elements, fp32 per-tensor weight_scale_2) are dequantized exactly
// and re-quantized to the codebook {-4,-1,1,4}; the UE8M0 block-32 output scales absorb scale_2.
//
// One thread per 32-element block. Every element is held exactly as N * 2^P with N < 2^32
// (N = twice the e2m1 magnitude m2 x the e4m3 significand x the fp32 significand; the last two
// are one factor SF per half-block), so the squared error comparisons are exact integer
// arithmetic, never rounded:
//   D(e) = SSE(e) - sum|x|^2 = Q(e) 4^e - 2^(e+1) A(e),  Q = sum q^2,  A = sum q |x|,
// and the optimum lies in [top-6, top] with top = ceil(log2 max|x|): above top every magnitude
// is 1 and the error grows with e; below max|x|/37 doubling the step always lowers the error.
// An element takes magnitude 4 at exponent e exactly when |x| > 2.5 * 2^e, i.e. when e is below
// its threshold t = P + floor(log2 N) - 1 + [4N > 5 * 2^floor(log2 N)] (ties go to 1), so each
// candidate needs only the per-half sums of m2 over the elements above it.
#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

__device__ __forceinline__ int ilog2_u32(uint32_t v) { return 31 - __clz(v); }  // v > 0

// Per half-block the search works on magnitude classes instead of elements: the 16 elements share
// SF and P, so an element's threshold depends only on its e2m1 magnitude class m (m2 = 1, 2, 3,
// 4, 6, 8, 12 for m = 1..7; class 0 is zero and never takes magnitude 4). The thresholds rise with
// m and come in two runs: m2 = 2^a (classes 1, 2, 4, 6) gives T1 + a, m2 = 3 * 2^a (classes 3, 5,
// 7) gives T3 + a, with T1, T3 from SF and 3 SF alone. At a candidate e the elements taking
// magnitude 4 are therefore those of class >= m*(e) = 1 + #{classes with threshold <= e}, and the
// counts and m2 sums over such suffixes of classes are tabulated once per half (counts by a
// compare on all 8 nibbles of a word at once). The candidate scores are exact in 64 bits: the
// scaled terms stay below 2^61 (top - min P <= 46, |P0 - P1| <= 14).
__device__ __forceinline__ uint32_t byte_at(uint32_t lo, uint32_t hi, int i) {   // byte i (0..7) of hi:lo
  return __builtin_amdgcn_ubfe(i < 4 ? lo : hi, 8 * (i & 3), 8);
}
// number of nibbles of w whose low three bits are >= m (1 <= m <= 8)
__device__ __forceinline__ int nibbles_ge(uint32_t y, int m) {
  return __popc((y + (uint32_t)(8 - m) * 0x11111111u) & 0x88888888u);
}
// 2-bit codes of 8 elements (nibbles of w): sign from bit 3 (flipped by nsg), magnitude 4 for the
// classes >= ms; code = 2 (+1), 3 (+4), 1 (-1), 0 (-4), element i at bits 2i..2i+1
__device__ __forceinline__ uint32_t word_codes(uint32_t w, uint32_t nsg, int ms) {
  const uint32_t negw = (w ^ (nsg ? 0x88888888u : 0u)) & 0x88888888u;
  const uint32_t q4w = ((w & 0x77777777u) + (uint32_t)(8 - ms) * 0x11111111u) & 0x88888888u;
  uint32_t x = ((~negw & 0x88888888u) >> 2) | ((q4w ^ negw) >> 3);
  x = (x | (x >> 2)) & 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0x0000FFFFu;
}

__global__ void __launch_bounds__(256)
nvfp4_to_w2_kernel(long long nblocks, long long blocks_per_tensor,
                   const uint8_t* __restrict__ e2m1, const uint8_t* __restrict__ e4m3,
                   const float* __restrict__ scale_2, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales, int32_t* __restrict__ flag) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const long long tensor = b / blocks_per_tensor;
  // fp32 scale_2 = F * 2^G
  const uint32_t su = __builtin_bit_cast(uint32_t, scale_2[tensor]);
  const int sexp = (su >> 23) & 255;
  const uint32_t neg2 = su >> 31;
  uint32_t F;
  int G;
  if (sexp == 255) { atomicOr(flag, 1); *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{0, 0}; scales[b] = 0; return; }
  if (sexp == 0) { F = su & 0x7fffffu; G = -149; } else { F = (su & 0x7fffffu) | 0x800000u; G = sexp - 150; }
  // e4m3 per half: significand S (<= 15) and exponent
  const uint16_t sb = *reinterpret_cast<const uint16_t*>(e4m3 + 2 * b);
  const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(e2m1 + 16 * b);
  constexpr int kNone = -100000;
  constexpr int kLow = -(1 << 20);   // thresholds of a half whose scale is zero: below every candidate
  uint32_t SF[2], nsg[2], cl[2], ch[2], sl[2], sh[2], tot[2];
  int P[2], T1[2], T3[2];
  int top = kNone;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t byte = (sb >> (8 * j)) & 0xffu;
    const int ex = (byte >> 3) & 15, mt = byte & 7;
    if (ex == 15 && mt == 7) { atomicOr(flag, 1); *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{0, 0}; scales[b] = 0; return; }
    uint32_t S;
    int pe;
    if (ex == 0) { S = mt; pe = -9; } else { S = 8 + mt; pe = ex - 10; }
    SF[j] = S * F;               // < 2^28
    P[j] = pe + G - 1;           // the -1 undoes the doubled e2m1 magnitude
    nsg[j] = (byte >> 7) ^ neg2;
    // suffix counts c[m] (elements of class >= m) and m2 sums s[m], m = 1..8, as bytes m - 1
    const uint32_t y0 = raw[2 * j] & 0x77777777u, y1 = raw[2 * j + 1] & 0x77777777u;
    int c[9], sm[9];
    c[8] = 0;
    sm[8] = 0;
#pragma unroll
    for (int m = 7; m >= 1; --m) {
      c[m] = nibbles_ge(y0, m) + nibbles_ge(y1, m);
      const int m2 = m == 1 ? 1 : m == 2 ? 2 : m == 3 ? 3 : m == 4 ? 4 : m == 5 ? 6 : m == 6 ? 8 : 12;
      sm[m] = sm[m + 1] + (c[m] - c[m + 1]) * m2;
    }
    cl[j] = (uint32_t)c[1] | (uint32_t)c[2] << 8 | (uint32_t)c[3] << 16 | (uint32_t)c[4] << 24;
    ch[j] = (uint32_t)c[5] | (uint32_t)c[6] << 8 | (uint32_t)c[7] << 16;
    sl[j] = (uint32_t)sm[1] | (uint32_t)sm[2] << 8 | (uint32_t)sm[3] << 16 | (uint32_t)sm[4] << 24;
    sh[j] = (uint32_t)sm[5] | (uint32_t)sm[6] << 8 | (uint32_t)sm[7] << 16;
    tot[j] = (uint32_t)sm[1];
    if (SF[j] == 0) {
      T1[j] = T3[j] = kLow;
    } else {
      const uint32_t s3 = 3u * SF[j];
      const int L1 = ilog2_u32(SF[j]), L3 = ilog2_u32(s3);
      T1[j] = P[j] - 1 + L1 + (4ull * SF[j] > (5ull << L1) ? 1 : 0);
      T3[j] = P[j] - 1 + L3 + (4ull * s3 > (5ull << L3) ? 1 : 0);
      // the half's largest magnitude: its highest class present
      const int mhi = (c[1] > 0) + (c[2] > 0) + (c[3] > 0) + (c[4] > 0) + (c[5] > 0) + (c[6] > 0) + (c[7] > 0);
      if (mhi > 0) {
        const uint32_t m2 = (uint32_t)((0x0C08060403020100ull >> (8 * mhi)) & 0xff);
        const uint32_t N = m2 * SF[j];
        const int L = ilog2_u32(N);
        const int ct = P[j] + L + ((N & (N - 1)) ? 1 : 0);
        top = ct > top ? ct : top;
      }
    }
  }
  // first class taking magnitude 4 at exponent e, per half
  auto mstar = [&](int j, int e) {
    return 1 + min(max(e - T1[j] + 1, 0), 4) + min(max(e - T3[j] + 1, 0), 3);
  };
  int best = -127;
  if (top != kNone) {
    const int lo = max(-127, min(127, top - 6));
    const int hi = max(-127, min(127, top));
    const int Pm = min(P[0], P[1]);
    const int Z = min(2 * lo, lo + 1 + Pm);
    long long best_v = 0;
    for (int e = lo; e <= hi; ++e) {
      const int m0 = mstar(0, e) - 1, m1 = mstar(1, e) - 1;
      const int n4 = (int)(byte_at(cl[0], ch[0], m0) + byte_at(cl[1], ch[1], m1));
      const uint64_t A0 = (uint64_t)SF[0] * (tot[0] + 3u * byte_at(sl[0], sh[0], m0));
      const uint64_t A1 = (uint64_t)SF[1] * (tot[1] + 3u * byte_at(sl[1], sh[1], m1));
      const uint64_t A = (A0 << (P[0] - Pm)) + (A1 << (P[1] - Pm));
      // D(e) = Q 2^(2e) - A 2^(e+1+Pm), scaled by 2^-Z with Z below both exponents for every
      // candidate, so both shifts are non-negative and every value is an exact integer
      const uint64_t Q = 32u + 15u * (uint32_t)n4;
      const long long v = (long long)(Q << (2 * e - Z)) - (long long)(A << (e + 1 + Pm - Z));
      if (e == lo || v < best_v) { best_v = v; best = e; }
    }
  }
  const int ms0 = top != kNone ? mstar(0, best) : 8, ms1 = top != kNone ? mstar(1, best) : 8;
  const uint32_t c0 = word_codes(raw[0], nsg[0], ms0) | word_codes(raw[1], nsg[0], ms0) << 16;
  const uint32_t c1 = word_codes(raw[2], nsg[1], ms1) | word_codes(raw[3], nsg[1], ms1) << 16;
  *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{c0, c1};
  scales[b] = (uint8_t)(best + 127);
}

// ------------------------------------------------------------------------------------------------
// FP8 block-quant and MXFP4 inputs ("The v0.24.0 port", section "Our hooks", fp8.py bullet: fp8
// weights with fp32 scales per 128 x 128 block re-quantized to the sign-symmetric codebook in
// float64 math; README: the FP8 block-quant and FP4 checkpoint flavours load). The same exact
// search, with every element's own exponent: |x_k| = N_k * 2^P_k (N_k < 2^28), each element
// aligned to the block's smallest exponent Pm in 64 bits (a_k = N_k << (P_k - Pm), the exponents
// of one block differ by at most 14 for fp8 and not at all for MXFP4, so a_k < 2^42):
//   D(e) 2^-Z = Q(e) 2^(2e - Z) - A(e) 2^(e + 1 + Pm - Z),  Q = 32 + 15 n4(e),
//   A(e) = sum a_k + 3 * sum over {t_k > e} a_k,
// with the same thresholds t_k and window [top-6, top] as above. Each format's structure shrinks
// the per-candidate work: FP8 blocks share the scale's significand, MXFP4 blocks also the exponent.
// ------------------------------------------------------------------------------------------------

// Candidate exponents [top-6, top] of a block (clamped to [-127, 127]) scored by D(e) 2^-Z, ties
// to the lower exponent, from per-candidate sums: n4(e) elements above their threshold and a4(e)
// the sum of their a_k / F. SUMS(e, n4, a4) computes them; A = F (tot + 3 a4) in units of 2^Pm.
template <class V = __int128, class Sums>
__device__ int best_exponent(int top, int Pm, uint64_t F, uint64_t tot, Sums sums) {
  const int lo = max(-127, min(127, top - 6));
  const int hi = max(-127, min(127, top));
  const int Z = min(2 * lo, lo + 1 + Pm);
  V best_v = 0;
  int best = lo;
  for (int e = lo; e <= hi; ++e) {
    uint32_t n4;
    uint64_t a4;
    sums(e, n4, a4);
    const V A = (V)(F * (tot + 3ull * a4));
    const V Q = 32 + 15 * (int)n4;
    const V v = (Q << (2 * e - Z)) - (A << (e + 1 + Pm - Z));
    if (e == lo || v < best_v) { best_v = v; best = e; }
  }
  return best;
}

// fp8 e4m3 [n][R][C] with fp32 scales [n][R/128][C/128]: one thread per 32-element block. The
// block's scale significand F is common to its elements, and every element's exponent P_k is at
// least G - 9 (the e4m3 subnormal exponent under the block scale), so a_k = F * (S_k << (P_k -
// G + 9)) in units of 2^(G-9), with the e4m3 significand S_k <= 15 and P_k - G + 9 <= 14: the
// per-candidate sums run in 32 bits over S_k << (P_k - G + 9) (< 2^18 each, < 2^23 over the block)
// with the count packed in bits 24 up. Each element takes magnitude 4 at the candidates lo + i
// with i < d = clamp(t - lo, 0, 7), so it is added once, to bucket d of its thread (LDS,
// bucket-major so that the lanes of a wave hit distinct banks), and candidate i reads the sum of
// the buckets above i. The scores are exact in 64 bits: A = F (tot + 3 a4) < 2^49 and the scaled
// terms stay below 2^57.
constexpr int kFp8Threads = 256;
__global__ void __launch_bounds__(kFp8Threads)
fp8_block128_to_w2_kernel(long long nblocks, int R, int C, const uint8_t* __restrict__ e4m3,
                          const float* __restrict__ bscale, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                          int32_t* __restrict__ flag) {
  __shared__ uint32_t bucket[8][kFp8Threads];   // this thread's column only: no barriers
  const int tid = threadIdx.x;
  const long long b = (long long)blockIdx.x * blockDim.x + tid;
  if (b >= nblocks) return;
  const int nb_row = C / 32;
  const long long row = b / nb_row;           // row over all tensors
  const int c32 = (int)(b - row * nb_row);
  const long long tensor = row / R;
  const int r = (int)(row - tensor * R);
  const float sc = bscale[(tensor * (R / 128) + r / 128) * (C / 128) + c32 / 4];
  const uint32_t su = __builtin_bit_cast(uint32_t, sc);
  const int sexp = (su >> 23) & 255;
  const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(e4m3 + 32 * b);
  const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(e4m3 + 32 * b + 16);
  const uint32_t wd[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  // NaN bytes (0x7f / 0xff) and the sign bits, four bytes at a time
  bool nan = sexp == 255;
  uint32_t neg = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t x = (wd[q] & 0x7f7f7f7fu) ^ 0x7f7f7f7fu;            // zero byte <=> NaN
    nan |= ((x - 0x01010101u) & ~x & 0x80808080u) != 0u;
    const uint32_t sg = (wd[q] >> 7) & 0x01010101u;                      // sign of byte i at bit 8i
    neg |= ((sg * 0x00204081u) >> 21 & 0xfu) << (4 * q);                 // bits 21..24: bytes 0..3
  }
  if (nan) { atomicOr(flag, 1); *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{0, 0}; scales[b] = 0; return; }
  if (su >> 31) neg = ~neg;
  const uint32_t F = sexp ? ((su & 0x7fffffu) | 0x800000u) : (su & 0x7fffffu);
  const int G = sexp ? sexp - 150 : -149;
  constexpr int kNone = -100000;
  int t[32];
  int top = kNone;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t byte = (wd[k >> 2] >> (8 * (k & 3))) & 0xffu;
    const int ex = (byte >> 3) & 15, mt = byte & 7;
    const uint32_t N = (ex ? 8u + mt : (uint32_t)mt) * F;   // < 2^28, so 4N and 5 * 2^L fit 32 bits
    const int P = (ex ? ex - 10 : -9) + G;
    // branch-free: a zero N gets the threshold kNone and no say in top
    const int L = ilog2_u32(N | 1u);
    const int tk = P + L - 1 + (4u * N > (5u << L) ? 1 : 0);
    const int c = P + L + ((N & (N - 1)) ? 1 : 0);
    t[k] = N ? tk : kNone;
    top = max(top, N ? c : kNone);
  }
  int best = -127;
  if (top != kNone) {
    const int lo = max(-127, min(127, top - 6));
    const int hi = max(-127, min(127, top));
    const int Pr = G - 9;                    // reference exponent, below every element's
    const int Z = min(2 * lo, lo + 1 + Pr);
#pragma unroll
    for (int d = 0; d < 8; ++d) bucket[d][tid] = 0u;
    uint32_t tot = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t byte = (wd[k >> 2] >> (8 * (k & 3))) & 0xffu;
      const int ex = (byte >> 3) & 15, mt = byte & 7;
      const uint32_t a = (ex ? 8u + mt : (uint32_t)mt) << (ex ? ex - 1 : 0);   // S << (P - Pr)
      tot += a;
      const int d = min(max(t[k] - lo, 0), 7);
      atomicAdd(&bucket[d][tid], a + (1u << 24));   // bucket 0: never magnitude 4 (unused)
    }
    // candidates from the top down; ties go to the lower exponent
    uint32_t acc = 0;
    long long best_v = 0;
#pragma unroll
    for (int i = 6; i >= 0; --i) {
      acc += bucket[i + 1][tid];
      const int e = lo + i;
      const uint64_t A = (uint64_t)F * (tot + 3ull * (acc & 0xffffffu));
      const uint64_t Q = 32u + 15u * (acc >> 24);
      if (e <= hi) {
        const long long v = (long long)(Q << (2 * e - Z)) - (long long)(A << (e + 1 + Pr - Z));
        if (e == hi || v <= best_v) { best_v = v; best = e; }
      }
    }
  }
  uint32_t c0 = 0, c1 = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const bool q4 = t[k] > best;
    const bool ng = (neg >> k) & 1u;
    const uint32_t c = ng ? (q4 ? 0u : 1u) : (q4 ? 3u : 2u);
    if (k < 16) c0 |= c << (2 * k); else c1 |= c << (2 * (k - 16));
  }
  *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{c0, c1};
  scales[b] = (uint8_t)(best + 127);
}

// MXFP4 e2m1 [n][R][C/2] with UE8M0 bytes [n][R][C/32]: one thread per 32-element block. Every
// element shares the exponent P = b - 128 and N = twice its e2m1 magnitude (0, 1, 2, 3, 4, 6, 8,
// 12 for magnitude index m = 0..7), so its threshold is P + d_m with d = -1, 0, 1, 1, 2, 2, 3 for
// m = 1..7 (from the formula above: L - 1 + [4N > 5 * 2^L]), rising with m: at a candidate e the
// elements taking magnitude 4 are those of index >= m*(e) = 1 + #{m : d_m <= e - P}. The suffix
// counts and m2 sums over m are tabulated once per block (counts by a compare on all 8 nibbles of
// a word at once) and each candidate reads one table entry; the final codes come from the same
// nibble compare. Every exponent lies within 6 below and 4 above P, so both shifts of the scores
// stay below 21 and the scores (< 2^31) fit in 64 bits.
__global__ void __launch_bounds__(256)
mxfp4_to_w2_kernel(long long nblocks, const uint8_t* __restrict__ e2m1, const uint8_t* __restrict__ ue8m0,
                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int32_t* __restrict__ flag) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int sb = ue8m0[b];
  if (sb == 255) { atomicOr(flag, 1); *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{0, 0}; scales[b] = 0; return; }
  const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(e2m1 + 16 * b);
  const int P = sb - 128;                     // 2^(b-127), halved
  uint32_t y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = raw[q] & 0x77777777u;
  // suffix counts c[m] and m2 sums s[m] (m = 1..8) of the indices >= m, as (c | s << 6) pairs,
  // two per word: entry m - 1 in bits 16 ((m - 1) & 1) of word (m - 1) >> 1
  int c[9], sm[9];
  c[8] = 0;
  sm[8] = 0;
#pragma unroll
  for (int m = 7; m >= 1; --m) {
    c[m] = nibbles_ge(y[0], m) + nibbles_ge(y[1], m) + nibbles_ge(y[2], m) + nibbles_ge(y[3], m);
    const int m2 = m == 1 ? 1 : m == 2 ? 2 : m == 3 ? 3 : m == 4 ? 4 : m == 5 ? 6 : m == 6 ? 8 : 12;
    sm[m] = sm[m + 1] + (c[m] - c[m + 1]) * m2;
  }
  uint32_t tab[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    tab[q] = ((uint32_t)c[2 * q + 1] | (uint32_t)sm[2 * q + 1] << 6) |
             ((uint32_t)c[2 * q + 2] | (uint32_t)sm[2 * q + 2] << 6) << 16;
  const int imax = (c[1] > 0) + (c[2] > 0) + (c[3] > 0) + (c[4] > 0) + (c[5] > 0) + (c[6] > 0) + (c[7] > 0);
  // #{m in 1..7 : d_m <= x} for x = -2 (or less) .. 3 (or more): 0, 1, 2, 4, 6, 7
  auto mstar = [&](int e) {
    const int x = min(max(e - P + 2, 0), 5);
    return 1 + (int)((0x764210u >> (4 * x)) & 15u);
  };
  int best = -127;
  if (imax) {
    // ceil(log2 N) of the largest magnitude: 0, 1, 2, 2, 3, 3, 4 for m = 1..7
    const int top = P + (int)((0x4332210u >> (4 * (imax - 1))) & 15u);
    best = best_exponent<int64_t>(top, P, 1ull, (uint64_t)sm[1], [&](int e, uint32_t& n4, uint64_t& a4) {
      const int q = mstar(e) - 1;
      const uint32_t v = (q & 2 ? (q & 4 ? tab[3] : tab[1]) : (q & 4 ? tab[2] : tab[0])) >> (16 * (q & 1));
      n4 = v & 63u;
      a4 = (v >> 6) & 1023u;
    });
  }
  const int ms = imax ? mstar(best) : 8;
  const uint32_t c0 = word_codes(raw[0], 0u, ms) | word_codes(raw[1], 0u, ms) << 16;
  const uint32_t c1 = word_codes(raw[2], 0u, ms) | word_codes(raw[3], 0u, ms) << 16;
  *reinterpret_cast<u32x2_t*>(codes + 8 * b) = u32x2_t{c0, c1};
  scales[b] = (uint8_t)(best + 127);
}

}  // namespace

hipError_t launch_fp8_block128_to_w2(int n, int R, int C, const uint8_t* e4m3, const float* bscale,
                                     uint8_t* codes, uint8_t* scales, int32_t* flag, hipStream_t s) {
  const long long nb = (long long)n * R * (C / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_block128_to_w2_kernel, dim3((unsigned)((nb + kFp8Threads - 1) / kFp8Threads)), dim3(kFp8Threads), 0,
                     s, nb, R, C, e4m3,
                     bscale, codes, scales, flag);
  return hipGetLastError();
}

hipError_t launch_mxfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* ue8m0, uint8_t* codes,
                              uint8_t* scales, int32_t* flag, hipStream_t s) {
  const long long nb = (long long)n * R * (C / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp4_to_w2_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, nb, e2m1, ue8m0, codes,
                     scales, flag);
  return hipGetLastError();
}

hipError_t launch_nvfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* e4m3,
                              const float* scale_2, uint8_t* codes, uint8_t* scales, int32_t* flag,
                              hipStream_t s) {
  const long long bpt = (long long)R * (C / 32);
  const long long nb = (long long)n * bpt;
  if (nb == 0) return hipSuccess;
  const int B = 256;
  hipLaunchKernelGGL(nvfp4_to_w2_kernel, dim3((unsigned)((nb + B - 1) / B)), dim3(B), 0, s, nb, bpt,
                     e2m1, e4m3, scale_2, codes, scales, flag);
  return hipGetLastError();
}

}  // namespace moew2
