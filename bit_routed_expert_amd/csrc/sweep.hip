// Sign-bias diagnostic of 2-bit codebooks: moe_w2_codebook_sweep.
//
// For every tensor and every candidate 4-value codebook, the tensor is quantized the way the
// 2-bit planes are (power-of-two scale per block of 32 along a row, nearest code per element)
// and two numbers are kept: the relative RMS error and the mean bias. The pages pick the
// sign-symmetric codebook {-4,-1,1,4} because the L2-optimal 2-bit codebook is sign-asymmetric
// and its per-expert bias compounds across layers, while the symmetric one reaches the same
// relative RMS with a far smaller bias (README, bullet "2-bit expert planes - the sign-bias
// finding"; vLLM-Moet article, section "Sign symmetry, not error size, is what collapses naive
// 2-bit experts").
//
// Arithmetic (readings where the pages are silent; float64 is the pages' precision for load-time
// quantization):
//  * the block exponent minimises the block's squared error over the ten exponents from 7 below
//    to 2 above e_c, the smallest exponent with max(|q0|,|q3|) 2^e_c >= the block's max |x|
//    (e_c = -127 for an all-zero block), clamped to [-127, 127]; equal errors -> lower exponent;
//  * nearest code, exactly halfway -> the code of smaller magnitude, equal magnitudes (x = 0) ->
//    the side of x's sign bit;
//  * a block's squared error is summed in float64 in element order, (x - v) * (x - v) rounded
//    before the add (no fused multiply-add in this file), so the exponent decision is
//    reproducible from the definition.
//
// Work split: one thread per block of 32 elements (x in 32 float64 registers); every codebook is
// swept over the same register block, ALU-bound. Per-tensor sums go through per-workgroup
// partials in a fixed order, so the result is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/moe_w2.h"

#pragma clang fp contract(off)

namespace moew2 {
namespace {

constexpr int kSweepThreads = 256;
constexpr int kSweepWaves = kSweepThreads / 64;
constexpr int kSweepMaxCodebooks = 4096;
constexpr int kSweepTargetWorkgroups = 8192;

struct Codebook {
  double q[4], mid[3];
  double tf[3];        // threshold for the fast path: mid, or the next double below it when a tie goes up
  bool eq[3];          // |q_k| = |q_{k+1}|: a zero midpoint
  bool hi_only;        // every q_k has a zero low word (at most 20 significant bits), at any scale
  double qmax;
  int qexp;            // ilogb(qmax)
};

__device__ __forceinline__ Codebook load_codebook(const float* cb, int m) {
  Codebook c;
#pragma unroll
  for (int k = 0; k < 4; ++k) c.q[k] = (double)cb[4 * m + k];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    c.mid[k] = 0.5 * (c.q[k] + c.q[k + 1]);
    const bool up = fabs(c.q[k + 1]) < fabs(c.q[k]);   // a tie goes to the smaller magnitude
    c.eq[k] = fabs(c.q[k + 1]) == fabs(c.q[k]);
    c.tf[k] = up ? nextafter(c.mid[k], -INFINITY) : c.mid[k];
  }
  c.hi_only = true;
#pragma unroll
  for (int k = 0; k < 4; ++k) c.hi_only = c.hi_only && (uint32_t)__double_as_longlong(c.q[k]) == 0u;
  c.qmax = fmax(fabs(c.q[0]), fabs(c.q[3]));
  c.qexp = ilogb(c.qmax);
  return c;
}

// Squared error and sum of (v - x) of one block at its chosen exponent. "x > tf_k" decides code
// boundary k: tf_k is mid_k, or the double just below it where a tie goes up (scaling by 2^e
// keeps that relation exact). The one tie it gets wrong is x = +0 at a zero midpoint (between
// q and -q, where the tie follows the sign bit and +0 goes up), so a block holding a +0 takes
// the general test. kHi: the code values have zero low words, so only the high words are selected.
template <bool kGeneral, bool kHi>
__device__ __forceinline__ void block_choice(const double (&x)[32], double amax,
                                             const Codebook& c, double& sse, double& err) {
  int ec = -127;
  if (amax != 0.0) {
    ec = ilogb(amax) - c.qexp;
    if (ldexp(c.qmax, ec) < amax) ++ec;
    ec = min(max(ec, -127), 127);
  }
  double best = INFINITY, best_err = 0.0;
  for (int d = 0; d < 10; ++d) {
    const int e = ec - 7 + d;
    if (e < -127 || e > 127) continue;
    const double s = ldexp(1.0, e);
    double v0 = c.q[0] * s, v1 = c.q[1] * s, v2 = c.q[2] * s, v3 = c.q[3] * s;
    // keep the scaled code values as selected operands (otherwise the selection is rewritten as
    // select-then-scale, one more multiply per element, and the high-word select is lost)
    asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
    double acc = 0.0, eacc = 0.0;
    const double t0 = c.tf[0] * s, t1 = c.tf[1] * s, t2 = c.tf[2] * s;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double xi = x[i];
      bool p0 = xi > t0, p1 = xi > t1, p2 = xi > t2;
      if (kGeneral) {   // +0 goes up at a zero midpoint (whose tf_k is that midpoint)
        // x * 2^e is +0 exactly when x is (no underflow for e >= -127); the product keeps the
        // test inside the loop, where 32 hoisted lane masks would not fit the scalar registers
        const bool pz = __double_as_longlong(xi * s) == 0;
        p0 = p0 || (c.eq[0] && pz);
        p1 = p1 || (c.eq[1] && pz);
        p2 = p2 || (c.eq[2] && pz);
      }
      double v;   // boundaries are ordered: p2 implies p1 implies p0
      if (kHi) {
        int h = p0 ? __double2hiint(v1) : __double2hiint(v0);
        h = p1 ? __double2hiint(v2) : h;
        h = p2 ? __double2hiint(v3) : h;
        v = __hiloint2double(h, 0);
      } else {
        v = p0 ? v1 : v0;
        v = p1 ? v2 : v;
        v = p2 ? v3 : v;
      }
      const double dx = xi - v;
      const double sq = dx * dx;
      acc = acc + sq;
      eacc = eacc - dx;
    }
    if (acc < best) {
      best = acc;
      best_err = eacc;
    }
  }
  sse = best;
  err = best_err;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = v + __shfl_xor(v, o, 64);
  return v;
}

// partials [n * G][M + 1] of {sse, err} (slot M: {sum x^2, sum x}); block b of tensor t is taken
// by workgroup t * G + b / (256 * iters), thread b % 256, in iteration (b / 256) % iters.
__global__ void __launch_bounds__(kSweepThreads)
sweep_kernel(const float* __restrict__ x, const float* __restrict__ cb, int M, long long nb, int G, int iters,
             double2* __restrict__ partials, int32_t* __restrict__ flag) {
  __shared__ double2 red[kSweepWaves];
  const int t = blockIdx.x / G, g = blockIdx.x % G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* xt = x + (long long)t * nb * 32;
  const long long b0 = (long long)g * kSweepThreads * iters + threadIdx.x;
  double2* out = partials + (long long)blockIdx.x * (M + 1);

  auto load = [&](long long b, double (&xv)[32], double& amax, bool& zero) {
    const float4* p = reinterpret_cast<const float4*>(xt + 32 * b);
    amax = 0.0;
    zero = false;
    bool finite = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 f = p[j];
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[4 * j + k] = (double)fv[k];
        finite = finite && isfinite(fv[k]);
        zero = zero || __float_as_uint(fv[k]) == 0u;
        amax = fmax(amax, fabs(xv[4 * j + k]));
      }
    }
    if (!finite) *flag = 1;
  };
  auto publish = [&](int slot, double a, double b) {
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) red[wave] = make_double2(a, b);
    __syncthreads();
    if (threadIdx.x == 0) {
      double2 s = red[0];
#pragma unroll
      for (int w = 1; w < kSweepWaves; ++w) {
        s.x = s.x + red[w].x;
        s.y = s.y + red[w].y;
      }
      out[slot] = s;
    }
    __syncthreads();
  };

  for (int m = 0; m < M; ++m) {
    const Codebook c = load_codebook(cb, m);
    double sse = 0.0, err = 0.0;
    for (int it = 0; it < iters; ++it) {
      const long long b = b0 + (long long)it * kSweepThreads;
      if (b >= nb) break;
      double xv[32], amax;
      bool zero;
      load(b, xv, amax, zero);
      double s, e;
      if (c.hi_only) {
        if (zero)   // holds a +0
          block_choice<true, true>(xv, amax, c, s, e);
        else
          block_choice<false, true>(xv, amax, c, s, e);
      } else {
        if (zero)
          block_choice<true, false>(xv, amax, c, s, e);
        else
          block_choice<false, false>(xv, amax, c, s, e);
      }
      sse = sse + s;
      err = err + e;
    }
    publish(m, sse, err);
  }
  double s2 = 0.0, s1 = 0.0;
  for (int it = 0; it < iters; ++it) {
    const long long b = b0 + (long long)it * kSweepThreads;
    if (b >= nb) break;
    double xv[32], amax;
    bool zero;
    load(b, xv, amax, zero);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double sq = xv[i] * xv[i];
      s2 = s2 + sq;
      s1 = s1 + xv[i];
    }
  }
  publish(M, s2, s1);
}

// one thread per (tensor, codebook): sums the tensor's G partials in order
__global__ void __launch_bounds__(256)
sweep_reduce_kernel(const double2* __restrict__ partials, int n, int M, int G, long long N,
                    double* __restrict__ stats, double* __restrict__ moments) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n * M) return;
  const int t = (int)(i / M), m = (int)(i % M);
  double sse = 0.0, err = 0.0, s2 = 0.0, s1 = 0.0;
  for (int g = 0; g < G; ++g) {
    const double2* p = partials + ((long long)t * G + g) * (M + 1);
    sse = sse + p[m].x;
    err = err + p[m].y;
    s2 = s2 + p[M].x;
    s1 = s1 + p[M].y;
  }
  double* o = stats + i * 4;
  o[0] = sse;
  o[1] = err;
  o[2] = s2 > 0.0 ? sqrt(sse / s2) : 0.0;
  o[3] = s2 > 0.0 ? err / sqrt((double)N * s2) : 0.0;
  if (m == 0) {
    moments[2 * t] = s2;
    moments[2 * t + 1] = s1;
  }
}

// one thread per tensor: least-sse symmetric (q0 = -q3, q1 = -q2) and asymmetric codebook
__global__ void __launch_bounds__(256)
sweep_best_kernel(const double* __restrict__ stats, const float* __restrict__ cb, int n, int M,
                  int32_t* __restrict__ best) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  int bs = -1, ba = -1;
  double vs = 0.0, va = 0.0;
  for (int m = 0; m < M; ++m) {
    const double s = stats[((long long)t * M + m) * 4];
    const float* q = cb + 4 * m;
    if (q[0] == -q[3] && q[1] == -q[2]) {
      if (bs < 0 || s < vs) { bs = m; vs = s; }
    } else if (ba < 0 || s < va) {
      ba = m;
      va = s;
    }
  }
  best[2 * t] = bs;
  best[2 * t + 1] = ba;
}

}  // namespace
}  // namespace moew2

using namespace moew2;

extern "C" int moe_w2_codebook_sweep(int n, int R, int C, const float* x, int M, const float* codebooks,
                                     double* stats, double* moments, int32_t* best, void* stream) {
  if (n < 0 || R < 0 || C < 0 || M < 1 || M > kSweepMaxCodebooks || !codebooks) return MOE_W2_EINVAL;
  if (C % 32) return MOE_W2_EUNSUPPORTED;
  for (int m = 0; m < M; ++m) {
    const float* q = codebooks + 4 * m;
    for (int k = 0; k < 4; ++k)
      if (!std::isfinite(q[k])) return MOE_W2_EINVAL;
    if (!(q[0] < q[1] && q[1] < q[2] && q[2] < q[3])) return MOE_W2_EINVAL;
  }
  if (n == 0) return MOE_W2_OK;
  if (!stats || !moments || !best || ((long long)R * C > 0 && !x)) return MOE_W2_EINVAL;
  if (reinterpret_cast<uintptr_t>(x) % 16) return MOE_W2_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const long long nb = (long long)R * C / 32;
  const long long per_tensor_target = (kSweepTargetWorkgroups + n - 1) / n;
  const long long iters =
      nb == 0 ? 1 : std::max(1LL, (nb + kSweepThreads * per_tensor_target - 1) / (kSweepThreads * per_tensor_target));
  const long long G = (nb + kSweepThreads * iters - 1) / (kSweepThreads * iters);
  if (iters > INT32_MAX || (long long)n * G > INT32_MAX) return MOE_W2_EUNSUPPORTED;

  const size_t part_bytes = (size_t)n * G * (M + 1) * sizeof(double2);
  const size_t cb_off = (part_bytes + 255) / 256 * 256, flag_off = cb_off + (size_t)M * 16;
  char* buf = nullptr;
  if (hipMalloc(&buf, flag_off + 256) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_W2_ENOMEM;
  }
  double2* partials = reinterpret_cast<double2*>(buf);
  float* dcb = reinterpret_cast<float*>(buf + cb_off);
  int32_t* dflag = reinterpret_cast<int32_t*>(buf + flag_off);
  int32_t flag = 0;
  hipError_t err = hipMemcpyAsync(dcb, codebooks, (size_t)M * 16, hipMemcpyHostToDevice, s);
  if (err == hipSuccess) err = hipMemsetAsync(dflag, 0, sizeof(int32_t), s);
  if (err == hipSuccess && G > 0) {
    sweep_kernel<<<dim3((unsigned)(n * G)), dim3(kSweepThreads), 0, s>>>(x, dcb, M, nb, (int)G, (int)iters,
                                                                         partials, dflag);
    err = hipGetLastError();
  }
  if (err == hipSuccess) {
    const long long nm = (long long)n * M;
    sweep_reduce_kernel<<<dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s>>>(partials, n, M, (int)G,
                                                                                 (long long)R * C, stats, moments);
    err = hipGetLastError();
  }
  if (err == hipSuccess) {
    sweep_best_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(stats, dcb, n, M, best);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipMemcpyAsync(&flag, dflag, 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  (void)hipFree(buf);
  if (err != hipSuccess) return MOE_W2_EHIP;
  return flag ? MOE_W2_ENAN : MOE_W2_OK;
}
