// Decode-shaped expert GEMMs: few tokens per expert, the whole activated expert set streamed
// from HBM once per call. Decode time is set by the weight bytes read from HBM (README bullet
// "FP4 recovery - used surgically"), so the kernels are organised around keeping enough
// weight tiles in flight: every wave streams its tiles through a 4-deep register ring while the
// matrix cores consume the previous ones, with the expert's tokens (up to kChunk at a time) as
// the 16-row A operand staged in LDS.
//
// gate_up: weights bf16 (2-bit codes -> e2m1 -> bf16, UE8M0 scale folded in by the MX
//          conversion instruction), x bf16, fp32 accumulation; a = silu(g) * u rounded to fp16.
// down:    weights fp16 (same decode; the per-row offset E0 is applied in the epilogue), a fp16.
// combine: y[t] = sum over j ascending of w[t, j] * o[t*top_k + j] in fp32.
//
// Two organisations ("The v0.24.0 port", bullet "Deterministic unpermute": per-pair outputs are
// placed bijectively and summed in a fixed order, no atomics on values):
//  * routed (after the routing pass): one group per active expert holding all its pairs; the
//    down kernel writes per-pair rows o[p] and combine_kernel sums them in j order per token.
//  * direct (tiny batches, P = T*top_k <= kDirectMaxPairs): no routing pass; gate_up runs one
//    group per pair, and one down kernel covers every pair of a column block and combines in LDS.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int kChunk = 4;     // token rows per pass (valid rows of the 16-row MFMA tile)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;      // weight tiles in flight per wave

struct TileRegs {
  u32x4_t c[2];   // codes of up to two row groups (gate, up) for one k-tile
  u32x2_t s[2];   // their scale bytes (8 blocks of this lane's row)
};

template <int NB>
MOEW2_DEV void load_tile(TileRegs& r, const uint8_t* codes, const uint8_t* scales, const long long* tile_idx,
                         int kt, int lane) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const long long t = tile_idx[b] + kt;
    r.c[b] = ld16(codes + t * kTileCodeBytes + 16 * lane);
    r.s[b] = ld8(scales + t * kTileScaleBytes + 8 * (lane & 15));
  }
}

template <int BLK>
MOEW2_DEV float block_scale(const u32x2_t& s) {
  return ue8m0_scale_operand<BLK & 3>(BLK < 4 ? s[0] : s[1]);
}

// One k-tile (256 reduction elements = 8 blocks) for NB weight row groups.
template <class Op, int NB>
MOEW2_DEV void mma_tile(const TileRegs& r, const uint8_t* a_row, int kt, f32x4_t* acc) {
  typedef typename Op::vec vec;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t f0[NB], f1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) native_to_fp4(r.c[b][j], f0[b], f1[b]);
    const vec a0 = *reinterpret_cast<const vec*>(a_row + (size_t)(kt * kTileK + 32 * (2 * j)) * 2);
    const vec a1 = *reinterpret_cast<const vec*>(a_row + (size_t)(kt * kTileK + 32 * (2 * j + 1)) * 2);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s0 = j == 0 ? block_scale<0>(r.s[b]) : j == 1 ? block_scale<2>(r.s[b])
                     : j == 2 ? block_scale<4>(r.s[b]) : block_scale<6>(r.s[b]);
      const float s1 = j == 0 ? block_scale<1>(r.s[b]) : j == 1 ? block_scale<3>(r.s[b])
                     : j == 2 ? block_scale<5>(r.s[b]) : block_scale<7>(r.s[b]);
      acc[b] = Op::mfma(a0, Op::dequant(f0[b], s0), acc[b]);
      acc[b] = Op::mfma(a1, Op::dequant(f1[b], s1), acc[b]);
    }
  }
}

// Stream k-tiles [kb, ke) of NB row groups through a kRing-deep register ring.
template <class Op, int NB>
MOEW2_DEV void stream_k(TileRegs (&ring)[kRing], const uint8_t* codes, const uint8_t* scales,
                        const long long* tile_idx, int kb, int ke, const uint8_t* a_row, f32x4_t* acc,
                        int lane) {
  for (int k0 = kb; k0 < ke; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kt = k0 + i;
      if (kt < ke) {
        mma_tile<Op, NB>(ring[i], a_row, kt, acc);
        if (kt + kRing < ke) load_tile<NB>(ring[i], codes, scales, tile_idx, kt + kRing, lane);
      }
    }
  }
}

template <int NB>
MOEW2_DEV void prime_ring(TileRegs (&ring)[kRing], const uint8_t* codes, const uint8_t* scales,
                          const long long* tile_idx, int kb, int ke, int lane) {
#pragma unroll
  for (int i = 0; i < kRing; ++i)
    if (kb + i < ke) load_tile<NB>(ring[i], codes, scales, tile_idx, kb + i, lane);
}

// Work group of rows: expert e, n pairs; pair m's index and its row in the gated-intermediate
// buffer.
struct Group {
  int e, n, row0;
};

// ---------------------------------------------------------------------------------------------
// gate_up: grid (I / (16*NP), groups). Wave w handles row-pair q = blockIdx.x*NP + w/KS (gate row
// group 2q, up row group 2q+1) over the reduction slice w%KS of KS = 4/NP.
// DIRECT: group = pair p (expert ids[p]); act row = p. Otherwise group = active slot; act row =
// sorted position.
// ---------------------------------------------------------------------------------------------
template <int NP, bool DIRECT>
__global__ void __launch_bounds__(kThreads)
decode_gate_up_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                      const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                      const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                      const int32_t* __restrict__ active, const int32_t* __restrict__ meta,
                      _Float16* __restrict__ act, long long* __restrict__ counters,
                      int E, int K, int I, int top_k) {
  constexpr int KS = kWaves / NP;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  Group g;
  if (DIRECT) {
    const int p = blockIdx.y;
    g.e = ids[p];
    if (g.e < 0 || g.e >= E) return;
    g.n = 1;
    g.row0 = p;
  } else {
    if ((int)blockIdx.y >= meta[0]) return;
    g.e = active[blockIdx.y];
    g.row0 = offsets[g.e];
    g.n = offsets[g.e + 1] - g.row0;
  }
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int pw = w / KS, ks = w % KS;
  const int q = blockIdx.x * NP + pw;
  long long tile_idx[2] = {((long long)g.e * nrg + 2 * q) * nkt, ((long long)g.e * nrg + 2 * q + 1) * nkt};
  const int kb = ks * nkt / KS, ke = (ks + 1) * nkt / KS;
  const int stride = K * 2 + 16;
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][2][4][16]
  TileRegs ring[kRing];
  for (int c0 = 0; c0 < g.n; c0 += kChunk) {
    const int n = min(kChunk, g.n - c0);
    prime_ring<2>(ring, codes, scales, tile_idx, kb, ke, lane);
    const int per_row = K / 8;
    for (int idx = tid; idx < n * per_row; idx += kThreads) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      const int p = DIRECT ? g.row0 : perm[g.row0 + c0 + m];
      const int t = p / top_k;
      *reinterpret_cast<u32x4_t*>(lds + (size_t)m * stride + (size_t)c8 * 16) =
          ld16(x + (size_t)t * K + (size_t)c8 * 8);
    }
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    const uint8_t* a_row = lds + (size_t)ma * stride + (size_t)(8 * (lane >> 4)) * 2;
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    stream_k<Bf16Op, 2>(ring, codes, scales, tile_idx, kb, ke, a_row, acc, lane);
    if (KS > 1) {
      if (ks > 0 && lane < 16) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((w * 2 + b) * 4 + r) * 16 + lane] = acc[b][r];
      }
      __syncthreads();
      if (ks == 0 && lane < 16) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = acc[b][r];
            for (int kk = 1; kk < KS; ++kk) v += red[(((w + kk) * 2 + b) * 4 + r) * 16 + lane];
            acc[b][r] = v;
          }
      }
    }
    if (ks == 0 && lane < 16) {
      // accumulator register r of lanes 0..15 holds token row r, column lane
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        if (r < n) {
          const float a = silu_mul(acc[0][r], acc[1][r]);
          const _Float16 h = (_Float16)a;
          if (__builtin_isinf((float)h) && !__builtin_isinf(a)) atomicAdd((unsigned long long*)&counters[1], 1ull);
          const int row = DIRECT ? g.row0 : g.row0 + c0 + r;
          act[(size_t)row * I + 16 * q + lane] = h;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// routed down: grid (K / (16*NP), active slots). Wave w handles row group rg = blockIdx.x*NP +
// w/KS over the reduction slice w%KS. Per-pair rows go to pair_out at the pair index (bijective);
// combine_kernel then sums them per token in j order.
// ---------------------------------------------------------------------------------------------
template <int NP>
__global__ void __launch_bounds__(kThreads)
decode_down_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                   const int32_t* __restrict__ dn_e0, const _Float16* __restrict__ act,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                   const int32_t* __restrict__ active, const int32_t* __restrict__ meta,
                   float* __restrict__ pair_out, int E, int K, int I, int top_k) {
  constexpr int KS = kWaves / NP;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_active = meta[0];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if ((int)blockIdx.y >= n_active) return;
  const int e = active[blockIdx.y];
  const int row0 = offsets[e];
  const int n_e = offsets[e + 1] - row0;
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int pw = w / KS, ks = w % KS;
  const int rg = blockIdx.x * NP + pw;
  long long tile_idx[1] = {((long long)e * nrg + rg) * nkt};
  const int kb = ks * nkt / KS, ke = (ks + 1) * nkt / KS;
  const int stride = I * 2 + 16;
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][4][16]
  TileRegs ring[kRing];
  for (int c0 = 0; c0 < n_e; c0 += kChunk) {
    const int n = min(kChunk, n_e - c0);
    prime_ring<1>(ring, codes, scales, tile_idx, kb, ke, lane);
    const int per_row = I / 8;
    for (int idx = tid; idx < n * per_row; idx += kThreads) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      *reinterpret_cast<u32x4_t*>(lds + (size_t)m * stride + (size_t)c8 * 16) =
          ld16(act + (size_t)(row0 + c0 + m) * I + (size_t)c8 * 8);
    }
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    const uint8_t* a_row = lds + (size_t)ma * stride + (size_t)(8 * (lane >> 4)) * 2;
    f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
    stream_k<F16Op, 1>(ring, codes, scales, tile_idx, kb, ke, a_row, acc, lane);
    if (KS > 1) {
      if (ks > 0 && lane < 16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(w * 4 + r) * 16 + lane] = acc[0][r];
      }
      __syncthreads();
      if (ks == 0 && lane < 16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[0][r];
          for (int kk = 1; kk < KS; ++kk) v += red[((w + kk) * 4 + r) * 16 + lane];
          acc[0][r] = v;
        }
      }
    }
    if (ks == 0 && lane < 16) {
      const int col = 16 * rg + lane;
      const int e0 = dn_e0[(size_t)e * K + col];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        if (r < n) {
          const int p = perm[row0 + c0 + r];
          pair_out[(size_t)p * K + col] = __builtin_ldexpf(acc[0][r], e0);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// direct down + combine for tiny batches: grid (K/16). The workgroup covers one row group of 16
// output columns for every pair; wave w takes pairs w, w+4, ...; per-pair results meet in LDS and
// are combined per token in j order. Also records the two counters (single writer: block 0).
// ---------------------------------------------------------------------------------------------
constexpr int kDirectWaves = 2 * kDirectMaxPairs;   // two reduction halves per pair
constexpr int kDirectThreads = 64 * kDirectWaves;

__global__ void __launch_bounds__(kDirectThreads)
decode_down_direct_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                          const int32_t* __restrict__ dn_e0, const _Float16* __restrict__ act,
                          const int32_t* __restrict__ ids, const float* __restrict__ wts,
                          void* __restrict__ y, long long* __restrict__ counters, int out_dtype,
                          int T, int E, int K, int I, int top_k) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int P = T * top_k;                         // <= kDirectMaxPairs
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int rg = blockIdx.x, col = 16 * rg + (lane & 15);
  const int stride = I * 2 + 16;
  float* o = reinterpret_cast<float*>(lds + (size_t)kDirectMaxPairs * stride);  // [P][16]
  float* red = o + kDirectMaxPairs * 16;                                        // [P][4][16]
  // wave w: pair p = w / 2, reduction half w % 2; its tiles are requested before anything else
  const int p = w >> 1, hk = w & 1;
  const int id = p < P ? ids[p] : -1;
  const bool valid = id >= 0 && id < E;
  const long long tb = valid ? ((long long)id * nrg + rg) * nkt : 0;
  const int kb = hk * nkt / 2, ke = valid ? (hk + 1) * nkt / 2 : kb;
  TileRegs ring[kRing];
  prime_ring<1>(ring, codes, scales, &tb, kb, ke, lane);
  const int e0 = valid ? dn_e0[(size_t)id * K + col] : 0;
  // stage the gated rows of all valid pairs
  const int per_row = I / 8;
  for (int idx = tid; idx < P * per_row; idx += kDirectThreads) {
    const int pp = idx / per_row, c8 = idx - pp * per_row;
    const int ii = ids[pp];
    if (ii >= 0 && ii < E)
      *reinterpret_cast<u32x4_t*>(lds + (size_t)pp * stride + (size_t)c8 * 16) =
          ld16(act + (size_t)pp * I + (size_t)c8 * 8);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    // counters: invalid pairs, and gated intermediates that are infinite (from the staged rows)
    __shared__ int cnt[2];
    if (tid < 2) cnt[tid] = 0;
    __syncthreads();
    int bad = 0, inf = 0;
    for (int pp = 0; pp < P; ++pp) {
      const int ii = ids[pp];
      if (ii < 0 || ii >= E) { bad += tid == 0 ? 1 : 0; continue; }
      for (int c = tid; c < I; c += kDirectThreads) {
        const _Float16 h = *reinterpret_cast<const _Float16*>(lds + (size_t)pp * stride + (size_t)c * 2);
        if (__builtin_isinf((float)h)) ++inf;
      }
    }
    if (bad) atomicAdd(&cnt[0], bad);
    if (inf) atomicAdd(&cnt[1], inf);
    __syncthreads();
    if (tid == 0) { counters[0] = cnt[0]; counters[1] = cnt[1]; }
  }
  f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
  if (valid) {
    const uint8_t* a_row = lds + (size_t)p * stride + (size_t)(8 * (lane >> 4)) * 2;
    stream_k<F16Op, 1>(ring, codes, scales, &tb, kb, ke, a_row, acc, lane);
    if (hk == 1 && lane < 16) red[p * 16 + lane] = acc[0][0];
  }
  __syncthreads();
  if (valid && hk == 0 && lane < 16) o[p * 16 + lane] = __builtin_ldexpf(acc[0][0] + red[p * 16 + lane], e0);
  __syncthreads();
  // combine: y[t][16*rg + c] = sum_j w[t,j] * o[t*top_k+j][c]
  for (int idx = tid; idx < T * 16; idx += kDirectThreads) {
    const int t = idx / 16, c = idx - t * 16;
    float sum = 0.f;
    for (int j = 0; j < top_k; ++j) {
      const int pp = t * top_k + j;
      const int ii = ids[pp];
      if (ii < 0 || ii >= E) continue;
      sum += wts[pp] * o[pp * 16 + c];
    }
    const size_t yo = (size_t)t * K + 16 * rg + c;
    if (out_dtype == MOE_W2_OUT_F32) reinterpret_cast<float*>(y)[yo] = sum;
    else reinterpret_cast<uint16_t*>(y)[yo] = f32_to_bf16_rne(sum);
  }
}

// y[t] = sum_j (ascending) w[t, j] * o[t*top_k + j]; ids outside [0, E) contribute nothing.
// One thread per 4 output columns of one token (used after the GEMM path).
__global__ void combine_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wts,
                               const float* __restrict__ pair_out, void* __restrict__ y,
                               int T, int top_k, int E, int K, int out_dtype) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = K / 4;
  if (gid >= (long long)T * q) return;
  const int t = (int)(gid / q), c = (int)(gid - (long long)t * q) * 4;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int j = 0; j < top_k; ++j) {
    const int p = t * top_k + j;
    const int id = ids[p];
    if (id < 0 || id >= E) continue;
    const float w = wts[p];
    const float4 o = *reinterpret_cast<const float4*>(pair_out + (size_t)p * K + c);
    acc0 += w * o.x; acc1 += w * o.y; acc2 += w * o.z; acc3 += w * o.w;
  }
  if (out_dtype == MOE_W2_OUT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * K + c) = make_float4(acc0, acc1, acc2, acc3);
  } else {
    uint16_t* yb = reinterpret_cast<uint16_t*>(y) + (size_t)t * K + c;
    u32x2_t v = {(uint32_t)f32_to_bf16_rne(acc0) | ((uint32_t)f32_to_bf16_rne(acc1) << 16),
                 (uint32_t)f32_to_bf16_rne(acc2) | ((uint32_t)f32_to_bf16_rne(acc3) << 16)};
    *reinterpret_cast<u32x2_t*>(yb) = v;
  }
}

inline int pick_np(int slots) { return slots >= 32 ? 4 : 1; }

}  // namespace

size_t decode_direct_lds(int I) { return (size_t)kDirectMaxPairs * (I * 2 + 16) + (size_t)kDirectMaxPairs * 2 * 16 * 4; }

hipError_t launch_decode_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                                 const int32_t* ids, const Workspace& ws, uint8_t* wsb, bool direct,
                                 hipStream_t s) {
  const int P = T * top_k;
  const int slots = direct ? P : min(p->E, P);
  if (slots == 0) return hipSuccess;
  const size_t lds = (size_t)kChunk * (p->K * 2 + 16) + (size_t)kWaves * 2 * 4 * 16 * 4;
  const uint16_t* xb = (const uint16_t*)x;
  const int32_t* off = (const int32_t*)(wsb + ws.offsets);
  const int32_t* perm = (const int32_t*)(wsb + ws.perm);
  const int32_t* act_list = (const int32_t*)(wsb + ws.active);
  const int32_t* meta = (const int32_t*)(wsb + ws.meta);
  _Float16* act = (_Float16*)(wsb + ws.act);
  long long* cnt = (long long*)(wsb + ws.counters);
  if (direct) {
    hipLaunchKernelGGL((decode_gate_up_kernel<1, true>), dim3(p->I / 16, slots), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, off, perm, act_list, meta, act, cnt, p->E, p->K, p->I, top_k);
  } else if (pick_np(slots) == 4) {
    hipLaunchKernelGGL((decode_gate_up_kernel<4, false>), dim3(p->I / 64, slots), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, off, perm, act_list, meta, act, cnt, p->E, p->K, p->I, top_k);
  } else {
    hipLaunchKernelGGL((decode_gate_up_kernel<1, false>), dim3(p->I / 16, slots), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, off, perm, act_list, meta, act, cnt, p->E, p->K, p->I, top_k);
  }
  return hipGetLastError();
}

hipError_t launch_decode_down(const moe_w2_planes* p, int T, int top_k, const int32_t* ids, const float* w,
                              void* y, int out_dtype, const Workspace& ws, uint8_t* wsb, bool direct,
                              hipStream_t s) {
  const int P = T * top_k;
  if (P == 0) return hipSuccess;
  const _Float16* act = (const _Float16*)(wsb + ws.act);
  if (direct) {
    hipLaunchKernelGGL(decode_down_direct_kernel, dim3(p->K / 16), dim3(kDirectThreads), decode_direct_lds(p->I), s,
                       p->dn_codes, p->dn_scales, p->dn_e0, act, ids, w, y, (long long*)(wsb + ws.counters),
                       out_dtype, T, p->E, p->K, p->I, top_k);
    return hipGetLastError();
  }
  const int slots = min(p->E, P);
  const size_t lds = (size_t)kChunk * (p->I * 2 + 16) + (size_t)kWaves * 4 * 16 * 4;
  const int np = pick_np(slots);
  auto args = [&](auto kern, int gx) {
    hipLaunchKernelGGL(kern, dim3(gx, slots), dim3(kThreads), lds, s,
                       p->dn_codes, p->dn_scales, p->dn_e0, act,
                       (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                       (const int32_t*)(wsb + ws.active), (const int32_t*)(wsb + ws.meta),
                       (float*)(wsb + ws.pair_out), p->E, p->K, p->I, top_k);
  };
  if (np == 4) args(decode_down_kernel<4>, p->K / 64);
  else args(decode_down_kernel<1>, p->K / 16);
  return hipGetLastError();
}

hipError_t launch_combine(int T, int top_k, int E, int K, const int32_t* ids, const float* w,
                          const float* pair_out, void* y, int out_dtype, hipStream_t s) {
  const long long n = (long long)T * (K / 4);
  if (n == 0) return hipSuccess;
  const int B = 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + B - 1) / B)), dim3(B), 0, s, ids, w, pair_out, y,
                     T, top_k, E, K, out_dtype);
  return hipGetLastError();
}

}  // namespace moew2
