// Decode-shaped expert GEMMs: few tokens per expert, the whole activated expert set streamed
// from HBM once per call. Decode is bound by the weight stream (README bullet "FP4 recovery -
// used surgically": decode is HBM-bound), so each workgroup streams one group of weight rows of
// one active expert through the matrix cores with the expert's tokens (up to kChunk at a time)
// as the 16-row A operand; the four waves split the reduction axis and are summed in a fixed
// order in LDS.
//
// gate_up: weights bf16 (2-bit codes -> e2m1 -> bf16 with the UE8M0 scale folded in by the MX
//          conversion instruction), x bf16, fp32 accumulation; epilogue a = silu(g) * u, rounded
//          to fp16 and stored at the pair's sorted position.
// down:    weights fp16 (same decode, per-row offset E0 applied in the epilogue), a fp16;
//          output rows o[p] (fp32) at the pair index p (bijective; no atomics).
#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int kChunk = 4;     // tokens per pass (rows of the 16-row MFMA tile that are valid)
constexpr int kWaves = 4;     // split of the reduction axis
constexpr int kThreads = 64 * kWaves;

struct TileRegs {
  u32x4_t c[2];   // codes of up to two row groups (gate, up) for one k-tile
  u32x2_t s[2];   // their scale bytes (8 blocks of this lane's row)
};

template <int NB>
MOEW2_DEV TileRegs load_tile(const uint8_t* codes, const uint8_t* scales, const long long* tile_idx,
                             int kt, int lane) {
  TileRegs r;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const long long t = tile_idx[b] + kt;
    r.c[b] = ld16(codes + t * kTileCodeBytes + 16 * lane);
    r.s[b] = ld8(scales + t * kTileScaleBytes + 8 * (lane & 15));
  }
  return r;
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
    // block 2j
    {
      const vec a = *reinterpret_cast<const vec*>(a_row + (size_t)(kt * kTileK + 32 * (2 * j)) * 2);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float sc = j == 0 ? block_scale<0>(r.s[b]) : j == 1 ? block_scale<2>(r.s[b])
                 : j == 2 ? block_scale<4>(r.s[b]) : block_scale<6>(r.s[b]);
        acc[b] = Op::mfma(a, Op::dequant(f0[b], sc), acc[b]);
      }
    }
    // block 2j+1
    {
      const vec a = *reinterpret_cast<const vec*>(a_row + (size_t)(kt * kTileK + 32 * (2 * j + 1)) * 2);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float sc = j == 0 ? block_scale<1>(r.s[b]) : j == 1 ? block_scale<3>(r.s[b])
                 : j == 2 ? block_scale<5>(r.s[b]) : block_scale<7>(r.s[b]);
        acc[b] = Op::mfma(a, Op::dequant(f1[b], sc), acc[b]);
      }
    }
  }
}

// GATE_UP: grid (I/16 column groups, active slots); DOWN: grid (K/16 row groups, active slots).
template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads)
decode_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
              const int32_t* __restrict__ dn_e0, const void* __restrict__ a_src,
              const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
              const int32_t* __restrict__ active, const int32_t* __restrict__ meta,
              void* __restrict__ out, long long* __restrict__ counters,
              int E, int K, int I, int top_k) {
  typedef typename std::conditional<GATE_UP, Bf16Op, F16Op>::type Op;
  constexpr int NB = GATE_UP ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slot = blockIdx.y;
  if (slot >= meta[0]) return;
  const int e = active[slot];
  const int row0 = offsets[e];
  const int n_e = offsets[e + 1] - row0;
  const int KR = GATE_UP ? K : I;              // reduction length
  const int NR = GATE_UP ? 2 * I : K;          // weight rows
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg0 = GATE_UP ? 2 * blockIdx.x : blockIdx.x;
  long long tile_idx[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) tile_idx[b] = ((long long)e * nrg + rg0 + b) * nkt;
  const int kb = w * nkt / kWaves, ke = (w + 1) * nkt / kWaves;
  const int stride = KR * 2 + 16;              // LDS row stride of the A rows, bytes
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves-1][NB][4][16]

  for (int c0 = 0; c0 < n_e; c0 += kChunk) {
    const int n = min(kChunk, n_e - c0);
    // first weight tiles of this wave are requested before the A rows are staged
    TileRegs cur = load_tile<NB>(codes, scales, tile_idx, min(kb, nkt - 1), lane);
    TileRegs nxt = load_tile<NB>(codes, scales, tile_idx, min(kb + 1, nkt - 1), lane);
    // stage the chunk's A rows: n rows of KR 2-byte elements
    const int per_row = KR / 8;  // 16-byte pieces
    for (int idx = tid; idx < n * per_row; idx += kThreads) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      const uint8_t* src;
      if (GATE_UP) {
        const int t = perm[row0 + c0 + m] / top_k;
        src = reinterpret_cast<const uint8_t*>(a_src) + ((size_t)t * K + (size_t)c8 * 8) * 2;
      } else {
        src = reinterpret_cast<const uint8_t*>(a_src) + ((size_t)(row0 + c0 + m) * I + (size_t)c8 * 8) * 2;
      }
      *reinterpret_cast<u32x4_t*>(lds + (size_t)m * stride + (size_t)c8 * 16) = ld16(src);
    }
    __syncthreads();
    // this lane's A row (rows >= n repeat the last valid row; their outputs are discarded)
    const int ma = min(lane & 15, n - 1);
    const uint8_t* a_row = lds + (size_t)ma * stride + (size_t)(8 * (lane >> 4)) * 2;
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kt = kb; kt < ke; ++kt) {
      TileRegs nn = load_tile<NB>(codes, scales, tile_idx, min(kt + 2, nkt - 1), lane);
      mma_tile<Op, NB>(cur, a_row, kt, acc);
      cur = nxt;
      nxt = nn;
    }
    // fixed-order split-K sum: waves 1..3 park their partials, wave 0 adds them in wave order
    if (w > 0 && lane < 16) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(((w - 1) * NB + b) * 4 + r) * 16 + lane] = acc[b][r];
    }
    __syncthreads();
    if (w == 0 && lane < 16) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[b][r];
#pragma unroll
          for (int ww = 1; ww < kWaves; ++ww) v += red[(((ww - 1) * NB + b) * 4 + r) * 16 + lane];
          acc[b][r] = v;
        }
      // accumulator register r of lanes 0..15 holds token row r, column lane
      for (int r = 0; r < n; ++r) {
        if (GATE_UP) {
          const float a = silu_mul(acc[0][r], acc[1][r]);
          const _Float16 h = (_Float16)a;
          if (__builtin_isinf((float)h) && !__builtin_isinf(a)) atomicAdd((unsigned long long*)&counters[1], 1ull);
          _Float16* act = reinterpret_cast<_Float16*>(out);
          act[(size_t)(row0 + c0 + r) * I + 16 * blockIdx.x + lane] = h;
        } else {
          const int col = 16 * blockIdx.x + lane;
          const float o = __builtin_ldexpf(acc[0][r], dn_e0[(size_t)e * K + col]);
          const int p = perm[row0 + c0 + r];
          reinterpret_cast<float*>(out)[(size_t)p * K + col] = o;
        }
      }
    }
    __syncthreads();
  }
}

// y[t] = sum_j (ascending) w[t, j] * o[t*top_k + j]; ids outside [0, E) contribute nothing.
// One thread per 4 output columns of one token.
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

}  // namespace

hipError_t launch_decode_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                                 const Workspace& ws, uint8_t* wsb, hipStream_t s) {
  const int max_slots = min(p->E, T * top_k);
  if (max_slots == 0) return hipSuccess;
  const size_t lds = (size_t)kChunk * (p->K * 2 + 16) + (size_t)(kWaves - 1) * 2 * 4 * 16 * 4;
  hipLaunchKernelGGL(decode_kernel<true>, dim3(p->I / 16, max_slots), dim3(kThreads), lds, s,
                     p->gu_codes, p->gu_scales, p->dn_e0, x,
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.active), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.act), (long long*)(wsb + ws.counters), p->E, p->K, p->I, top_k);
  return hipGetLastError();
}

hipError_t launch_decode_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                              uint8_t* wsb, hipStream_t s) {
  const int max_slots = min(p->E, T * top_k);
  if (max_slots == 0) return hipSuccess;
  const size_t lds = (size_t)kChunk * (p->I * 2 + 16) + (size_t)(kWaves - 1) * 1 * 4 * 16 * 4;
  hipLaunchKernelGGL(decode_kernel<false>, dim3(p->K / 16, max_slots), dim3(kThreads), lds, s,
                     p->dn_codes, p->dn_scales, p->dn_e0, (const void*)(wsb + ws.act),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.active), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.pair_out), (long long*)(wsb + ws.counters), p->E, p->K, p->I, top_k);
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
