// Decode-shaped expert GEMMs: few tokens per expert, the whole activated expert set streamed
// from HBM once per call. Decode time is set by the weight bytes read from HBM (README bullet
// "FP4 recovery - used surgically"), so the kernels are organised around keeping enough weight
// tiles in flight: every wave streams its tiles through a 4-deep register ring while the matrix
// cores consume the previous ones, with the expert's tokens (up to kChunk at a time) as the
// 16-row A operand staged in LDS.
//
// gate_up: weights bf16 (2-bit codes -> e2m1 -> bf16, UE8M0 scale folded in by the MX
//          conversion instruction), x bf16, fp32 accumulation; a = silu(g) * u rounded to fp16.
// down:    weights fp16 (same decode; the per-row offset E0 is applied in the epilogue), a fp16.
// combine: y[t] = sum over j ascending of w[t, j] * o[t*top_k + j] in fp32.
//
// Load ordering: a workgroup first issues its staging loads (x or the gated rows), then the
// first kRing weight tiles of every wave, and only then waits - for the staging loads alone -
// before writing LDS. Weight tiles are raw buffer loads; a tile past the end of a wave's range is
// requested at an out-of-range offset (no memory access), so the load sequence never branches
// and the ring's waits stay exact.
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
constexpr int kStage = 4;     // 16-byte staging pieces per thread per memory round trip

struct TileRegs {
  u32x4_t c[2];   // codes of up to two row groups (gate, up) for one k-tile
  u32x2_t s[2];   // their scale bytes (8 blocks of this lane's row)
};

// One expert's planes as buffer views, and the tile index (within the expert) of k-tile 0 of
// each of the wave's NB row groups.
template <int NB>
struct WaveTiles {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t tile[NB];
};

template <int NB>
MOEW2_DEV WaveTiles<NB> wave_tiles(const uint8_t* codes, const uint8_t* scales, int e, uint32_t tiles_per_expert) {
  WaveTiles<NB> wt;
  wt.codes = buffer_view(codes + (size_t)e * tiles_per_expert * kTileCodeBytes, tiles_per_expert * kTileCodeBytes);
  wt.scales = buffer_view(scales + (size_t)e * tiles_per_expert * kTileScaleBytes, tiles_per_expert * kTileScaleBytes);
  return wt;
}

// The tile's byte offset goes in the scalar offset; the lane's offset (shifted out of range when
// the tile is not wanted - a wave-uniform condition) in the range-checked vector offset.
template <int NB>
MOEW2_DEV void load_tile(TileRegs& r, const WaveTiles<NB>& wt, int kt, bool valid, int lane) {
  const uint32_t oob = valid ? 0u : kOutOfRange;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t t = wt.tile[b] + (uint32_t)kt;
    r.c[b] = buf_ld16_nt(wt.codes, (16u * (uint32_t)lane) | oob, t * kTileCodeBytes);
    r.s[b] = buf_ld8_nt(wt.scales, (8u * (uint32_t)(lane & 15)) | oob, t * kTileScaleBytes);
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

// ring[i] <- k-tile kb + i (out-of-range requests past ke)
template <int NB>
MOEW2_DEV void prime_ring(TileRegs (&ring)[kRing], const WaveTiles<NB>& wt, int kb, int ke, int lane) {
#pragma unroll
  for (int i = 0; i < kRing; ++i) load_tile<NB>(ring[i], wt, kb + i, kb + i < ke, lane);
}

// Consume k-tiles [kb, ke) from the primed ring; each consumed slot is refilled with the tile
// kRing further on (or an out-of-range request), so every iteration issues the same loads.
template <class Op, int NB>
MOEW2_DEV void stream_k(TileRegs (&ring)[kRing], const WaveTiles<NB>& wt, int kb, int ke, const uint8_t* a_row,
                        f32x4_t* acc, int lane) {
  for (int k0 = kb; k0 < ke; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kt = k0 + i;
      if (kt < ke) mma_tile<Op, NB>(ring[i], a_row, kt, acc);
      load_tile<NB>(ring[i], wt, kt + kRing, kt + kRing < ke, lane);
    }
  }
}

// Staging of n rows (row length `len` 16-bit elements, a multiple of 256) into LDS rows of
// `stride` bytes; row m starts at element row_off(m) of src. Piece idx (16 bytes) of the flat
// [n][len/8] range goes to thread idx % NT; a batch covers kStage pieces per thread, issued
// together (stage_issue) and written to LDS together (stage_commit).
struct Stage {
  u32x4_t v[kStage];
};

template <int NT, class RowOff>
MOEW2_DEV void stage_issue(Stage& st, const uint16_t* src, int len, int n, int base, RowOff row_off, int tid) {
  const int per_row = len / 8, total = n * per_row;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int idx = base + i * NT + tid;
    if (idx < total) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      st.v[i] = ld16(src + row_off(m) + (size_t)c8 * 8);
    }
  }
}

template <int NT>
MOEW2_DEV void stage_commit(const Stage& st, uint8_t* lds, int stride, int len, int n, int base, int tid) {
  const int per_row = len / 8, total = n * per_row;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int idx = base + i * NT + tid;
    if (idx < total) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      *reinterpret_cast<u32x4_t*>(lds + (size_t)m * stride + (size_t)c8 * 16) = st.v[i];
    }
  }
}

// Stage n rows while the weight ring is primed. Batches beyond the first (rows longer than
// kStage * NT / n pieces) go first, one round trip each; the first batch is issued just before
// the prime and written after it. Every path thus reaches the streaming loop with the same loads
// outstanding, which keeps the compiler's waits inside the loop exact.
template <int NT, int NB, class RowOff>
MOEW2_DEV void stage_and_prime(TileRegs (&ring)[kRing], const WaveTiles<NB>& wt, int kb, int ke, int lane,
                               uint8_t* lds, int stride, const uint16_t* src, int len, int n, RowOff row_off,
                               int tid) {
  Stage st;
  for (int base = kStage * NT; base < n * (len / 8); base += kStage * NT) {
    stage_issue<NT>(st, src, len, n, base, row_off, tid);
    stage_commit<NT>(st, lds, stride, len, n, base, tid);
  }
  stage_issue<NT>(st, src, len, n, 0, row_off, tid);
  prime_ring<NB>(ring, wt, kb, ke, lane);
  stage_commit<NT>(st, lds, stride, len, n, 0, tid);
}

// ---------------------------------------------------------------------------------------------
// gate_up on the block-scaled matrix instruction (fp8 x, fp4 weights; operand order in common.h).
// The staged x rows are split into hi and lo e4m3 parts while they are written to LDS:
//   row layout in LDS: hi [K] bytes | lo [K] bytes | scale words [K/256][4 lane groups][4 bytes:
//   hi chunk 0, hi chunk 1, lo chunk 0, lo chunk 1] | pad.
// ---------------------------------------------------------------------------------------------
__host__ __device__ inline int gu_row_stride(int K) { return 2 * K + K / 16 + 64; }

struct GuTileRegs {
  u32x4_t c[2];     // codes of the gate and up row groups (block layout)
  uint32_t s[2];    // their two scale bytes (chunks 0 and 1)
};

MOEW2_DEV void load_gu_tile(GuTileRegs& r, const WaveTiles<2>& wt, int kt, bool valid, int lane) {
  const uint32_t oob = valid ? 0u : kOutOfRange;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t t = wt.tile[b] + (uint32_t)kt;
    r.c[b] = buf_ld16_nt(wt.codes, (16u * (uint32_t)lane) | oob, t * kTileCodeBytes);
    r.s[b] = buf_ld2_nt(wt.scales, (2u * (uint32_t)lane) | oob, t * kTileScaleBytes);
  }
}

template <int C>
MOEW2_DEV void mma_gu_chunk(const GuTileRegs& r, const uint8_t* hi, const uint8_t* lo, uint32_t sa, int g,
                            f32x4_t* acc) {
  const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(hi + 128 * C + 16 * g);
  const u32x4_t h1 = *reinterpret_cast<const u32x4_t*>(hi + 128 * C + 64 + 16 * g);
  const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(lo + 128 * C + 16 * g);
  const u32x4_t l1 = *reinterpret_cast<const u32x4_t*>(lo + 128 * C + 64 + 16 * g);
  const i32x8_t ah = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
  const i32x8_t al = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const i32x8_t bo = mx_b_operand(r.c[b][2 * C], r.c[b][2 * C + 1]);
    acc[b] = mx_mfma<C, C>(ah, bo, acc[b], sa, r.s[b]);
    acc[b] = mx_mfma<2 + C, C>(al, bo, acc[b], sa, r.s[b]);
  }
}

// One k-tile: `arow` is the lane's staged row (hi part at +0, lo at +K, scale words at +2K).
MOEW2_DEV void mma_gu_tile(const GuTileRegs& r, const uint8_t* arow, int K, int kt, int g, f32x4_t* acc) {
  const uint8_t* hi = arow + kt * kTileK;
  const uint8_t* lo = hi + K;
  const uint32_t sa = *reinterpret_cast<const uint32_t*>(arow + 2 * K + kt * 16 + 4 * g);
  mma_gu_chunk<0>(r, hi, lo, sa, g, acc);
  mma_gu_chunk<1>(r, hi, lo, sa, g, acc);
}

MOEW2_DEV void prime_gu(GuTileRegs (&ring)[kRing], const WaveTiles<2>& wt, int kb, int ke, int lane) {
#pragma unroll
  for (int i = 0; i < kRing; ++i) load_gu_tile(ring[i], wt, kb + i, kb + i < ke, lane);
}

MOEW2_DEV void stream_gu(GuTileRegs (&ring)[kRing], const WaveTiles<2>& wt, int kb, int ke, const uint8_t* arow,
                         int K, int g, f32x4_t* acc, int lane) {
  for (int k0 = kb; k0 < ke; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kt = k0 + i;
      if (kt < ke) mma_gu_tile(ring[i], arow, K, kt, g, acc);
      load_gu_tile(ring[i], wt, kt + kRing, kt + kRing < ke, lane);
    }
  }
}

// Quantizing commit of staged bf16 pieces (8 values each): the 4 pieces of a 32-value block sit
// in 4 consecutive lanes, which agree on the block maximum through two lane swaps.
template <int NT>
MOEW2_DEV void stage_commit_x8(const Stage& st, uint8_t* lds, int stride, int K, int n, int base, int tid) {
  const int per_row = K / 8, total = n * per_row;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int idx = base + i * NT + tid;
    const bool ok = idx < total;
    const u32x4_t v = st.v[i];
    float a = 0.f;
    if (ok) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[q])), __builtin_fabsf(bf16_hi(v[q]))));
    }
    a = __builtin_fmaxf(a, __shfl_xor(a, 1, 64));
    a = __builtin_fmaxf(a, __shfl_xor(a, 2, 64));
    if (ok) {
      const int m = idx / per_row, c8 = idx - m * per_row;
      const uint32_t sx = x_scale_byte(a);
      uint32_t h0, l0, h1, l1;
      x_split4(bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1]), sx, h0, l0);
      x_split4(bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3]), sx, h1, l1);
      uint8_t* row = lds + (size_t)m * stride;
      *reinterpret_cast<u32x2_t*>(row + 8 * c8) = u32x2_t{h0, h1};
      *reinterpret_cast<u32x2_t*>(row + K + 8 * c8) = u32x2_t{l0, l1};
      if ((c8 & 3) == 0) {
        const int b = c8 >> 2, kt = b >> 3, d = b & 7, gg = d & 3, c = d >> 2;
        uint8_t* sw = row + 2 * K + kt * 16 + 4 * gg;
        sw[c] = (uint8_t)sx;
        sw[2 + c] = (uint8_t)x_lo_scale_byte(sx);
      }
    }
    // one piece at a time: interleaving the pieces' conversions would raise the register peak
    // while the weight ring is in flight
    __builtin_amdgcn_sched_barrier(0);
  }
}

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
  int e, n_total, row0;
  if (DIRECT) {
    row0 = blockIdx.y;             // the pair
    e = ids[row0];
    if (e < 0 || e >= E) return;
    n_total = 1;
  } else {
    if ((int)blockIdx.y >= meta[0]) return;
    e = active[blockIdx.y];
    row0 = offsets[e];
    n_total = offsets[e + 1] - row0;
  }
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  const int pw = w / KS, ks = w % KS;
  const int q = blockIdx.x * NP + pw;
  WaveTiles<2> wt = wave_tiles<2>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * q * nkt);
  wt.tile[1] = (uint32_t)((2 * q + 1) * nkt);
  const int kb = ks * nkt / KS, ke = (ks + 1) * nkt / KS;
  const int stride = gu_row_stride(K);
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][2][4][16]
  GuTileRegs ring[kRing];
  for (int c0 = 0; c0 < n_total; c0 += kChunk) {
    const int n = min(kChunk, n_total - c0);
    // token of each staged row (wave-uniform loads)
    int tk[kChunk];
#pragma unroll
    for (int m = 0; m < kChunk; ++m) tk[m] = (DIRECT ? row0 : perm[row0 + c0 + min(m, n - 1)]) / top_k;
    auto row_off = [&](int m) -> size_t {
      const int t = m == 0 ? tk[0] : m == 1 ? tk[1] : m == 2 ? tk[2] : tk[3];
      return (size_t)t * K;
    };
    // staging (extra batches first, the last one overlapped with the ring prime; see
    // stage_and_prime), quantized to the hi / lo parts on the way into LDS. The thread index
    // is passed through an empty asm so that the staging addresses are recomputed here instead
    // of being hoisted out of the chunk loop and held in registers across the stream.
    int st_tid = tid;
    asm volatile("" : "+v"(st_tid));
    Stage st;
    for (int base = kStage * kThreads; base < n * (K / 8); base += kStage * kThreads) {
      stage_issue<kThreads>(st, x, K, n, base, row_off, st_tid);
      stage_commit_x8<kThreads>(st, lds, stride, K, n, base, st_tid);
    }
    stage_issue<kThreads>(st, x, K, n, 0, row_off, st_tid);
    prime_gu(ring, wt, kb, ke, lane);
    stage_commit_x8<kThreads>(st, lds, stride, K, n, 0, st_tid);
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    stream_gu(ring, wt, kb, ke, lds + (size_t)ma * stride, K, lane >> 4, acc, lane);
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
          const int row = DIRECT ? row0 : row0 + c0 + r;
          act[(size_t)row * I + 16 * q + lane] = h;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// routed down: grid (K / (32*NP), active slots). Wave w handles row groups 2*rq and 2*rq + 1,
// rq = blockIdx.x*NP + w/KS, over the reduction slice w%KS. Per-pair rows go to pair_out at the
// pair index (bijective); combine_kernel then sums them per token in j order.
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  if ((int)blockIdx.y >= meta[0]) return;
  const int e = active[blockIdx.y];
  const int row0 = offsets[e];
  const int n_e = offsets[e + 1] - row0;
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int pw = w / KS, ks = w % KS;
  const int rq = blockIdx.x * NP + pw;
  WaveTiles<2> wt = wave_tiles<2>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * rq * nkt);
  wt.tile[1] = (uint32_t)((2 * rq + 1) * nkt);
  const int kb = ks * nkt / KS, ke = (ks + 1) * nkt / KS;
  const int stride = I * 2 + 16;
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][2][4][16]
  const uint16_t* act16 = reinterpret_cast<const uint16_t*>(act);
  TileRegs ring[kRing];
  for (int c0 = 0; c0 < n_e; c0 += kChunk) {
    const int n = min(kChunk, n_e - c0);
    auto row_off = [&](int m) -> size_t { return (size_t)(row0 + c0 + m) * I; };
    stage_and_prime<kThreads, 2>(ring, wt, kb, ke, lane, lds, stride, act16, I, n, row_off, tid);
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    const uint8_t* a_row = lds + (size_t)ma * stride + (size_t)(8 * (lane >> 4)) * 2;
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    stream_k<F16Op, 2>(ring, wt, kb, ke, a_row, acc, lane);
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
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = 16 * (2 * rq + b) + lane;
        const int e0 = dn_e0[(size_t)e * K + col];
#pragma unroll
        for (int r = 0; r < kChunk; ++r) {
          if (r < n) {
            const int p = perm[row0 + c0 + r];
            pair_out[(size_t)p * K + col] = __builtin_ldexpf(acc[b][r], e0);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// direct down + combine for tiny batches: grid (K/16). The workgroup covers one row group of 16
// output columns for every pair; wave w takes pair w/2 and half w%2 of the reduction; per-pair
// results meet in LDS and are combined per token in j order. Block 0 also records the two
// counters (single writer).
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int rg = blockIdx.x, col = 16 * rg + (lane & 15);
  const int stride = I * 2 + 16;
  float* o = reinterpret_cast<float*>(lds + (size_t)kDirectMaxPairs * stride);  // [P][16]
  float* red = o + kDirectMaxPairs * 16;                                        // [P][4][16]
  // wave w: pair p = w / 2, reduction half w % 2
  const int p = w >> 1, hk = w & 1;
  const int id = p < P ? ids[p] : -1;
  const bool valid = id >= 0 && id < E;
  WaveTiles<1> wt = wave_tiles<1>(codes, scales, valid ? id : 0, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(rg * nkt);
  const int kb = hk * nkt / 2, ke = valid ? (hk + 1) * nkt / 2 : kb;
  const int e0 = valid ? dn_e0[(size_t)id * K + col] : 0;
  // gated rows of all pairs (rows of invalid pairs are staged but never read)
  const uint16_t* act16 = reinterpret_cast<const uint16_t*>(act);
  auto row_off = [&](int m) -> size_t { return (size_t)m * I; };
  TileRegs ring[kRing];
  stage_and_prime<kDirectThreads, 1>(ring, wt, kb, ke, lane, lds, stride, act16, I, P, row_off, tid);
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
  const uint8_t* a_row = lds + (size_t)(p < P ? p : 0) * stride + (size_t)(8 * (lane >> 4)) * 2;
  stream_k<F16Op, 1>(ring, wt, kb, ke, a_row, acc, lane);
  if (valid && hk == 1 && lane < 16) red[p * 16 + lane] = acc[0][0];
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
// One thread per 4 output columns of one token. A group of up to 8 pairs has its ids, weights and
// pair rows requested together (rows of invalid pairs are read but not used), so a token costs
// one memory round trip per 8 pairs; the sum itself runs in ascending j.
__global__ void combine_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wts,
                               const float* __restrict__ pair_out, void* __restrict__ y,
                               int T, int top_k, int E, int K, int out_dtype) {
  constexpr int G = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = K / 4;
  if (gid >= (long long)T * q) return;
  const int t = (int)(gid / q), c = (int)(gid - (long long)t * q) * 4;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int j0 = 0; j0 < top_k; j0 += G) {
    int id[G];
    float w[G];
    float4 o[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (j0 + i < top_k) {
        const int p = t * top_k + j0 + i;
        id[i] = ids[p];
        w[i] = wts[p];
        o[i] = *reinterpret_cast<const float4*>(pair_out + (size_t)p * K + c);
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (j0 + i < top_k && id[i] >= 0 && id[i] < E) {
        acc0 += w[i] * o[i].x; acc1 += w[i] * o[i].y; acc2 += w[i] * o[i].z; acc3 += w[i] * o[i].w;
      }
    }
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
  const size_t lds = (size_t)kChunk * gu_row_stride(p->K) + (size_t)kWaves * 2 * 4 * 16 * 4;
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
  const size_t lds = (size_t)kChunk * (p->I * 2 + 16) + (size_t)kWaves * 2 * 4 * 16 * 4;
  const int np = pick_np(slots);
  auto args = [&](auto kern, int gx) {
    hipLaunchKernelGGL(kern, dim3(gx, slots), dim3(kThreads), lds, s,
                       p->dn_codes, p->dn_scales, p->dn_e0, act,
                       (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                       (const int32_t*)(wsb + ws.active), (const int32_t*)(wsb + ws.meta),
                       (float*)(wsb + ws.pair_out), p->E, p->K, p->I, top_k);
  };
  if (np == 4) args(decode_down_kernel<4>, p->K / 128);
  else args(decode_down_kernel<1>, p->K / 32);
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
