// Prefill-shaped grouped expert GEMMs (many tokens per expert), on the gfx950 matrix cores.
//
// Each workgroup computes a BM x BN tile of one expert: BM consecutive sorted pair rows (an
// M-tile from the routing pass) by BN weight rows. The A operand (activations) is staged through
// LDS one 256-wide k-tile at a time, double-buffered; for gate_up the rows are gathered from the
// split x through the sort permutation while they are staged, so gathered activations never
// round-trip through HBM (the pages' AFRAG variant repacks activations fragment-major in a
// separate pass - README bullet "The kernels", "The v0.24.0 port" bullet "AFRAG prefill"; here
// the LDS staging plays that role and every lane's A fragment is one 16-byte LDS read). The B
// operand (2-bit weights) is read by each wave straight from the native planes.
//
//  gate_up: block-scaled fp8 x fp4 instruction; x is first split into two e4m3 parts by
//           quant_x_kernel (one pass over x), the weights' codes become e2m1 operands with two
//           bit operations per 8 values and their UE8M0 bytes are the instruction's B scales.
//  down:    the same instruction with the gated intermediate (fp16) split into three e4m3 parts
//           by quant_act_kernel.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int BM = kGemmBM;     // 64 sorted pair rows (4 MFMA row tiles)
constexpr int kWaves = 8;       // each wave: all BM rows x 64 weight rows (4 row groups of 16)
constexpr int BN = 64 * kWaves; // 512 weight rows per workgroup
constexpr int kThreads = 64 * kWaves;

// Tile shape: the 2-bit weights cost 0.28 byte per element against 2 bytes for the activations,
// so the workgroup tile is wide in N (512 weight rows) and short in M (64 rows).
//
// The workgroup -> tile mapping is XCD-aware: consecutive workgroup ids are dispatched to the
// 8 XCDs in turn, so workgroup b takes logical tile (b % 8) * per_xcd + b / 8. Each XCD then walks
// a contiguous run of (M-tile, N-block) pairs, N-block fastest: the N-blocks of one M-tile run on
// one XCD at about the same time and read the M-tile's activations from that XCD's L2 once.
struct TileMap {
  int e, rs, rows_valid, nb;
  bool live;
};
MOEW2_DEV TileMap map_tile(const int32_t* tiles, const int32_t* meta, const int32_t* offsets, int n_blocks) {
  TileMap m;
  const int n_tiles = meta[1];
  const int total = n_tiles * n_blocks;
  const int per_xcd = (total + 7) / 8;
  const int b = blockIdx.x;
  const int logical = (b & 7) * per_xcd + (b >> 3);
  m.live = (b >> 3) < per_xcd && logical < total;
  if (!m.live) return m;
  const int ti = logical / n_blocks;
  m.nb = logical - ti * n_blocks;
  m.e = tiles[2 * ti];
  m.rs = tiles[2 * ti + 1];
  m.rows_valid = min(BM, offsets[m.e + 1] - m.rs);
  return m;
}

// ------------------------------------------------------------------------------------------------
// x split: one thread per 32-value block of x (layout of the workspace region in internal.h).
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
quant_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, int T, int K) {
  const int nb = K / 32;
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (long long)T * nb) return;
  const int t = (int)(b / nb), blk = (int)(b - (long long)t * nb);
  const uint16_t* src = x + (size_t)t * K + 32 * blk;
  u32x4_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = ld16(src + 8 * q);
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[q][j])), __builtin_fabsf(bf16_hi(v[q][j]))));
  const uint32_t sx = x_scale_byte(a);
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x_split4(bf16_lo(v[q][0]), bf16_hi(v[q][0]), bf16_lo(v[q][1]), bf16_hi(v[q][1]), sx, hi[2 * q], lo[2 * q]);
    x_split4(bf16_lo(v[q][2]), bf16_hi(v[q][2]), bf16_lo(v[q][3]), bf16_hi(v[q][3]), sx, hi[2 * q + 1], lo[2 * q + 1]);
  }
  uint8_t* dh = xq + (size_t)t * K + 32 * blk;
  uint8_t* dl = dh + (size_t)T * K;
  *reinterpret_cast<u32x4_t*>(dh) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<u32x4_t*>(dh + 16) = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
  *reinterpret_cast<u32x4_t*>(dl) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  *reinterpret_cast<u32x4_t*>(dl + 16) = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
  const int kt = blk >> 3, d = blk & 7, g = d & 3, c = d >> 2;
  uint8_t* sw = xq + 2 * (size_t)T * K + ((size_t)t * (K / kTileK) + kt) * 16 + 4 * g;
  sw[c] = (uint8_t)sx;
  sw[2 + c] = (uint8_t)x_lo_scale_byte(sx);
}

// ------------------------------------------------------------------------------------------------
// gate_up (block-scaled). LDS row of one k-tile: hi [256] | lo [256] | scale words [4][4] | pad.
// ------------------------------------------------------------------------------------------------
constexpr int kMxStride = 2 * kTileK + 16 + 16;
constexpr int kMxABytes = BM * kMxStride;

__global__ void __launch_bounds__(kThreads, 1)
gemm_gate_up_mx_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       const uint8_t* __restrict__ xq, const int32_t* __restrict__ offsets,
                       const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                       const int32_t* __restrict__ meta, _Float16* __restrict__ act,
                       long long* __restrict__ counters, int T, int K, int I, int top_k, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kMxABytes];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  // row groups 4*(nb*kWaves + w) .. +3 of this wave (gate, up, gate, up)
  const int rg0 = 4 * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;   // a matrix with fewer than BN rows leaves waves idle

  // ---- A staging: piece p (16 bytes) = tid % 32 of rows tid/32 + 16*i (p < 16: hi, else lo);
  //      threads 0..63 also copy row tid's 16 scale-word bytes ----
  const int piece = tid & 31;
  const size_t part = piece < 16 ? 16 * piece : (size_t)T * K + 16 * (piece - 16);
  const uint8_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tid / 32 + 16 * i;
    const int tok = perm[rs + min(r, rows_valid - 1)] / top_k;
    asrc[i] = xq + (size_t)tok * K + part;
  }
  const int srow = min(tid, BM - 1);
  const uint8_t* ssrc = xq + 2 * (size_t)T * K + (size_t)(perm[rs + min(srow, rows_valid - 1)] / top_k) * (nkt * 16);
  u32x4_t areg[4], sreg;
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) areg[i] = ld16(asrc[i] + kt * kTileK);
    if (tid < BM) sreg = ld16(ssrc + kt * 16);
  };
  auto store_a = [&](int buf) {
    uint8_t* base = lds + buf * kMxABytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(base + (tid / 32 + 16 * i) * kMxStride + 16 * piece) = areg[i];
    if (tid < BM) *reinterpret_cast<u32x4_t*>(base + tid * kMxStride + 2 * kTileK) = sreg;
  };

  // ---- B: 4 row groups per wave, one native k-tile at a time, in two register sets ----
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;
  struct BRegs { u32x4_t c[4]; uint32_t s[4]; };
  BRegs bA, bB;
  auto load_b = [&](int kt, BRegs& r) {
    if (!wave_active) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const size_t ti = tb0 + (size_t)t * nkt + kt;
      r.c[t] = ld16(codes + ti * kTileCodeBytes + 16 * lane);
      r.s[t] = *reinterpret_cast<const uint16_t*>(scales + ti * kTileScaleBytes + 2 * lane);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto chunk = [&](const uint8_t* abuf, const BRegs& br, auto cc) {
    constexpr int C = decltype(cc)::value;
    i32x8_t bo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bo[t] = mx_b_operand(br.c[t][2 * C], br.c[t][2 * C + 1]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* ar = abuf + (m * 16 + (lane & 15)) * kMxStride;
      const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(ar + 128 * C + 16 * g);
      const u32x4_t h1 = *reinterpret_cast<const u32x4_t*>(ar + 128 * C + 64 + 16 * g);
      const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(ar + kTileK + 128 * C + 16 * g);
      const u32x4_t l1 = *reinterpret_cast<const u32x4_t*>(ar + kTileK + 128 * C + 64 + 16 * g);
      const uint32_t sa = *reinterpret_cast<const uint32_t*>(ar + 2 * kTileK + 4 * g);
      const i32x8_t ah = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      const i32x8_t al = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[m][t] = mx_mfma<C, C>(ah, bo[t], acc[m][t], sa, br.s[t]);
        acc[m][t] = mx_mfma<2 + C, C>(al, bo[t], acc[m][t], sa, br.s[t]);
      }
    }
  };
  // k-tile kt computes from LDS buffer kt % 2 with B from `cur` (loaded one k-tile earlier);
  // meanwhile A and B of k-tile kt+1 are in flight and A lands in the other buffer at the end.
  auto k_tile = [&](int kt, const BRegs& cur, BRegs& nxt) {
    const bool more = kt + 1 < nkt;
    if (more) { load_b(kt + 1, nxt); load_a(kt + 1); }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) {
      chunk(lds + (kt & 1) * kMxABytes, cur, std::integral_constant<int, 0>());
      chunk(lds + (kt & 1) * kMxABytes, cur, std::integral_constant<int, 1>());
    }
    if (more) store_a((kt + 1) & 1);
    __syncthreads();
  };

  load_b(0, bA);
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += 2) {
    k_tile(kt, bA, bB);
    if (kt + 1 < nkt) k_tile(kt + 1, bB, bA);
  }
  if (!wave_active) return;

  // ---- epilogue: a = silu(g) * u in fp16 at the sorted row ----
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int sr = rs + row;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const float a = silu_mul(acc[m][2 * pr][r], acc[m][2 * pr + 1][r]);
        const _Float16 h = (_Float16)a;
        if (__builtin_isinf((float)h)) atomicAdd((unsigned long long*)&counters[1], 1ull);
        const int col = 16 * (rg0 / 2 + pr) + (lane & 15);
        act[(size_t)sr * I + col] = h;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// gated intermediate split: one thread per 32-value block of act [P][I] (fp16), three parts
// (layout of the workspace region in internal.h).
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
quant_act_kernel(const uint16_t* __restrict__ act, uint8_t* __restrict__ aq, int P, int I) {
  const int nb = I / 32;
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (long long)P * nb) return;
  const int r = (int)(b / nb), blk = (int)(b - (long long)r * nb);
  const uint16_t* src = act + (size_t)r * I + 32 * blk;
  u32x4_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = ld16(src + 8 * q);
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(f16_lo(v[q][j])), __builtin_fabsf(f16_hi(v[q][j]))));
  const uint32_t sa = x_scale_byte(a);
  uint32_t p0[8], p1[8], p2[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a_split4(f16_lo(v[q][0]), f16_hi(v[q][0]), f16_lo(v[q][1]), f16_hi(v[q][1]), sa, p0[2 * q], p1[2 * q], p2[2 * q]);
    a_split4(f16_lo(v[q][2]), f16_hi(v[q][2]), f16_lo(v[q][3]), f16_hi(v[q][3]), sa, p0[2 * q + 1], p1[2 * q + 1],
             p2[2 * q + 1]);
  }
  const size_t part = (size_t)P * I;
  uint8_t* d0 = aq + (size_t)r * I + 32 * blk;
  *reinterpret_cast<u32x4_t*>(d0) = u32x4_t{p0[0], p0[1], p0[2], p0[3]};
  *reinterpret_cast<u32x4_t*>(d0 + 16) = u32x4_t{p0[4], p0[5], p0[6], p0[7]};
  *reinterpret_cast<u32x4_t*>(d0 + part) = u32x4_t{p1[0], p1[1], p1[2], p1[3]};
  *reinterpret_cast<u32x4_t*>(d0 + part + 16) = u32x4_t{p1[4], p1[5], p1[6], p1[7]};
  *reinterpret_cast<u32x4_t*>(d0 + 2 * part) = u32x4_t{p2[0], p2[1], p2[2], p2[3]};
  *reinterpret_cast<u32x4_t*>(d0 + 2 * part + 16) = u32x4_t{p2[4], p2[5], p2[6], p2[7]};
  const int kt = blk >> 3, d = blk & 7, g = d & 3, c = d >> 2;
  uint8_t* sw = aq + 3 * part + ((size_t)r * (I / kTileK) + kt) * 32 + 8 * g;
  sw[c] = (uint8_t)sa;
  sw[2 + c] = (uint8_t)a_part_scale(sa, 1);
  sw[4 + c] = (uint8_t)a_part_scale(sa, 2);
}

// ------------------------------------------------------------------------------------------------
// down (block-scaled, three parts). LDS row of one k-tile: part 0 [256] | part 1 [256] |
// part 2 [256] | scale words [4][8] | pad.
// ------------------------------------------------------------------------------------------------
constexpr int kDnStride = 3 * kTileK + 32 + 16;
constexpr int kDnABytes = BM * kDnStride;
constexpr int kDnPieces = BM * 48 / kThreads;   // 16-byte part pieces per thread per k-tile
static_assert(kDnPieces == 6, "down A staging layout");

__global__ void __launch_bounds__(kThreads, 1)
gemm_down_mx_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                    const uint8_t* __restrict__ aq, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                    const int32_t* __restrict__ meta, float* __restrict__ pair_out, int P, int K, int I,
                    int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int rg0 = 4 * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;

  // ---- A staging: thread t copies 16-byte slot t % 16 of part q of rows t/16 and t/16 + 32
  //      (pieces i = 0..5: q = i/2, row half i%2); threads 0..127 also copy half (t % 2) of
  //      row t/2's 32 scale-word bytes ----
  const size_t part = (size_t)P * I;
  const int sl = tid & 15;
  size_t arow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) arow[h] = (size_t)(rs + min((tid >> 4) + 32 * h, rows_valid - 1)) * I + 16 * sl;
  const int srow = min(tid >> 1, BM - 1);
  const uint8_t* ssrc = aq + 3 * part + (size_t)(rs + min(srow, rows_valid - 1)) * (nkt * 32) + 16 * (tid & 1);
  u32x4_t areg[kDnPieces], sreg;
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kDnPieces; ++i) areg[i] = ld16(aq + (i >> 1) * part + arow[i & 1] + kt * kTileK);
    if (tid < 2 * BM) sreg = ld16(ssrc + kt * 32);
  };
  auto store_a = [&](int buf) {
    uint8_t* base = lds + buf * kDnABytes + (tid >> 4) * kDnStride + 16 * sl;
#pragma unroll
    for (int i = 0; i < kDnPieces; ++i)
      *reinterpret_cast<u32x4_t*>(base + (i & 1) * 32 * kDnStride + (i >> 1) * kTileK) = areg[i];
    if (tid < 2 * BM) *reinterpret_cast<u32x4_t*>(lds + buf * kDnABytes + (tid >> 1) * kDnStride + 3 * kTileK + 16 * (tid & 1)) = sreg;
  };

  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;
  struct BRegs { u32x4_t c[4]; uint32_t s[4]; };
  BRegs bA, bB;
  auto load_b = [&](int kt, BRegs& r) {
    if (!wave_active) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const size_t ti = tb0 + (size_t)t * nkt + kt;
      r.c[t] = ld16(codes + ti * kTileCodeBytes + 16 * lane);
      r.s[t] = *reinterpret_cast<const uint16_t*>(scales + ti * kTileScaleBytes + 2 * lane);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto chunk = [&](const uint8_t* abuf, const BRegs& br, auto cc) {
    constexpr int C = decltype(cc)::value;
    i32x8_t bo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bo[t] = mx_b_operand(br.c[t][2 * C], br.c[t][2 * C + 1]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* ar = abuf + (m * 16 + (lane & 15)) * kDnStride;
      const u32x2_t sw = *reinterpret_cast<const u32x2_t*>(ar + 3 * kTileK + 8 * g);
      i32x8_t ap[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(ar + q * kTileK + 128 * C + 16 * g);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(ar + q * kTileK + 128 * C + 64 + 16 * g);
        ap[q] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[m][t] = mx_mfma<C, C>(ap[0], bo[t], acc[m][t], sw[0], br.s[t]);
        acc[m][t] = mx_mfma<2 + C, C>(ap[1], bo[t], acc[m][t], sw[0], br.s[t]);
        acc[m][t] = mx_mfma<C, C>(ap[2], bo[t], acc[m][t], sw[1], br.s[t]);
      }
    }
  };
  auto k_tile = [&](int kt, const BRegs& cur, BRegs& nxt) {
    const bool more = kt + 1 < nkt;
    if (more) { load_b(kt + 1, nxt); load_a(kt + 1); }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) {
      chunk(lds + (kt & 1) * kDnABytes, cur, std::integral_constant<int, 0>());
      chunk(lds + (kt & 1) * kDnABytes, cur, std::integral_constant<int, 1>());
    }
    if (more) store_a((kt + 1) & 1);
    __syncthreads();
  };

  load_b(0, bA);
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += 2) {
    k_tile(kt, bA, bB);
    if (kt + 1 < nkt) k_tile(kt + 1, bB, bA);
  }
  if (!wave_active) return;

  // ---- epilogue: per-pair rows at the pair index ----
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int p = perm[rs + row];
#pragma unroll
      for (int t = 0; t < 4; ++t) pair_out[(size_t)p * K + 16 * (rg0 + t) + (lane & 15)] = acc[m][t][r];
    }
  }
}

}  // namespace

inline unsigned gemm_grid(int max_tiles, int n_blocks) {
  const long long g = (long long)max_tiles * n_blocks;
  return (unsigned)((g + 7) / 8 * 8);
}

hipError_t launch_gemm_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                               const Workspace& ws, uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  const long long nblk32 = (long long)T * (p->K / 32);
  hipLaunchKernelGGL(quant_x_kernel, dim3((unsigned)((nblk32 + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)x, wsb + ws.xq, T, p->K);
  const int nblk = (2 * p->I + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_gate_up_mx_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads), 0, s,
                     p->gu_codes, p->gu_scales, (const uint8_t*)(wsb + ws.xq),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (_Float16*)(wsb + ws.act), (long long*)(wsb + ws.counters), T, p->K, p->I, top_k, nblk);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                            uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  const int P = T * top_k;
  const long long nblk32 = (long long)P * (p->I / 32);
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((nblk32 + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)(wsb + ws.act), wsb + ws.aq, P, p->I);
  const int nblk = (p->K + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_down_mx_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads), 2 * kDnABytes, s,
                     p->dn_codes, p->dn_scales, (const uint8_t*)(wsb + ws.aq),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (float*)(wsb + ws.pair_out), P, p->K, p->I, nblk);
  return hipGetLastError();
}

}  // namespace moew2
