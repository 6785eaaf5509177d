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
// A-operand pipeline shared by both GEMMs. The A tile of one k-tile (BM rows) is one LDS stage of
// BM * CH 16-byte chunks, row r at chunk r*CH. An operand read has lane l take 16 bytes of row
// l % 16 at chunk offset l / 16 (+ const); on gfx950 such reads run without bank conflicts when
// the row stride is an odd multiple of 32 bytes (measured with the LDS bank-conflict counter:
// strides of 528 or 816 bytes cost ~3 conflict cycles per read, 544 and 800 none). The split
// activations are laid
// out per (row, k-tile) as SRC contiguous chunks, so a stage is filled by direct global -> LDS
// loads: wave-instruction j writes chunks 64j .. 64j+63, lane i chunk 64j+i, from the source chunk
// of that (row, chunk) (chunks past SRC repeat the last one; they pad the stride only).
// kStages stages rotate; k-tile kt+2 is requested while kt is computed, and the B registers of
// each wave rotate the same way. Every wave issues the same loads every k-tile (the tail repeats
// the last k-tile into a free stage), so the counted waits below are exact.
// ------------------------------------------------------------------------------------------------
constexpr int kStages = 3;

// waits until at most N vector memory operations of this wave are outstanding
template <int N>
MOEW2_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int CH, int SRC>
struct ATile {
  static constexpr int kChunks = BM * CH;
  static constexpr int kBytes = kChunks * 16;
  static constexpr int kInstr = (kChunks + 63) / 64;       // wave-instructions per stage
  static constexpr int kPerWave = (kInstr + kWaves - 1) / kWaves;
  static constexpr int kSrcBytes = SRC * 16;              // one (row, k-tile) block of the source
  static_assert(kChunks % 64 == 0, "a stage is a whole number of wave-instructions");
};

// Per-lane source byte offsets (k-tile 0) of this wave's DMA instructions; instruction i of wave
// w is j = min(w + kWaves*i, kInstr - 1). rowoff(r) is the offset of tile row r's first block.
// The offsets are 32-bit: the forward entry point keeps the split activations below 4 GiB.
template <class AT, class RowOff>
MOEW2_DEV void a_sources(uint32_t (&off)[AT::kPerWave], int w, int lane, RowOff rowoff) {
  constexpr int CH = AT::kChunks / BM, SRC = AT::kSrcBytes / 16;
#pragma unroll
  for (int i = 0; i < AT::kPerWave; ++i) {
    const int j = min(w + kWaves * i, AT::kInstr - 1);
    const int q = min(64 * j + lane, AT::kChunks - 1);
    const int r = q / CH, c = q - r * CH;
    off[i] = rowoff(r) + 16u * (uint32_t)min(c, SRC - 1);
  }
}

// B: the 4 row groups of a wave, one native k-tile
struct BRegs {
  u32x4_t c[4];
  uint32_t s[4];
};
constexpr int kBLoads = 8;   // vector memory instructions for one BRegs
constexpr int kGroups = 8;   // instruction groups per k-tile: 2 columns C x 4 row tiles m

template <int I, int N, class F>
MOEW2_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// The loads of one k-tile for one wave, as kItems single instructions: the B code and scale loads,
// then the stage's DMA instructions (waves whose last instruction index lies past the stage
// repeat the stage's last instruction - the same bytes to the same chunks - so every wave issues
// kPerWave). Group i of the computing k-tile issues items [i*kItems/8, (i+1)*kItems/8)
// of the k-tile two ahead, so the loads spread over the step instead of queueing behind the
// barrier.
template <class AT>
struct KLoads {
  static constexpr int kItems = AT::kPerWave + kBLoads;
  const uint8_t* abase;
  const uint32_t* aoff;
  const uint8_t* codes;
  const uint8_t* scales;
  size_t tb0;
  int nkt, w, lane;

  template <int N>
  MOEW2_DEV void item(int kt, uint8_t* stage, BRegs& r) const {
    if constexpr (N < kBLoads) {       // B first: it comes from HBM, A mostly from L2
      constexpr int t = N / 2;
      const size_t ti = tb0 + (size_t)t * nkt + kt;
      if constexpr (N % 2 == 0)
        r.c[t] = ld16(codes + ti * kTileCodeBytes + 16 * lane);
      else
        r.s[t] = *reinterpret_cast<const uint16_t*>(scales + ti * kTileScaleBytes + 2 * lane);
    } else {
      constexpr int n = N - kBLoads;
      const int j = min(w + kWaves * n, AT::kInstr - 1);
      __builtin_amdgcn_global_load_lds((const void*)(abase + (aoff[n] + (uint32_t)kt * AT::kSrcBytes)),
                                       (__attribute__((address_space(3))) void*)(stage + 1024 * j), 16, 0, 0);
    }
  }
  template <int N0, int N1>
  MOEW2_DEV void items(int kt, uint8_t* stage, BRegs& r) const {
    if constexpr (N0 < N1) {
      item<N0>(kt, stage, r);
      items<N0 + 1, N1>(kt, stage, r);
    }
  }
  template <int I>
  MOEW2_DEV void group(int kt, uint8_t* stage, BRegs& r) const {
    items<I * kItems / kGroups, (I + 1) * kItems / kGroups>(kt, stage, r);
  }
};

// The k-loop: COMPUTE(stage, BRegs, part, mma) for every step, where part(integral_constant<I>)
// issues load group I of the k-tile two ahead (COMPUTE calls it for I = 0..7 in order, always)
// and mma says whether the step has a k-tile to multiply (not the first two steps, the tail of
// the last round or idle waves). K-tile j uses stage j % kStages and register set j % kStages.
template <class AT, class Compute>
MOEW2_DEV void k_loop(uint8_t* lds, const KLoads<AT>& ld, int nkt, bool active, Compute compute) {
  BRegs b0, b1, b2;
  auto step = [&](int kt, BRegs& cur, BRegs& ahead) {
    // k-tile kt has landed (the loads of kt + 1, issued after it, may still be in flight)
    wait_vm<KLoads<AT>::kItems>();
    __builtin_amdgcn_s_barrier();      // ... in every wave; and every wave is done with kt - 1
    const int kc = min(kt + 2, nkt - 1);
    uint8_t* ahead_stage = lds + ((kt + 2) % kStages) * AT::kBytes;   // the stage kt - 1 used
    auto part = [&](auto ic) { ld.template group<decltype(ic)::value>(kc, ahead_stage, ahead); };
    // Every step runs the same instruction stream except the matrix instructions themselves: the
    // loads and LDS reads are unconditional (a step without a k-tile reads a stale stage), so the
    // compiler's count of outstanding loads stays exact and no operand needs a merge copy.
    const bool mma = active && kt >= 0 && kt < nkt;
    compute(lds + ((kt + kStages) % kStages) * AT::kBytes, cur, part, mma);
  };
  // Whole rounds of kStages steps, so that every round issues and waits alike: the first round's
  // first two steps only issue k-tiles 0 and 1, steps past the last k-tile only load repeats of
  // it. (With the first two issues peeled off before the loop, the compiler's own wait analysis
  // lost track of the stage writes across the loop entry and drained every load once a round.)
  for (int kt = -2; kt < nkt; kt += 3) {
    step(kt, b1, b0);
    step(kt + 1, b2, b1);
    step(kt + 2, b0, b2);
  }
  wait_vm<0>();                        // no DMA may still target this workgroup's LDS
}

// ------------------------------------------------------------------------------------------------
// x split: one thread per 32-value block of x. Output per (token, k-tile): hi [256] | lo [256] |
// scale words [4][4] (hi c0, hi c1, lo c0, lo c1 for lane group g).
// ------------------------------------------------------------------------------------------------
constexpr int kGuSrc = 33;   // 16-byte chunks per (token, k-tile)

__global__ void __launch_bounds__(256)
quant_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, int T, int K) {
  const int nb = K / 32, nkt = K / kTileK;
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
  const int kt = blk >> 3, d = blk & 7, g = d & 3, c = d >> 2;
  uint8_t* blkp = xq + ((size_t)t * nkt + kt) * (16 * kGuSrc);
  uint8_t* dh = blkp + 32 * d;
  uint8_t* dl = dh + kTileK;
  *reinterpret_cast<u32x4_t*>(dh) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  *reinterpret_cast<u32x4_t*>(dh + 16) = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
  *reinterpret_cast<u32x4_t*>(dl) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  *reinterpret_cast<u32x4_t*>(dl + 16) = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
  uint8_t* sw = blkp + 2 * kTileK + 4 * g;
  sw[c] = (uint8_t)sx;
  sw[2 + c] = (uint8_t)x_lo_scale_byte(sx);
}

// ------------------------------------------------------------------------------------------------
// gate_up (block-scaled). LDS row of one k-tile: hi [256] | lo [256] | scale words [4][4] | pad
// (34 chunks, 544 bytes).
// ------------------------------------------------------------------------------------------------
using GuTile = ATile<kGuSrc + 1, kGuSrc>;
constexpr int kMxStride = 16 * (kGuSrc + 1);

__global__ void __launch_bounds__(kThreads, 1)
gemm_gate_up_mx_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       const uint8_t* __restrict__ xq, const int32_t* __restrict__ offsets,
                       const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                       const int32_t* __restrict__ meta, _Float16* __restrict__ act,
                       long long* __restrict__ counters, int T, int K, int I, int top_k, int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  // row groups 4*(nb*kWaves + w) .. +3 of this wave (gate, up, gate, up); a matrix with fewer
  // than BN rows leaves waves idle (they still load a valid row group to keep the waits exact)
  const int rg0 = 4 * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[GuTile::kPerWave];
  a_sources<GuTile>(aoff, w, lane, [&](int r) {
    const int tok = perm[rs + min(r, rows_valid - 1)] / top_k;
    return (uint32_t)tok * (uint32_t)(nkt * GuTile::kSrcBytes);
  });

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A operand of row tile m, instruction C of the k-tile: hi and lo parts and their scale word
  struct AOp {
    i32x8_t h, l;
    uint32_t s;
  };
  auto a_load = [&](const uint8_t* abuf, int m, int C) {
    const uint8_t* ar = abuf + (m * 16 + (lane & 15)) * kMxStride;
    const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(ar + 128 * C + 16 * g);
    const u32x4_t h1 = *reinterpret_cast<const u32x4_t*>(ar + 128 * C + 64 + 16 * g);
    const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(ar + kTileK + 128 * C + 16 * g);
    const u32x4_t l1 = *reinterpret_cast<const u32x4_t*>(ar + kTileK + 128 * C + 64 + 16 * g);
    AOp a;
    a.s = *reinterpret_cast<const uint32_t*>(ar + 2 * kTileK + 4 * g);
    a.h = i32x8_t{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
    a.l = i32x8_t{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
    return a;
  };
  // One instruction column C of the k-tile for the 4 x 4 tiles of the wave. The next row tile's
  // operand is read from LDS while this one's 8 instructions run, the group's share of the loads
  // two k-tiles ahead goes out with it, and the two parts of one accumulator are 4 instructions
  // apart (back-to-back dependent instructions stall).
  const Fp4Masks fm = fp4_masks();
  auto chunk = [&](const uint8_t* abuf, const BRegs& br, auto cc, auto part, bool mma) {
    constexpr int C = decltype(cc)::value;
    i32x8_t bo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bo[t] = mx_b_operand(br.c[t][2 * C], br.c[t][2 * C + 1], fm);
    AOp cur = a_load(abuf, 0, C), nxt;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < 3) nxt = a_load(abuf, m + 1, C);
      if (m == 0) part(std::integral_constant<int, 4 * C + 0>());
      if (m == 1) part(std::integral_constant<int, 4 * C + 1>());
      if (m == 2) part(std::integral_constant<int, 4 * C + 2>());
      if (m == 3) part(std::integral_constant<int, 4 * C + 3>());
      __builtin_amdgcn_sched_barrier(0);
      if (mma) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mx_mfma<C, C>(cur.h, bo[t], acc[m][t], cur.s, br.s[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mx_mfma<2 + C, C>(cur.l, bo[t], acc[m][t], cur.s, br.s[t]);
      }
      if (m < 3) cur = nxt;
    }
  };
  const KLoads<GuTile> ld{xq, aoff, codes, scales, tb0, nkt, w, lane};
  k_loop<GuTile>(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs& br, auto part, bool mma) {
    chunk(abuf, br, std::integral_constant<int, 0>(), part, mma);
    chunk(abuf, br, std::integral_constant<int, 1>(), part, mma);
  });
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
// gated intermediate split: one thread per 32-value block of act [P][I] (fp16), three parts.
// Output per (sorted row, k-tile): part 0 [256] | part 1 [256] | part 2 [256] | scale words
// [4][8] (part 0 c0, c1, part 1 c0, c1, part 2 c0, c1, 0, 0 for lane group g).
// ------------------------------------------------------------------------------------------------
constexpr int kDnSrc = 50;   // 16-byte chunks per (row, k-tile)

__global__ void __launch_bounds__(256)
quant_act_kernel(const uint16_t* __restrict__ act, uint8_t* __restrict__ aq, int P, int I) {
  const int nb = I / 32, nkt = I / kTileK;
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
  const int kt = blk >> 3, d = blk & 7, g = d & 3, c = d >> 2;
  uint8_t* blkp = aq + ((size_t)r * nkt + kt) * (16 * kDnSrc);
  uint8_t* d0 = blkp + 32 * d;
  *reinterpret_cast<u32x4_t*>(d0) = u32x4_t{p0[0], p0[1], p0[2], p0[3]};
  *reinterpret_cast<u32x4_t*>(d0 + 16) = u32x4_t{p0[4], p0[5], p0[6], p0[7]};
  *reinterpret_cast<u32x4_t*>(d0 + kTileK) = u32x4_t{p1[0], p1[1], p1[2], p1[3]};
  *reinterpret_cast<u32x4_t*>(d0 + kTileK + 16) = u32x4_t{p1[4], p1[5], p1[6], p1[7]};
  *reinterpret_cast<u32x4_t*>(d0 + 2 * kTileK) = u32x4_t{p2[0], p2[1], p2[2], p2[3]};
  *reinterpret_cast<u32x4_t*>(d0 + 2 * kTileK + 16) = u32x4_t{p2[4], p2[5], p2[6], p2[7]};
  uint8_t* sw = blkp + 3 * kTileK + 8 * g;
  sw[c] = (uint8_t)sa;
  sw[2 + c] = (uint8_t)a_part_scale(sa, 1);
  sw[4 + c] = (uint8_t)a_part_scale(sa, 2);
  if (c == 0) *reinterpret_cast<uint16_t*>(sw + 6) = 0;
}

// ------------------------------------------------------------------------------------------------
// down (block-scaled, three parts). LDS row of one k-tile: part 0 [256] | part 1 [256] |
// part 2 [256] | scale words [4][8] (50 chunks, 800 bytes).
// ------------------------------------------------------------------------------------------------
using DnTile = ATile<kDnSrc, kDnSrc>;
constexpr int kDnStride = 16 * kDnSrc;

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
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[DnTile::kPerWave];
  a_sources<DnTile>(aoff, w, lane, [&](int r) {
    return (uint32_t)(rs + min(r, rows_valid - 1)) * (uint32_t)(nkt * DnTile::kSrcBytes);
  });

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A operand of row tile m, instruction C of the k-tile: three parts and their scale words
  struct AOp {
    i32x8_t p[3];
    u32x2_t s;
  };
  auto a_load = [&](const uint8_t* abuf, int m, int C) {
    const uint8_t* ar = abuf + (m * 16 + (lane & 15)) * kDnStride;
    AOp a;
    a.s = *reinterpret_cast<const u32x2_t*>(ar + 3 * kTileK + 8 * g);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(ar + q * kTileK + 128 * C + 16 * g);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(ar + q * kTileK + 128 * C + 64 + 16 * g);
      a.p[q] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return a;
  };
  // as in the gate_up kernel, with 12 instructions per row tile (three parts)
  const Fp4Masks fm = fp4_masks();
  auto chunk = [&](const uint8_t* abuf, const BRegs& br, auto cc, auto part, bool mma) {
    constexpr int C = decltype(cc)::value;
    i32x8_t bo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bo[t] = mx_b_operand(br.c[t][2 * C], br.c[t][2 * C + 1], fm);
    AOp cur = a_load(abuf, 0, C), nxt;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < 3) nxt = a_load(abuf, m + 1, C);
      if (m == 0) part(std::integral_constant<int, 4 * C + 0>());
      if (m == 1) part(std::integral_constant<int, 4 * C + 1>());
      if (m == 2) part(std::integral_constant<int, 4 * C + 2>());
      if (m == 3) part(std::integral_constant<int, 4 * C + 3>());
      __builtin_amdgcn_sched_barrier(0);
      if (mma) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mx_mfma<C, C>(cur.p[0], bo[t], acc[m][t], cur.s[0], br.s[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mx_mfma<2 + C, C>(cur.p[1], bo[t], acc[m][t], cur.s[0], br.s[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = mx_mfma<C, C>(cur.p[2], bo[t], acc[m][t], cur.s[1], br.s[t]);
      }
      if (m < 3) cur = nxt;
    }
  };
  const KLoads<DnTile> ld{aq, aoff, codes, scales, tb0, nkt, w, lane};
  k_loop<DnTile>(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs& br, auto part, bool mma) {
    chunk(abuf, br, std::integral_constant<int, 0>(), part, mma);
    chunk(abuf, br, std::integral_constant<int, 1>(), part, mma);
  });
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
  hipLaunchKernelGGL(gemm_gate_up_mx_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads),
                     kStages * GuTile::kBytes, s,
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
  hipLaunchKernelGGL(gemm_down_mx_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads),
                     kStages * DnTile::kBytes, s,
                     p->dn_codes, p->dn_scales, (const uint8_t*)(wsb + ws.aq),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (float*)(wsb + ws.pair_out), P, p->K, p->I, nblk);
  return hipGetLastError();
}

}  // namespace moew2
