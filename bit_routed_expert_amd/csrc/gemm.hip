// Prefill-shaped grouped expert GEMMs (many tokens per expert), on the gfx950 matrix cores.
//
// Each workgroup computes a BM x BN tile of one expert: BM consecutive sorted pair rows (an
// M-tile from the routing pass) by BN weight rows. The A operand (activations) is staged through
// LDS one 256-wide k-tile at a time; for gate_up the rows are gathered from the split x through
// the sort permutation while they are staged, so gathered activations never round-trip through
// HBM (the pages' AFRAG variant repacks activations fragment-major in a separate pass - README
// bullet "The kernels", "The v0.24.0 port" bullet "AFRAG prefill"; here the LDS staging plays
// that role). The B operand (2-bit weights) is read by each wave straight from the native planes.
//
// Both GEMMs run on the block-scaled instruction with A = fp6 (e2m3) and B = fp4 (e2m1): the
// weights' codes become e2m1 operands with two bit operations per 8 values and their UE8M0 bytes
// are the instruction's B scales; the activations are expanded into three block-scaled e2m3
// parts: x by quant_x6_kernel (one pass before gate_up), the fp16 gated intermediate by the
// gate_up epilogue itself (each gate_up workgroup holds whole 32-value blocks of its rows, so it
// writes the down GEMM's split records directly and the intermediate never goes to HBM).
// fp6 x fp4 runs at twice the rate of fp8 x fp4, so three fp6 parts cost less than two fp8 ones.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int BM = kGemmBM;     // 64 sorted pair rows (4 MFMA row tiles)
constexpr int kRGW = 4;         // weight row groups of 16 per wave: each wave is BM rows x 64 weight rows
constexpr int kWaves = 8;       // two waves per SIMD
constexpr int BN = 16 * kRGW * kWaves;   // 512 weight rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kWgPerCu = 1;

// Tile shape: the 2-bit weights cost 0.28 byte per element against 2.4 bytes for the split
// activations, so the workgroup tile is wide in N (512 weight rows) and short in M (64 rows): per
// k-tile a workgroup moves 39 KB of split activations and 37 KB of weights into the CU. Measured
// alternatives, in alternating runs on one box (gate_up / down GEMM): this tiling 2.54 / 1.48 ms;
// 4 waves of 64 x 128 (half the LDS operand reads per instruction, one wave per SIMD)
// 2.63 / 1.52 ms; each with a third A stage (A two k-tiles ahead) 2.60 / 1.51 and 2.64 / 1.56 ms.
// Earlier: two workgroups of 64 x 256 per CU moved 1.5x the bytes per flop, 32 x 128 wave tiles
// doubled the B loads; neither was faster.
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
// Operand pipeline shared by both GEMMs. The A tile of one k-tile (BM rows) is one LDS stage of
// BM * CH 16-byte chunks, row r at chunk r*CH; the split activations are laid out per (row,
// k-tile) as SRC contiguous chunks, so a stage is filled by direct global -> LDS loads: wave
// instruction j writes chunks 64j .. 64j+63, lane i chunk 64j+i, from the source chunk of that
// (row, chunk) (chunks past SRC repeat the last one; they pad the stride only).
// kAStages A stages rotate (k-tile kt + kAStages - 1 is requested into the stage kt - 1 used
// while kt is computed); the B registers of each wave rotate through three sets (k-tile kt + 2 is
// requested while kt is computed), since B comes from HBM and A mostly from L2. In each step the A
// loads are issued before the B loads, so with two stages "k-tile kt has landed" is "at most the
// kBLoads B loads of kt + 2 are outstanding" (with three, at most the previous step's loads).
// Every wave issues the same loads every step (the tail repeats the last k-tile into a free
// stage), so the counted waits below are exact.
// ------------------------------------------------------------------------------------------------
constexpr int kAStages = 2;

// waits until at most N vector memory operations of this wave are outstanding
template <int N>
MOEW2_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the k-loop, as an asm statement with a memory clobber: the compiler may
// move no memory access across it in either direction (no LDS read of the k-tile it releases, no
// direct-to-LDS load into the stage it frees), and it adds no wait of its own. A workgroup-scope
// fence would order the same accesses but makes the compiler drain every outstanding load
// (vmcnt(0)) at each barrier, since it counts the direct-to-LDS loads as LDS stores; the k-loop's
// explicit vmcnt(N) waits already say which of those loads have landed.
MOEW2_DEV void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// B: the kRGW row groups of a wave, one native k-tile (code loads per row group: 1 for 2-bit
// codes, 2 for fp4 codes; scale words per row group: one with the two UE8M0 bytes, or two of four
// e4m3 bytes for NVFP4 planes)
template <int FMT>
struct BRegs {
  u32x4_t c[kRGW][WFmt<FMT>::kLoads];
  uint32_t s[kRGW][WFmt<FMT>::kScaleWords];
};
template <int FMT>
constexpr int kBLoads = kRGW * (WFmt<FMT>::kLoads + 1);   // vector memory instructions for one BRegs
constexpr int kGroups = 8;   // instruction groups per k-tile: 2 columns C x 4 row tiles m

// The loads of one step for one wave, as kItems single instructions: the stage's DMA instructions
// for k-tile ka (waves whose last instruction index lies past the stage repeat the stage's last
// instruction - the same bytes to the same chunks - so every wave issues kPerWave), then the B
// code and scale loads of k-tile kb. Group i of the computing k-tile issues items
// [i*kItems/8, (i+1)*kItems/8), so the loads spread over the step instead of queueing behind the
// barrier.
template <class AT, int FMT>
struct KLoads {
  static constexpr int kItems = AT::kPerWave + kBLoads<FMT>;
  const uint8_t* abase;
  const uint32_t* aoff;
  const uint8_t* codes;
  const uint8_t* scales;
  size_t tb0;
  int nkt, w, lane;

  template <int N>
  MOEW2_DEV void item(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    if constexpr (N < AT::kPerWave) {
      const int j = min(w + kWaves * N, AT::kInstr - 1);
      __builtin_amdgcn_global_load_lds((const void*)(abase + (aoff[N] + (uint32_t)ka * AT::kSrcBytes)),
                                       (__attribute__((address_space(3))) void*)(stage + 1024 * j), 16, 0, 0);
      if constexpr (N == AT::kPerWave - 1) {
        // The k-loop's wait for this stage counts on every DMA instruction of the step being
        // issued before the step's B loads. Items of one group may otherwise be interleaved by
        // the compiler (it placed B loads ahead of the last DMA instruction), which would leave
        // that DMA uncounted by the wait and let its chunks be read before they land.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      constexpr int L = WFmt<FMT>::kLoads;
      constexpr int n = N - AT::kPerWave, t = n / (L + 1), q = n % (L + 1);
      const size_t ti = tb0 + (size_t)t * nkt + kb;
      if constexpr (q < L) {
        r.c[t][q] = ld16(codes + ti * WFmt<FMT>::kCodeBytes + 1024 * q + 16 * lane);
      } else if constexpr (FMT == kFmtNV4) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(scales + ti * kTileScaleBytesNV4 +
                                                              128 * (lane >> 5) + 8 * (lane & 15));
        r.s[t][0] = v[0];
        r.s[t][1] = v[1];
      } else {
        r.s[t][0] = *reinterpret_cast<const uint16_t*>(scales + ti * kTileScaleBytes + 2 * lane);
      }
    }
  }
  template <int N0, int N1>
  MOEW2_DEV void items(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    if constexpr (N0 < N1) {
      item<N0>(ka, stage, kb, r);
      items<N0 + 1, N1>(ka, stage, kb, r);
    }
  }
  template <int I>
  MOEW2_DEV void group(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    items<I * kItems / kGroups, (I + 1) * kItems / kGroups>(ka, stage, kb, r);
  }
};

// The k-loop: COMPUTE(stage, BRegs, part, mma) for every step, where part(integral_constant<I>)
// issues load group I (COMPUTE calls it for I = 0..7 in order, always) and mma says whether the
// step has a k-tile to multiply (not the first two steps, the tail of the last round or idle
// waves). K-tile j uses A stage j % 3 and B register set j % 3.
template <class AT, int FMT, class Compute>
MOEW2_DEV void k_loop(uint8_t* lds, const KLoads<AT, FMT>& ld, int nkt, bool active, Compute compute) {
  static_assert(kAStages == 2 || kAStages == 3, "A runs kAStages - 1 k-tiles ahead");
  BRegs<FMT> b0, b1, b2;
  // POS = kt mod 3 (kt = -2 starts the first round, so the round positions are 1, 2, 0)
  auto step = [&](int kt, auto pos, BRegs<FMT>& cur, BRegs<FMT>& ahead) {
    constexpr int POS = decltype(pos)::value;
    // k-tile kt has landed: its B was issued two steps ago, its A kAStages - 1 steps ago, each
    // before the B loads of its step; what may still be outstanding is what came after
    wait_vm<kAStages == 3 ? AT::kPerWave + kBLoads<FMT> : kBLoads<FMT>>();
    lds_barrier();                     // ... in every wave; and every wave is done with kt - 1
    const int ka = max(0, min(kt + kAStages - 1, nkt - 1));
    const int kb = max(0, min(kt + 2, nkt - 1));
    // A: the stage kt - 1 used; computing from the stage of kt
    const int a_next = kAStages == 3 ? (POS + 2) % 3 : ((kt + 1) & 1);
    const int a_cur = kAStages == 3 ? POS : (kt & 1);
    uint8_t* a_stage = lds + a_next * AT::kBytes;
    auto part = [&](auto ic) { ld.template group<decltype(ic)::value>(ka, a_stage, kb, ahead); };
    // Every step runs the same instruction stream except the matrix instructions themselves: the
    // loads and LDS reads are unconditional (a step without a k-tile reads a stale stage), so the
    // compiler's count of outstanding loads stays exact and no operand needs a merge copy.
    const bool mma = active && kt >= 0 && kt < nkt;
    compute(lds + a_cur * AT::kBytes, cur, part, mma);
  };
  // Whole rounds of three steps (B register sets, and three A stages, rotate by three): the first
  // round's first two steps only issue, steps past the last k-tile only load repeats of it.
  for (int kt = -2; kt < nkt; kt += 3) {
    step(kt, std::integral_constant<int, 1>(), b1, b0);
    step(kt + 1, std::integral_constant<int, 2>(), b2, b1);
    step(kt + 2, std::integral_constant<int, 0>(), b0, b2);
  }
  wait_vm<0>();                        // no DMA may still target this workgroup's LDS
}

// ------------------------------------------------------------------------------------------------
// x split: one thread per 32-value block of x (bf16 [T][K]), three e2m3 parts into the 608-byte
// record of its (token, k-tile) (layout at kA6Bytes in common.h). The gated intermediate's
// records are written by the gate_up epilogue with the same arithmetic.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
quant_x6_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst, int rows, int n) {
  const int nb = n / 32, nkt = n / kTileK;
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (long long)rows * nb) return;
  const int r = (int)(b / nb), blk = (int)(b - (long long)r * nb);
  const uint16_t* sp = src + (size_t)r * n + 32 * blk;
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t w = ld16(sp + 8 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_lo(w[j]);
      v[8 * q + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < 32; ++q) a = __builtin_fmaxf(a, __builtin_fabsf(v[q]));
  const uint32_t sb = a6_scale_byte(a);
  u32x6_t part[3];
  a6_split(v, sb, part);
  a6_store(dst + ((size_t)r * nkt + (blk >> 3)) * kA6Bytes, blk & 7, part, sb);
}

// A operand of one instruction (C = 0, 1 of the k-tile) from a staged split record: the three
// parts of block 4C + g and their scale word (part p's byte is picked by op_sel p).
struct A6Op {
  i32x8_t p[3];
  uint32_t s;
};
MOEW2_DEV A6Op a6_load(const uint8_t* ar, int C, int g) {
  A6Op a;
  const int d = 4 * C + g;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(ar + 16 * (8 * q + d));
    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(ar + kA6Hi + 8 * (8 * q + d));
    a.p[q] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], 0, 0};
  }
  a.s = *reinterpret_cast<const uint32_t*>(ar + kA6Scale + 4 * d);
  return a;
}

// LDS rows hold one split record plus one pad chunk: a row stride of 39 chunks (156 dwords,
// 4 mod 8) is the one at which the operand reads of 16, 8 and 4 bytes per lane (16 rows x 4
// consecutive pieces) all run at their minimum LDS cycles (measured with the LDS bank-conflict
// counter; strides of 8 mod 16 dwords double the cycles of the 8- and 4-byte reads).
constexpr int kA6Chunks = kA6Bytes / 16;   // 38 16-byte chunks per (row, k-tile)
constexpr int kA6Stride = 16 * (kA6Chunks + 1);
using A6Tile = ATile<kA6Chunks + 1, kA6Chunks>;
static_assert(kA6Bytes % 16 == 0, "split record is whole chunks");

// The k-loop body shared by both GEMMs: for each instruction column C of the k-tile, the B
// operands of the wave's kRGW row groups, then per row tile m the three parts x kRGW row groups
// of instructions. The next row tile's operand is read from LDS while this one's 3 * kRGW
// instructions run, the group's share of the loads two k-tiles ahead goes out with it, and the
// three parts of one accumulator are kRGW instructions apart (back-to-back dependent instructions
// stall).
template <int FMT, class Part>
MOEW2_DEV void a6_ktile(f32x4_t (&acc)[4][kRGW], const uint8_t* abuf, const BRegs<FMT>& br, Part part, bool mma,
                        int rows_valid, int lane, const Fp4Masks& fm, int sshift = 0) {
  const int g = lane >> 4;
  // scale words: the row group's two UE8M0 bytes in the low half (sshift bits down)
  uint32_t bs[kRGW];
#pragma unroll
  for (int t = 0; t < kRGW; ++t) bs[t] = br.s[t][0] >> sshift;
  const uint8_t* arow = abuf + (lane & 15) * kA6Stride;
  static_for<0, 2>([&](auto cc) {
    constexpr int C = decltype(cc)::value;
    i32x8_t bo[kRGW];
#pragma unroll
    for (int t = 0; t < kRGW; ++t) bo[t] = b_operand<FMT, C>(br.c[t], fm);
    A6Op cur = a6_load(arow, C, g), nxt;
    static_for<0, 4>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 3) nxt = a6_load(arow + (m + 1) * 16 * kA6Stride, C, g);
      part(std::integral_constant<int, 4 * C + m>());
      __builtin_amdgcn_sched_barrier(0);
      // a row tile with no valid row (the ragged end of an expert's group) skips its instructions
      if (mma && 16 * m < rows_valid) {
#pragma unroll
        for (int t = 0; t < kRGW; ++t) acc[m][t] = mx6_mfma<0, C>(cur.p[0], bo[t], acc[m][t], cur.s, bs[t]);
#pragma unroll
        for (int t = 0; t < kRGW; ++t) acc[m][t] = mx6_mfma<1, C>(cur.p[1], bo[t], acc[m][t], cur.s, bs[t]);
#pragma unroll
        for (int t = 0; t < kRGW; ++t) acc[m][t] = mx6_mfma<2, C>(cur.p[2], bo[t], acc[m][t], cur.s, bs[t]);
      }
      if constexpr (m < 3) cur = nxt;
    });
  });
}

// ------------------------------------------------------------------------------------------------
// gate_up: rows of the split x gathered through the sort permutation (token = pair / top_k).
// Wave w of N-block nb holds row groups kRGW * (kWaves nb + w) .. + kRGW - 1 (gate, up, gate, up,
// ...), i.e. gated columns 8 kRGW (kWaves nb + w) .. + 8 kRGW - 1 of its BM rows: blocks
// kBPW w .. kBPW w + kBPW - 1 (kBPW = kRGW / 4 blocks of 32) of the down GEMM's k-tile nb (2I is a
// multiple of BN, so every wave has its blocks). The epilogue rounds a = silu(g) * u to fp16,
// passes each BM x 32 block through the wave's own LDS region (row stride 36 floats, 4 mod 8
// dwords, for the row-per-lane reads), lane r splits row r of each block into its three e2m3
// parts (the arithmetic of quant_x6_kernel, on the fp16-rounded values) and puts them in row r's
// split record, assembled in LDS; the workgroup then writes the BM whole records (sorted row,
// k-tile nb) with 16-byte stores of consecutive chunks.
// ------------------------------------------------------------------------------------------------
constexpr int kBPW = kRGW / 4;                          // 32-value blocks of gated columns per wave
constexpr int kTpStride = 36;                           // floats per row of the epilogue's block
constexpr int kTpBlock = BM * kTpStride;                // floats of one block in the wave's region
constexpr int kTpBytes = kBPW * kTpBlock * 4;           // one wave's region
constexpr int kRecOff = kWaves * kTpBytes;              // the assembled records
constexpr int kGateUpLds = kRecOff + BM * kA6Bytes > kAStages * A6Tile::kBytes ? kRecOff + BM * kA6Bytes
                                                                                 : kAStages * A6Tile::kBytes;
static_assert(kRGW % 4 == 0, "a wave holds whole 32-value blocks of gated columns");
static_assert(kWaves * kBPW * 32 == kTileK, "a gate_up workgroup covers one down k-tile of gated columns");
template <int FMT>
__global__ void __launch_bounds__(kThreads, kWgPerCu)
gemm_gate_up_mx_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       const uint8_t* __restrict__ xq, const int32_t* __restrict__ offsets,
                       const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                       const int32_t* __restrict__ meta, uint8_t* __restrict__ aq,
                       long long* __restrict__ counters, int T, int K, int I, int top_k, int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // row groups kRGW*(nb*kWaves + w) .. + kRGW - 1 of this wave (gate, up, gate, up, ...); a matrix
  // with fewer than BN rows leaves waves idle (they still load a valid row group to keep the waits
  // exact)
  const int rg0 = kRGW * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[A6Tile::kPerWave];
  a_sources<A6Tile>(aoff, w, lane, [&](int r) {
    const int tok = perm[rs + min(r, rows_valid - 1)] / top_k;
    return (uint32_t)tok * (uint32_t)(nkt * A6Tile::kSrcBytes);
  });

  f32x4_t acc[4][kRGW];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const Fp4Masks fm = fp4_masks();
  const KLoads<A6Tile, FMT> ld{xq, aoff, codes, scales, tb0, nkt, w, lane};
  k_loop(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs<FMT>& br, auto part, bool mma) {
    a6_ktile(acc, abuf, br, part, mma, rows_valid, lane, fm);
  });
  __syncthreads();   // every wave is done with the A stages, which the epilogue reuses

  // ---- epilogue: a = silu(g) * u in fp16, blocks kBPW w .. of each sorted row's split record ----
  if (wave_active) {
    float* tp = reinterpret_cast<float*>(lds + w * kTpBytes);
    unsigned n_inf = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m * 16 + 4 * (lane >> 4) + r;
        // gate/up row-group pair pr: gated columns 16 pr .. 16 pr + 15 of the wave, i.e. block
        // pr / 2, columns 16 (pr % 2) .. of it
#pragma unroll
        for (int pr = 0; pr < kRGW / 2; ++pr) {
          const float a = silu_mul(acc[m][2 * pr][r], acc[m][2 * pr + 1][r]);
          const float h = (float)(_Float16)a;
          n_inf += row < rows_valid && __builtin_isinf(h) ? 1u : 0u;
          tp[(pr / 2) * kTpBlock + row * kTpStride + 16 * (pr % 2) + (lane & 15)] = h;
        }
      }
    }
    // one counter update per lane that saw an overflow (none on finite workloads)
    if (n_inf) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)n_inf);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the region is this wave's alone
    if (lane < rows_valid) {
#pragma unroll
      for (int b = 0; b < kBPW; ++b) {
        float v[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f32x4_t f = *reinterpret_cast<const f32x4_t*>(tp + b * kTpBlock + lane * kTpStride + 4 * q);
          v[4 * q] = f[0], v[4 * q + 1] = f[1], v[4 * q + 2] = f[2], v[4 * q + 3] = f[3];
        }
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 32; ++q) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[q]));
        const uint32_t sb = a6_scale_byte(amax);
        u32x6_t part[3];
        a6_split(v, sb, part);
        a6_store(lds + kRecOff + lane * kA6Bytes, kBPW * w + b, part, sb);
      }
    }
  }
  __syncthreads();   // every block of every record is in LDS
  const size_t rec_stride = (size_t)(I / kTileK) * kA6Bytes;
  uint8_t* rec0 = aq + ((size_t)rs * (I / kTileK) + tm.nb) * kA6Bytes;
  for (int c = tid; c < rows_valid * kA6Chunks; c += kThreads) {
    const int row = c / kA6Chunks, j = c - row * kA6Chunks;
    *reinterpret_cast<u32x4_t*>(rec0 + row * rec_stride + 16 * j) =
        *reinterpret_cast<const u32x4_t*>(lds + kRecOff + row * kA6Bytes + 16 * j);
  }
}

// ------------------------------------------------------------------------------------------------
// down: rows of the split gated intermediate in sorted order; per-pair fp32 rows out.
// ------------------------------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kThreads, kWgPerCu)
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
  const int rg0 = kRGW * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[A6Tile::kPerWave];
  a_sources<A6Tile>(aoff, w, lane, [&](int r) {
    return (uint32_t)(rs + min(r, rows_valid - 1)) * (uint32_t)(nkt * A6Tile::kSrcBytes);
  });

  f32x4_t acc[4][kRGW];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the tile's pair indices, fetched now so that the epilogue's stores do not wait on them
  __shared__ int tile_pairs[BM];
  if (tid < BM) tile_pairs[tid] = perm[rs + min(tid, rows_valid - 1)];

  const Fp4Masks fm = fp4_masks();
  const KLoads<A6Tile, FMT> ld{aq, aoff, codes, scales, tb0, nkt, w, lane};
  k_loop(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs<FMT>& br, auto part, bool mma) {
    a6_ktile(acc, abuf, br, part, mma, rows_valid, lane, fm);
  });
  __syncthreads();   // tile_pairs visible to every wave
  if (!wave_active) return;

  // ---- epilogue: per-pair rows at the pair index ----
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int p = tile_pairs[row];
#pragma unroll
      for (int t = 0; t < kRGW; ++t) pair_out[(size_t)p * K + 16 * (rg0 + t) + (lane & 15)] = acc[m][t][r];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// down, streamed across tiles: one workgroup per CU walks its XCD's share of the tile list (the
// logical order of map_tile: workgroup j of an XCD takes logical tiles lo + j, lo + j + G, ...
// with G workgroups per XCD, so the tiles in flight on an XCD are still a run of consecutive
// logical tiles). The k-tiles of consecutive tiles form one stream of steps; a tile is NKT
// compute steps and one epilogue step, NKT + 1 a multiple of 3, so the three B register sets
// and three A stages keep static roles (position p of a tile reads B set p % 3 and A stage
// p % 3). Step p requests A k-tile p + 1 and B k-tile p + 2; past the tile's end those are the
// next tile's first k-tiles (its A k-tile 0 goes to stage 0 from the last compute step on, B
// k-tiles 0 and 1 to sets 0 and 1), and the B loads aimed at the epilogue position (which
// multiplies nothing) only keep the count (out-of-range offsets, no memory access). So a tile
// starts on loads already in flight and no step only fills or drains.
//
// The epilogue step stores the finished tile's rows first and then issues its loads, so "at
// most kBLoads outstanding" at the next step still means the step's A stage and B k-tile have
// landed. Its rows go out through the epilogue position's A stage (free in that step): each
// wave passes 16 rows of its 64 columns at a time through its own part of the stage and stores
// them as 16-byte pieces, 4 rows x 256 contiguous bytes per instruction.
// ------------------------------------------------------------------------------------------------
constexpr int kDnTpStride = 16 * kRGW + 4;           // floats per row (4 mod 8 dwords)
constexpr int kDnTpRows = 16;                        // rows per pass
constexpr int kDnTpFloats = kDnTpRows * kDnTpStride; // one wave's part of the stage
constexpr int kDnPairsOff = 3 * A6Tile::kBytes;
constexpr int kDnStreamLds = kDnPairsOff + kWaves * 2 * BM * 4;
static_assert(kWaves * kDnTpFloats * 4 <= A6Tile::kBytes, "epilogue passes fit in one A stage");

// The step loads of the streamed kernel: the same items and groups as KLoads, with the B code and
// scale loads as raw buffer loads (tile offset in a scalar register, one lane offset for all), so
// that no per-lane 64-bit B address has to stay live across the stream.
// Volatile (the compiler-implemented bit of the buffer intrinsics' policy operand): the compiler
// keeps each load in its step instead of moving it to another one. Loads with equal operands can
// still be merged into one, so the count-keeping loads use distinct offsets (one per row group)
// and their registers are named at the epilogue position; every step then issues the loads its
// counted waits assume (checked in the assembly by the tests).
constexpr int kVolatileLoad = (int)0x80000000u;
constexpr uint32_t kOobLoad = 0x7FFFF000u;   // past any plane view (views up to kMaxPlaneView bytes)
constexpr long long kMaxPlaneView = 0x7FFF0000ll;
template <int FMT>
struct SLoads {
  static constexpr int kItems = A6Tile::kPerWave + kBLoads<FMT>;
  const uint8_t* abase;
  const uint32_t* aoff;
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t tb0;
  int nkt, w, lane;

  template <int N>
  MOEW2_DEV void item(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    if constexpr (N < A6Tile::kPerWave) {
      const int j = min(w + kWaves * N, A6Tile::kInstr - 1);
      __builtin_amdgcn_global_load_lds((const void*)(abase + (aoff[N] + (uint32_t)ka * A6Tile::kSrcBytes)),
                                       (__attribute__((address_space(3))) void*)(stage + 1024 * j), 16, 0, 0);
      if constexpr (N == A6Tile::kPerWave - 1) {
        // every DMA instruction of the step goes out before its B loads (see KLoads)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      constexpr int L = WFmt<FMT>::kLoads;
      constexpr int n = N - A6Tile::kPerWave, t = n / (L + 1), q = n % (L + 1);
      // kb < 0: a load that only keeps the count, at an out-of-range offset (no memory access)
      const uint32_t ti = kb < 0 ? (uint32_t)t : tb0 + (uint32_t)(t * nkt + kb);
      const uint32_t oob = kb < 0 ? kOobLoad : 0u;
      if constexpr (q < L) {
        r.c[t][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
            codes, (int)(oob + 1024 * q + 16 * lane), (int)(ti * (uint32_t)WFmt<FMT>::kCodeBytes), kVolatileLoad));
      } else {
        // the aligned dword holding this lane's two scale bytes (the upper half for odd lanes,
        // shifted down where the operand is formed): a 32-bit load needs no zero-extension
        r.s[t][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(scales, (int)(oob + 4 * (lane >> 1)),
                                                                    (int)(ti * (uint32_t)kTileScaleBytes), kVolatileLoad);
      }
    }
  }
  template <int N0, int N1>
  MOEW2_DEV void items(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    if constexpr (N0 < N1) {
      item<N0>(ka, stage, kb, r);
      items<N0 + 1, N1>(ka, stage, kb, r);
    }
  }
  template <int I>
  MOEW2_DEV void group(int ka, uint8_t* stage, int kb, BRegs<FMT>& r) const {
    items<I * kItems / kGroups, (I + 1) * kItems / kGroups>(ka, stage, kb, r);
  }
};

struct DnTile {
  int e, rs, rows_valid, nb;
};
MOEW2_DEV DnTile dn_tile(int logical, const int32_t* tiles, const int32_t* offsets, int n_blocks) {
  DnTile t;
  const int ti = logical / n_blocks;
  t.nb = logical - ti * n_blocks;
  t.e = tiles[2 * ti];
  t.rs = tiles[2 * ti + 1];
  t.rows_valid = min(BM, offsets[t.e + 1] - t.rs);
  return t;
}

template <int FMT, int NKT>
__global__ void __launch_bounds__(kThreads, 1)
gemm_down_mx_stream_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                           const uint8_t* __restrict__ aq, const int32_t* __restrict__ offsets,
                           const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                           const int32_t* __restrict__ meta, float* __restrict__ pair_out, int P, int K,
                           int n_blocks, uint32_t n_tiles_b) {
  static_assert((NKT + 1) % 3 == 0, "a tile is whole rounds of three steps");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int total = meta[1] * n_blocks;
  const int per_xcd = (total + 7) / 8;
  const int G = (int)(gridDim.x >> 3);
  const int lo = (int)(blockIdx.x & 7) * per_xcd, hi = min(lo + per_xcd, total);
  int lg = lo + (int)(blockIdx.x >> 3);
  if (lg >= hi) return;
  const int nrg = K / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t out = buffer_view(pair_out, (uint32_t)P * (uint32_t)K * 4u);
  constexpr int LB = kBLoads<FMT>;

  // the current tile and the next one of this workgroup's walk (the current one again past the
  // end, so that the loads issued for it stay valid and counted)
  DnTile cur = dn_tile(lg, tiles, offsets, n_blocks);
  DnTile nxt = lg + G < hi ? dn_tile(lg + G, tiles, offsets, n_blocks) : cur;
  auto tb0_of = [&](const DnTile& t) {
    return (uint32_t)t.e * (uint32_t)(nrg * NKT) + (uint32_t)(kRGW * (t.nb * kWaves + w) * NKT);
  };
  const __amdgpu_buffer_rsrc_t crs = buffer_view(codes, (uint32_t)(n_tiles_b * WFmt<FMT>::kCodeBytes));
  const __amdgpu_buffer_rsrc_t srs = buffer_view(scales, (uint32_t)(n_tiles_b * kTileScaleBytes));
  // per DMA instruction of this lane, 16 bits: its tile row (bits 10..15) and byte offset within
  // the row's record (bits 0..9), two to a register; a tile's source offsets are formed from these
  constexpr int kDesc = (A6Tile::kPerWave + 1) / 2;
  uint32_t adesc[kDesc];
  {
    uint32_t d[A6Tile::kPerWave];
    a_sources<A6Tile>(d, w, lane, [&](int r) { return (uint32_t)r << 10; });
#pragma unroll
    for (int i = 0; i < kDesc; ++i) adesc[i] = d[2 * i] | (2 * i + 1 < A6Tile::kPerWave ? d[2 * i + 1] << 16 : 0u);
  }
  static_assert(A6Tile::kSrcBytes <= 1024 && BM <= 64, "descriptor fields");
  constexpr uint32_t kRecStride = (uint32_t)(NKT * A6Tile::kSrcBytes);
  auto loads_for = [&](const DnTile& ta, const DnTile& tb, uint32_t (&ao)[A6Tile::kPerWave]) {
#pragma unroll
    for (int i = 0; i < A6Tile::kPerWave; ++i) {
      const uint32_t d = (adesc[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      ao[i] = (uint32_t)(ta.rs + min((int)(d >> 10), ta.rows_valid - 1)) * kRecStride + (d & 1023u);
    }
    return SLoads<FMT>{aq, ao, crs, srs, tb0_of(tb), NKT, w, lane};
  };
  // the pair index of each tile row, per wave in LDS past the stages: two tiles' worth (this
  // tile's for its epilogue, the next one's written during this tile)
  int* wpairs = reinterpret_cast<int*>(lds + kDnPairsOff) + w * 2 * BM;
  auto pair_of = [&](const DnTile& t) { return perm[t.rs + min(lane, t.rows_valid - 1)]; };
  int par = 0;   // buffer of the current tile's pairs
  int pr_nxt = 0;

  f32x4_t acc[4][kRGW];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const Fp4Masks fm = fp4_masks();
  const int sshift = 16 * (lane & 1);
  BRegs<FMT> b[3];

  // prologue: the first tile's pairs, A k-tile 0 into stage 0, B k-tiles 0 and 1 into sets 0 and 1
  {
    const int pr = pair_of(cur);
    uint32_t ao[A6Tile::kPerWave];
    const SLoads<FMT> ld = loads_for(cur, cur, ao);
    static_for<0, kGroups>([&](auto ic) { ld.template group<decltype(ic)::value>(0, lds, 0, b[0]); });
    static_for<A6Tile::kPerWave, SLoads<FMT>::kItems>(
        [&](auto ic) { ld.template item<decltype(ic)::value>(0, lds, 1, b[1]); });
    wpairs[lane] = pr;   // waits for the pair load only (the oldest)
  }

  for (;;) {
    static_for<0, NKT + 1>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      // the step's k-tile (or, at the epilogue position, the previous steps' loads) has landed
      wait_vm<LB>();
      lds_barrier();
      if constexpr (p == 0) pr_nxt = pair_of(nxt);   // landed by the next step's wait
      if constexpr (p == 1) wpairs[(par ^ 1) * BM + lane] = pr_nxt;
      // this step's loads: A k-tile p + 1 (the next tile's k-tile 0 into stage 0 from the last
      // compute step on), B k-tile p + 2 (the epilogue position's set gets out-of-range loads
      // that only keep the count; then the next tile's k-tiles 0 and 1)
      constexpr bool a_nxt = p + 1 >= NKT;
      constexpr int a_stage = a_nxt ? 0 : (p + 1) % 3;
      constexpr int ka = a_nxt ? 0 : p + 1;
      constexpr int pb = p + 2;
      constexpr bool b_nxt = pb > NKT;
      constexpr int kb = pb < NKT ? pb : (pb == NKT ? -1 : pb - NKT - 1);
      constexpr int b_set = pb % 3;
      uint32_t ao[A6Tile::kPerWave];
      const SLoads<FMT> ld = loads_for(a_nxt ? nxt : cur, b_nxt ? nxt : cur, ao);
      uint8_t* stage = lds + a_stage * A6Tile::kBytes;
      if constexpr (p < NKT) {
        auto part = [&](auto ic) { ld.template group<decltype(ic)::value>(ka, stage, kb, b[b_set]); };
        a6_ktile(acc, lds + (p % 3) * A6Tile::kBytes, b[p % 3], part, true, cur.rows_valid, lane, fm, sshift);
      } else {
        // The B set of this position holds a repeat nobody multiplies; naming its registers here
        // (landed by this step's wait, so no wait is added) keeps those loads in the instruction
        // stream, where the counted waits expect them.
#pragma unroll
        for (int t = 0; t < kRGW; ++t)
#pragma unroll
          for (int q = 0; q < WFmt<FMT>::kLoads; ++q)
            asm volatile("" ::"v"(b[p % 3].c[t][q]), "v"(b[p % 3].s[t][0]));
        // epilogue: the finished tile's rows, 16 at a time through this wave's part of the
        // epilogue position's stage, then the step's loads
        float* tp = reinterpret_cast<float*>(lds + (p % 3) * A6Tile::kBytes) + w * kDnTpFloats;
        const uint32_t col = (uint32_t)(16 * kRGW * (cur.nb * kWaves + w) + 4 * (lane & 15));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < kRGW; ++t)
              tp[(4 * (lane >> 4) + r) * kDnTpStride + 16 * t + (lane & 15)] = acc[m][t][r];
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's part alone
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int rl = 4 * j + (lane >> 4), row = 16 * m + rl;
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(tp + rl * kDnTpStride + 4 * (lane & 15));
            const int pp = wpairs[par * BM + row];
            // a row past the valid rows goes to an out-of-range offset: dropped, still counted
            const uint32_t off = row < cur.rows_valid ? ((uint32_t)pp * (uint32_t)K) * 4u + 4u * col : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b128(v, out, (int)off, 0, 0);
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // reads done before the next pass
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);   // the stores go out before the step's loads
        static_for<0, kGroups>([&](auto ic) { ld.template group<decltype(ic)::value>(ka, stage, kb, b[b_set]); });
      }
    });
    lg += G;
    if (lg >= hi) break;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    cur = nxt;
    par ^= 1;
    nxt = lg + G < hi ? dn_tile(lg + G, tiles, offsets, n_blocks) : cur;
  }
  wait_vm<0>();   // no DMA may still target this workgroup's LDS
}

// ------------------------------------------------------------------------------------------------
// NVFP4 planes (e2m1 codes, one E4M3 scale per 16 values, fp32 scale_2 per tensor; layout in
// common.h). Their block-16 scales carry mantissa bits, which the block-scaled instruction's
// UE8M0 scales cannot, so these GEMMs run on the 16 x 16 x 32 bf16 (gate_up: A = x as it is) and
// fp16 (down: A = the fp16 gated intermediate) instructions, each B operand of 8 weights formed
// exactly in registers from its codes and scale byte (nv4_b_bf16 / nv4_b_f16); scale_2 multiplies
// the fp32 results. A needs no split pass: a stage holds BM rows of 256 16-bit values, filled by
// direct global -> LDS loads straight from x (gathered through the sort permutation) or from the
// gate_up epilogue's fp16 rows in sorted order. The k-loop, tile map, B register rotation and
// counted waits are the ones above.
// ------------------------------------------------------------------------------------------------
constexpr int kN4Src = kTileK * 2 / 16;        // 32 chunks: one (row, k-tile) of 16-bit values
constexpr int kN4Stride = 16 * (kN4Src + 1);   // LDS row stride 528 bytes (132 dwords, 4 mod 16)
using N4Tile = ATile<kN4Src + 1, kN4Src>;

// One k-tile: instruction J = 4C + j reduces values 32J .. 32J + 31; lane l's A operand is the
// 16 bytes of values 32J + 8(l/16) .. + 7 of row l % 16 of each row tile, its B operand dword j of
// half C of its code loads with scale byte j of scale word C. Per J: the wave's kRGW B operands,
// then 4 row tiles x kRGW instructions (same accumulator 16 instructions apart); the step's load
// group J goes out with it.
template <int NP, class Part>
MOEW2_DEV void nv4_ktile(f32x4_t (&acc)[4][kRGW], const uint8_t* abuf, const BRegs<kFmtNV4>& br, Part part,
                         bool mma, int rows_valid, int lane) {
  const uint8_t* arow = abuf + (lane & 15) * kN4Stride + 16 * (lane >> 4);
  static_for<0, 8>([&](auto jc) {
    constexpr int J = decltype(jc)::value, C = J / 4, j = J % 4;
    typedef std::conditional_t<NP == 0, bf16x8_t, f16x8_t> BOp;
    BOp bo[kRGW];
#pragma unroll
    for (int t = 0; t < kRGW; ++t) {
      if constexpr (NP == 0) bo[t] = nv4_b_bf16<j>(br.c[t][C][j], br.s[t][C]);
      else bo[t] = nv4_b_f16<j>(br.c[t][C][j], br.s[t][C]);
    }
    u32x4_t cur = *reinterpret_cast<const u32x4_t*>(arow + 64 * J), nxt;
    part(std::integral_constant<int, J>());
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 4>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 3) nxt = *reinterpret_cast<const u32x4_t*>(arow + (m + 1) * 16 * kN4Stride + 64 * J);
      if (mma && 16 * m < rows_valid) {
#pragma unroll
        for (int t = 0; t < kRGW; ++t) {
          if constexpr (NP == 0) acc[m][t] = mfma32_bf16(cur, bo[t], acc[m][t]);
          else acc[m][t] = mfma32_f16(cur, bo[t], acc[m][t]);
        }
      }
      if constexpr (m < 3) cur = nxt;
    });
  });
}

// gate_up on NVFP4 planes: A = x rows gathered through the sort permutation; the epilogue writes
// a = silu(sg g) (su u) in fp16 to the sorted rows of the intermediate ([sorted row][I]), which
// the down GEMM reads as its A records.
__global__ void __launch_bounds__(kThreads, kWgPerCu)
gemm_gate_up_nv4_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                        const float* __restrict__ scale2, const uint16_t* __restrict__ x,
                        const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                        const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta,
                        _Float16* __restrict__ act, long long* __restrict__ counters, int K, int I, int top_k,
                        int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg0 = kRGW * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[N4Tile::kPerWave];
  a_sources<N4Tile>(aoff, w, lane, [&](int r) {
    const int tok = perm[rs + min(r, rows_valid - 1)] / top_k;
    return (uint32_t)tok * (uint32_t)(nkt * N4Tile::kSrcBytes);
  });

  f32x4_t acc[4][kRGW];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const KLoads<N4Tile, kFmtNV4> ld{reinterpret_cast<const uint8_t*>(x), aoff, codes, scales, tb0, nkt, w, lane};
  k_loop(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs<kFmtNV4>& br, auto part, bool mma) {
    nv4_ktile<0>(acc, abuf, br, part, mma, rows_valid, lane);
  });
  if (!wave_active) return;

  // ---- epilogue: gated columns 16 (rg0 / 2 + pr) + lane % 16 of rows 16 m + 4 (lane / 16) + r ----
  const float sg = scale2[3 * e], su = scale2[3 * e + 1];
  unsigned n_inf = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
#pragma unroll
      for (int pr = 0; pr < kRGW / 2; ++pr) {
        const _Float16 h = (_Float16)silu_mul(acc[m][2 * pr][r] * sg, acc[m][2 * pr + 1][r] * su);
        n_inf += __builtin_isinf((float)h) ? 1u : 0u;
        act[(size_t)(rs + row) * I + 16 * (rg0 / 2 + pr) + (lane & 15)] = h;
      }
    }
  }
  if (n_inf) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)n_inf);
}

// down on NVFP4 planes: A = the fp16 gated rows in sorted order; per-pair fp32 rows out, times the
// down tensor's scale_2.
__global__ void __launch_bounds__(kThreads, kWgPerCu)
gemm_down_nv4_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     const float* __restrict__ scale2, const _Float16* __restrict__ act,
                     const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                     const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta,
                     float* __restrict__ pair_out, int K, int I, int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const TileMap tm = map_tile(tiles, meta, offsets, n_blocks);
  if (!tm.live) return;
  const int e = tm.e, rs = tm.rs, rows_valid = tm.rows_valid;
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg0 = kRGW * (tm.nb * kWaves + w);
  const bool wave_active = rg0 < nrg;
  const size_t tb0 = (size_t)e * nrg * nkt + (size_t)(wave_active ? rg0 : 0) * nkt;

  uint32_t aoff[N4Tile::kPerWave];
  a_sources<N4Tile>(aoff, w, lane, [&](int r) {
    return (uint32_t)(rs + min(r, rows_valid - 1)) * (uint32_t)(nkt * N4Tile::kSrcBytes);
  });

  f32x4_t acc[4][kRGW];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < kRGW; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __shared__ int tile_pairs[BM];
  if (tid < BM) tile_pairs[tid] = perm[rs + min(tid, rows_valid - 1)];

  const KLoads<N4Tile, kFmtNV4> ld{reinterpret_cast<const uint8_t*>(act), aoff, codes, scales, tb0, nkt, w, lane};
  k_loop(lds, ld, nkt, wave_active, [&](const uint8_t* abuf, const BRegs<kFmtNV4>& br, auto part, bool mma) {
    nv4_ktile<1>(acc, abuf, br, part, mma, rows_valid, lane);
  });
  __syncthreads();   // tile_pairs visible to every wave
  if (!wave_active) return;
  const float sd = scale2[3 * e + 2];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int p = tile_pairs[row];
#pragma unroll
      for (int t = 0; t < kRGW; ++t) pair_out[(size_t)p * K + 16 * (rg0 + t) + (lane & 15)] = acc[m][t][r] * sd;
    }
  }
}

}  // namespace

// One workgroup per compute unit (a whole number per XCD) for the streamed kernels; the count is
// read once per device.
inline unsigned stream_grid() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
    cus[dev] = n;
  }
  return (unsigned)(cus[dev] / 8 * 8);
}

inline unsigned gemm_grid(int max_tiles, int n_blocks) {
  const long long g = (long long)max_tiles * n_blocks;
  return (unsigned)((g + 7) / 8 * 8);
}

hipError_t launch_gemm_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                               const Workspace& ws, uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  if (p->fmt == kFmtNV4) {
    const int nblk = (2 * p->I + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_gate_up_nv4_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads),
                       kAStages * N4Tile::kBytes, s, p->gu_codes, p->gu_scales, p->scale2, (const uint16_t*)x,
                       (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                       (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta), (_Float16*)(wsb + ws.aq),
                       (long long*)(wsb + ws.counters), p->K, p->I, top_k, nblk);
    return hipGetLastError();
  }
  const long long nblk32 = (long long)T * (p->K / 32);
  hipLaunchKernelGGL(quant_x6_kernel, dim3((unsigned)((nblk32 + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)x, wsb + ws.xq, T, p->K);
  const int nblk = (2 * p->I + BN - 1) / BN;
  auto kern = p->fmt == kFmtW4 ? gemm_gate_up_mx_kernel<kFmtW4> : gemm_gate_up_mx_kernel<kFmtW2>;
  hipLaunchKernelGGL(kern, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads), kGateUpLds, s,
                     p->gu_codes, p->gu_scales, (const uint8_t*)(wsb + ws.xq),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     wsb + ws.aq, (long long*)(wsb + ws.counters), T, p->K, p->I, top_k, nblk);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                            uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  const int P = T * top_k;
  const int nblk = (p->K + BN - 1) / BN;
  if (p->fmt == kFmtNV4) {
    hipLaunchKernelGGL(gemm_down_nv4_kernel, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads),
                       kAStages * N4Tile::kBytes, s, p->dn_codes, p->dn_scales, p->scale2,
                       (const _Float16*)(wsb + ws.aq), (const int32_t*)(wsb + ws.offsets),
                       (const int32_t*)(wsb + ws.perm), (const int32_t*)(wsb + ws.tiles),
                       (const int32_t*)(wsb + ws.meta), (float*)(wsb + ws.pair_out), p->K, p->I, nblk);
    return hipGetLastError();
  }
  // the streamed kernel (2-bit planes; the MXFP4 instance would not fit its registers): tiles of
  // 8 or 2 k-tiles (I = 2048, or 512 as on a 4-way tensor-parallel rank: with the epilogue
  // position a multiple of 3), whole N-blocks, pair rows and planes addressable by 31-bit offsets
  const long long b_tiles = (long long)p->E * (p->K / kTileRows) * (p->I / kTileK);   // down B tiles
  if (p->fmt == kFmtW2 && (p->I == 8 * kTileK || p->I == 2 * kTileK) && p->K % BN == 0 &&
      (long long)P * p->K * 4 < (1ll << 31) && b_tiles * kTileCodeBytes <= kMaxPlaneView) {
    auto kern = p->I == 8 * kTileK ? gemm_down_mx_stream_kernel<kFmtW2, 8> : gemm_down_mx_stream_kernel<kFmtW2, 2>;
    hipLaunchKernelGGL(kern, dim3(stream_grid()), dim3(kThreads), kDnStreamLds, s,
                       p->dn_codes, p->dn_scales, (const uint8_t*)(wsb + ws.aq),
                       (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                       (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                       (float*)(wsb + ws.pair_out), P, p->K, nblk, (uint32_t)b_tiles);
    return hipGetLastError();
  }
  auto kern = p->fmt == kFmtW4 ? gemm_down_mx_kernel<kFmtW4> : gemm_down_mx_kernel<kFmtW2>;
  hipLaunchKernelGGL(kern, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads),
                     kAStages * A6Tile::kBytes, s,
                     p->dn_codes, p->dn_scales, (const uint8_t*)(wsb + ws.aq),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (float*)(wsb + ws.pair_out), P, p->K, p->I, nblk);
  return hipGetLastError();
}

}  // namespace moew2
