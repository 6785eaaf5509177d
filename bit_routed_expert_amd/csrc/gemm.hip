// Prefill-shaped grouped expert GEMMs (many tokens per expert), on the gfx950 matrix cores.
//
// Each workgroup computes a BM x BN tile of one expert: BM consecutive sorted pair rows (an
// M-tile from the routing pass) by BN weight rows. The A operand (activations) is staged through
// LDS one 256-wide k-tile at a time, double-buffered; for gate_up the rows are gathered from x through the
// sort permutation while they are staged, so gathered activations never round-trip through HBM
// (the pages' AFRAG variant repacks activations fragment-major in a separate pass - README
// bullet "The kernels", "The v0.24.0 port" bullet "AFRAG prefill"; here the LDS staging plays
// that role and every lane's A fragment is one 16-byte LDS read). The B operand (2-bit weights)
// is read by each wave straight from the native planes and decoded in registers.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int BM = kGemmBM;     // 64 sorted pair rows (4 MFMA row tiles)
constexpr int kWaves = 8;       // each wave: all BM rows x 64 weight rows (4 row groups of 16)
constexpr int BN = 64 * kWaves; // 512 weight rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kAStride = kTileK * 2 + 16;  // LDS row stride (bytes) of one k-tile of A, padded
constexpr int kABytes = BM * kAStride;
constexpr int kAPieces = BM * kTileK * 2 / 16 / kThreads;  // 16-byte A pieces per thread per k-tile
static_assert(kAPieces == 4, "A staging layout");

// Tile shape: the 2-bit weights cost 0.28 byte per element against 2 bytes for the bf16/fp16
// activations, so the workgroup tile is wide in N (512 weight rows) and short in M (64 rows):
// per k-tile it reads 32 KiB of A and 12 KiB of B for 1024 matrix instructions.
//
// The workgroup -> tile mapping is XCD-aware: consecutive workgroup ids are dispatched to the
// 8 XCDs in turn, so workgroup b takes logical tile (b % 8) * per_xcd + b / 8. Each XCD then walks
// a contiguous run of (M-tile, N-block) pairs, N-block fastest: the N-blocks of one M-tile run on
// one XCD at about the same time and read the M-tile's activations from that XCD's L2 once.
template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 1)
gemm_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
            const int32_t* __restrict__ dn_e0, const void* __restrict__ a_src,
            const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta,
            void* __restrict__ out, long long* __restrict__ counters,
            int K, int I, int top_k, int n_blocks) {
  typedef typename std::conditional<GATE_UP, Bf16Op, F16Op>::type Op;
  typedef typename Op::vec vec;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kABytes];
  // ---- tile of this workgroup ----
  const int n_tiles = meta[1];
  const int total = n_tiles * n_blocks;
  const int per_xcd = (total + 7) / 8;
  const int b = blockIdx.x;
  const int logical = (b & 7) * per_xcd + (b >> 3);
  if ((b >> 3) >= per_xcd || logical >= total) return;
  const int ti = logical / n_blocks, nb = logical - ti * n_blocks;
  const int e = tiles[2 * ti], rs = tiles[2 * ti + 1];
  const int rows_valid = min(BM, offsets[e + 1] - rs);
  const int KR = GATE_UP ? K : I;
  const int NR = GATE_UP ? 2 * I : K;
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // row groups 4*(nb*kWaves + w) .. +3 of this wave (gate_up: gate, up, gate, up)
  const int rg0 = 4 * (nb * kWaves + w);
  const bool wave_active = rg0 < nrg;   // a matrix with fewer than BN rows leaves waves idle

  // ---- A staging: thread t copies 16-byte piece (t % 32) of rows t/32 + 16*i, i = 0..3 ----
  const int piece = tid & 31;
  uint32_t arow[kAPieces];   // element offset of the piece's row start in the source matrix
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int r = tid / 32 + 16 * i;
    const int sr = rs + min(r, rows_valid - 1);
    arow[i] = GATE_UP ? (uint32_t)(perm[sr] / top_k) * (uint32_t)K : (uint32_t)sr * (uint32_t)I;
  }
  const uint16_t* asrc = reinterpret_cast<const uint16_t*>(a_src);
  u32x4_t areg[kAPieces];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) areg[i] = ld16(asrc + arow[i] + kt * kTileK + piece * 8);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i)
      *reinterpret_cast<u32x4_t*>(lds + buf * kABytes + (tid / 32 + 16 * i) * kAStride + piece * 16) = areg[i];
  };

  // ---- B: 4 row groups per wave, one native k-tile at a time, in two register sets ----
  const uint32_t tb0 = (uint32_t)((e * nrg + (wave_active ? rg0 : 0)) * nkt);
  struct BRegs { u32x4_t c[4]; u32x2_t s[4]; };
  BRegs bA, bB;
  auto load_b = [&](int kt, BRegs& r) {
    if (!wave_active) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t ti_ = tb0 + t * nkt + kt;
      r.c[t] = ld16(codes + (size_t)ti_ * kTileCodeBytes + 16 * lane);
      r.s[t] = ld8(scales + (size_t)ti_ * kTileScaleBytes + 8 * (lane & 15));
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one k-tile = 8 blocks of 32 = native dwords 0..3 (two blocks each)
  auto compute = [&](const uint8_t* abuf, const BRegs& br) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vec b0[4], b1[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t f0, f1;
        native_to_fp4(br.c[t][j], f0, f1);
        const uint32_t sw = j < 2 ? br.s[t][0] : br.s[t][1];
        const float s0 = (j & 1) == 0 ? ue8m0_scale_operand<0>(sw) : ue8m0_scale_operand<2>(sw);
        const float s1 = (j & 1) == 0 ? ue8m0_scale_operand<1>(sw) : ue8m0_scale_operand<3>(sw);
        b0[t] = Op::dequant(f0, s0);
        b1[t] = Op::dequant(f1, s1);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint8_t* ar = abuf + (m * 16 + (lane & 15)) * kAStride + (8 * (lane >> 4)) * 2;
        const vec a0 = *reinterpret_cast<const vec*>(ar + (32 * (2 * j)) * 2);
        const vec a1 = *reinterpret_cast<const vec*>(ar + (32 * (2 * j + 1)) * 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[m][t] = Op::mfma(a0, b0[t], acc[m][t]);
          acc[m][t] = Op::mfma(a1, b1[t], acc[m][t]);
        }
      }
    }
  };
  // k-tile kt computes from LDS buffer kt % 2 with B from `cur` (loaded one k-tile earlier);
  // meanwhile A and B of k-tile kt+1 are in flight and A lands in the other buffer at the end.
  auto k_tile = [&](int kt, const BRegs& cur, BRegs& nxt) {
    const bool more = kt + 1 < nkt;
    if (more) { load_b(kt + 1, nxt); load_a(kt + 1); }
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) compute(lds + (kt & 1) * kABytes, cur);
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

  // ---- epilogue ----
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int sr = rs + row;
      if (GATE_UP) {
        _Float16* act = reinterpret_cast<_Float16*>(out);
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float a = silu_mul(acc[m][2 * pr][r], acc[m][2 * pr + 1][r]);
          const _Float16 h = (_Float16)a;
          if (__builtin_isinf((float)h) && !__builtin_isinf(a)) atomicAdd((unsigned long long*)&counters[1], 1ull);
          const int col = 16 * (rg0 / 2 + pr) + (lane & 15);
          act[(size_t)sr * I + col] = h;
        }
      } else {
        const int p = perm[sr];
        float* o = reinterpret_cast<float*>(out);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = 16 * (rg0 + t) + (lane & 15);
          o[(size_t)p * K + col] = __builtin_ldexpf(acc[m][t][r], dn_e0[(size_t)e * K + col]);
        }
      }
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
  const int nblk = (2 * p->I + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_kernel<true>, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads), 0, s,
                     p->gu_codes, p->gu_scales, p->dn_e0, x,
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.act), (long long*)(wsb + ws.counters), p->K, p->I, top_k, nblk);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                            uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  const int nblk = (p->K + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_kernel<false>, dim3(gemm_grid(ws.max_tiles, nblk)), dim3(kThreads), 0, s,
                     p->dn_codes, p->dn_scales, p->dn_e0, (const void*)(wsb + ws.act),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.pair_out), (long long*)(wsb + ws.counters), p->K, p->I, top_k, nblk);
  return hipGetLastError();
}

}  // namespace moew2
