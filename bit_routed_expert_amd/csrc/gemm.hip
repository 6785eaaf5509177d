// Prefill-shaped grouped expert GEMMs (many tokens per expert), on the gfx950 matrix cores.
//
// Each workgroup computes a BM x BN tile of one expert: BM consecutive sorted pair rows (an
// M-tile from the routing pass) by BN weight rows. The A operand (activations) is staged through
// LDS in BK-wide slices, double-buffered; for gate_up the rows are gathered from x through the
// sort permutation while they are staged, so gathered activations never round-trip through HBM
// (the pages' AFRAG variant repacks activations fragment-major in a separate pass - README
// bullet "The kernels", "The v0.24.0 port" bullet "AFRAG prefill"; here the LDS staging plays
// that role and every lane's A fragment is one 16-byte LDS read). The B operand (2-bit weights)
// is read by each wave straight from the native planes and decoded in registers.
#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int BM = kGemmBM;     // 128 sorted rows
constexpr int BN = 128;         // weight rows (8 row groups of 16)
constexpr int BK = 128;         // reduction slice per LDS buffer (half a native k-tile)
constexpr int kThreads = 256;   // 4 waves: 2 (M) x 2 (N), 64 x 64 each
constexpr int kAStride = BK * 2 + 16;  // LDS row stride (bytes), padded against bank conflicts
constexpr int kABytes = BM * kAStride;

template <bool GATE_UP>
__global__ void __launch_bounds__(kThreads, 2)
gemm_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
            const int32_t* __restrict__ dn_e0, const void* __restrict__ a_src,
            const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ tiles, const int32_t* __restrict__ meta,
            void* __restrict__ out, long long* __restrict__ counters,
            int K, int I, int top_k) {
  typedef typename std::conditional<GATE_UP, Bf16Op, F16Op>::type Op;
  typedef typename Op::vec vec;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kABytes];
  const int ti = blockIdx.x;
  if (ti >= meta[1]) return;
  const int e = tiles[2 * ti], rs = tiles[2 * ti + 1];
  const int rows_valid = min(BM, offsets[e + 1] - rs);
  const int KR = GATE_UP ? K : I;
  const int NR = GATE_UP ? 2 * I : K;
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const int nkb = KR / BK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  // ---- A staging: thread t copies 16-byte piece (t % 16) of rows t/16 + 16*i, i = 0..7 ----
  const uint8_t* arow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = tid / 16 + 16 * i;
    const int sr = rs + min(r, rows_valid - 1);
    if (GATE_UP) {
      const int t = perm[sr] / top_k;
      arow[i] = reinterpret_cast<const uint8_t*>(a_src) + (size_t)t * K * 2;
    } else {
      arow[i] = reinterpret_cast<const uint8_t*>(a_src) + (size_t)sr * I * 2;
    }
  }
  const int piece = tid & 15;
  u32x4_t areg[8];
  auto load_a = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) areg[i] = ld16(arow[i] + (size_t)(kb * BK + piece * 8) * 2);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4_t*>(lds + buf * kABytes + (tid / 16 + 16 * i) * kAStride + piece * 16) = areg[i];
  };

  // ---- B: 4 row groups per wave ----
  long long tbase[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) tbase[t] = ((long long)e * nrg + blockIdx.y * 8 + 4 * wn + t) * nkt;
  u32x4_t bc[4];
  u32x2_t bs[4];
  auto load_b = [&](int kt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bc[t] = ld16(codes + (tbase[t] + kt) * kTileCodeBytes + 16 * lane);
      bs[t] = ld8(scales + (tbase[t] + kt) * kTileScaleBytes + 8 * (lane & 15));
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();
  u32x4_t bc_next[4];
  u32x2_t bs_next[4];
  for (int kb = 0; kb < nkb; ++kb) {
    const int half = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) load_a(kb + 1);
    if (half == 0 && kb + 2 < nkb) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bc_next[t] = ld16(codes + (tbase[t] + kb / 2 + 1) * kTileCodeBytes + 16 * lane);
        bs_next[t] = ld8(scales + (tbase[t] + kb / 2 + 1) * kTileScaleBytes + 8 * (lane & 15));
      }
    }
    const uint8_t* abuf = lds + half * 0 + (kb & 1) * kABytes;
    // blocks 4*half .. 4*half+3 of the current k-tile: native dwords 2*half, 2*half+1
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * half + jj;
      vec b0[4], b1[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t f0, f1;
        native_to_fp4(bc[t][j], f0, f1);
        const uint32_t sw = j < 2 ? bs[t][0] : bs[t][1];
        float s0, s1;
        if ((j & 1) == 0) { s0 = ue8m0_scale_operand<0>(sw); s1 = ue8m0_scale_operand<1>(sw); }
        else { s0 = ue8m0_scale_operand<2>(sw); s1 = ue8m0_scale_operand<3>(sw); }
        b0[t] = Op::dequant(f0, s0);
        b1[t] = Op::dequant(f1, s1);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint8_t* ar = abuf + (wm * 64 + m * 16 + (lane & 15)) * kAStride + (8 * (lane >> 4)) * 2;
        const vec a0 = *reinterpret_cast<const vec*>(ar + (32 * (2 * jj)) * 2);
        const vec a1 = *reinterpret_cast<const vec*>(ar + (32 * (2 * jj + 1)) * 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[m][t] = Op::mfma(a0, b0[t], acc[m][t]);
          acc[m][t] = Op::mfma(a1, b1[t], acc[m][t]);
        }
      }
    }
    if (more) store_a((kb + 1) & 1);
    if (half == 1 && kb + 1 < nkb) {
#pragma unroll
      for (int t = 0; t < 4; ++t) { bc[t] = bc_next[t]; bs[t] = bs_next[t]; }
    }
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + m * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int sr = rs + row;
      if (GATE_UP) {
        _Float16* act = reinterpret_cast<_Float16*>(out);
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float a = silu_mul(acc[m][2 * pr][r], acc[m][2 * pr + 1][r]);
          const _Float16 h = (_Float16)a;
          if (__builtin_isinf((float)h) && !__builtin_isinf(a)) atomicAdd((unsigned long long*)&counters[1], 1ull);
          const int col = 16 * (blockIdx.y * 4 + 2 * wn + pr) + (lane & 15);
          act[(size_t)sr * I + col] = h;
        }
      } else {
        const int p = perm[sr];
        float* o = reinterpret_cast<float*>(out);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = 16 * (blockIdx.y * 8 + 4 * wn + t) + (lane & 15);
          o[(size_t)p * K + col] = __builtin_ldexpf(acc[m][t][r], dn_e0[(size_t)e * K + col]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                               const Workspace& ws, uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_kernel<true>, dim3(ws.max_tiles, 2 * p->I / BN), dim3(kThreads), 0, s,
                     p->gu_codes, p->gu_scales, p->dn_e0, x,
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.act), (long long*)(wsb + ws.counters), p->K, p->I, top_k);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                            uint8_t* wsb, hipStream_t s) {
  if (ws.max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_kernel<false>, dim3(ws.max_tiles, p->K / BN), dim3(kThreads), 0, s,
                     p->dn_codes, p->dn_scales, p->dn_e0, (const void*)(wsb + ws.act),
                     (const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta),
                     (void*)(wsb + ws.pair_out), (long long*)(wsb + ws.counters), p->K, p->I, top_k);
  return hipGetLastError();
}

}  // namespace moew2
