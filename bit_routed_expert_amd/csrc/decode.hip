// Decode-shaped expert GEMMs: few tokens per expert, the whole activated expert set streamed
// from HBM once per call. Decode time is set by the weight bytes read from HBM (README bullet
// "FP4 recovery - used surgically"), so the kernels are organised around keeping enough weight
// tiles in flight: every wave streams its tiles through a 4-deep register ring while the matrix
// cores consume the previous ones, with the expert's tokens (up to kChunk at a time) as the
// 16-row A operand staged in LDS.
//
// For 2-bit and MXFP4 planes both projections run on the block-scaled instruction (fp8 A x fp4 B,
// operand order in common.h): the 2-bit codes become e2m1 operands with two bit operations per 8
// values and their UE8M0 bytes are the instruction's B scales. The A operand is split into e4m3
// parts while it is staged: x (bf16) into two parts, the gated intermediate (fp16) into three;
// both splits are exact for every value within 2^-10 of its block maximum. NVFP4 planes run on
// the 16 x 16 x 32 bf16 / fp16 instructions with the rows staged as they are and each B operand
// formed exactly in registers (e2m1 x e4m3), scale_2 applied to the fp32 results.
// gate_up: a = silu(g) * u from fp32 accumulators, rounded to fp16.
// down:    per-pair fp32 rows.
// combine: y[t] = sum over j ascending of w[t, j] * o[t*top_k + j] in fp32.
//
// Load ordering: a workgroup first issues its staging loads (x or the gated rows), then the
// first kRing weight tiles of every wave, and only then waits - for the staging loads alone -
// before writing LDS. Weight tiles are raw buffer loads; a tile past the end of a wave's range is
// requested at an out-of-range offset (no memory access), so the load sequence never branches
// and the ring's waits stay exact.
//
// Three organisations ("The v0.24.0 port", bullet "Deterministic unpermute": per-pair outputs are
// placed bijectively and summed in a fixed order, no atomics on values):
//  * routed (8 < P <= kDecodeMaxPairs): one group per kChunk pairs of an active expert, found
//    by each workgroup from the ids (no routing pass, see pair_group); the down kernel writes
//    per-pair rows o[p] and combine_kernel sums them in j order per token.
//  * sorted (any P; AUTO from kSortedMinPairs): workgroup rows walk the chunk list of a routing
//    pass in expert order; up to kWideMaxPairs pairs an expert's rows form groups of 16 whose
//    gate_up reduction is split over workgroups (one weight pass per 16 rows) and whose down
//    stage takes 8 rows per pass (decode_gate_up_sorted_kernel, decode_down_sorted_kernel).
//  * direct (tiny batches, P = T*top_k <= kDirectMaxPairs): no routing pass; gate_up runs one
//    group per pair, and one down kernel covers every pair of a column block and combines in LDS.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int kChunk = 4;     // token rows per pass (valid rows of the 16-row MFMA tile)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;      // weight tiles in flight per wave
constexpr int kStage = 4;     // 16-byte staging pieces per thread per memory round trip

// One expert's planes as buffer views, and the tile index (within the expert) of k-tile 0 of
// each of the wave's row groups (up to two).
struct WaveTiles {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t tile[2];
};

template <int FMT>
MOEW2_DEV WaveTiles wave_tiles(const uint8_t* codes, const uint8_t* scales, int e, uint32_t tiles_per_expert) {
  constexpr uint32_t cb = WFmt<FMT>::kCodeBytes;
  WaveTiles wt;
  wt.codes = buffer_view(codes + (size_t)e * tiles_per_expert * cb, tiles_per_expert * cb);
  constexpr uint32_t sb = WFmt<FMT>::kScaleBytes;
  wt.scales = buffer_view(scales + (size_t)e * tiles_per_expert * sb, tiles_per_expert * sb);
  return wt;
}

// Weight tile registers of one k-tile: per row group (NB of them), the lane's code bytes (16 for
// 2-bit codes, 2 x 16 for fp4 codes; tile layouts in common.h) and its scales: two UE8M0 bytes
// (instructions 0 and 1 of the k-tile), or for NVFP4 planes two words of four e4m3 bytes (half c,
// instruction j).
template <int NB, int FMT>
struct TileRegs {
  u32x4_t c[NB][WFmt<FMT>::kLoads];
  uint32_t s[NB][WFmt<FMT>::kScaleWords];
};

// The tile's byte offset goes in the scalar offset; the lane's offset (shifted out of range when
// the tile is not wanted - a wave-uniform condition) in the range-checked vector offset.
template <int NB, int FMT>
MOEW2_DEV void load_tile(TileRegs<NB, FMT>& r, const WaveTiles& wt, int kt, bool valid, int lane) {
  const uint32_t oob = valid ? 0u : kOutOfRange;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t t = wt.tile[b] + (uint32_t)kt;
#pragma unroll
    for (int q = 0; q < WFmt<FMT>::kLoads; ++q)
      r.c[b][q] = buf_ld16_nt(wt.codes, (16u * (uint32_t)lane) | oob, t * WFmt<FMT>::kCodeBytes + 1024u * q);
    if constexpr (FMT == kFmtNV4) {
      const u32x2_t sv = buf_ld8_nt(wt.scales, (128u * (uint32_t)(lane >> 5) + 8u * (uint32_t)(lane & 15)) | oob,
                                    t * kTileScaleBytesNV4);
      r.s[b][0] = sv[0];
      r.s[b][1] = sv[1];
    } else {
      r.s[b][0] = buf_ld2_nt(wt.scales, (2u * (uint32_t)lane) | oob, t * kTileScaleBytes);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Staged A rows. A row of reduction length KR split into NP parts is laid out in LDS as
//   part 0 [KR] bytes | ... | part NP-1 [KR] | scale words [KR/256][4 lane groups][SW bytes] | pad
// with SW = 4 for two parts (part 0 c0, c1, part 1 c0, c1) and 8 for three parts (the same,
// then part 2 c0, c1, 0, 0); c = instruction 0 or 1 of the k-tile.
// NP = 0 (bf16) and 1 (fp16): the row's 16-bit values unchanged, for the NVFP4 planes' 16 x 16 x 32
// instructions; a 16-byte pad per row puts the 16 rows of an operand read on distinct banks.
// ---------------------------------------------------------------------------------------------
template <int NP>
struct MxRow {
  static constexpr bool kRaw = NP < 2;
  static constexpr int kSW = NP == 2 ? 4 : 8;
  __host__ __device__ static int stride(int KR) { return kRaw ? 2 * KR + 16 : NP * KR + KR / kTileK * 4 * kSW + 64; }
};
// activation row formats: x (bf16) and the gated intermediate (fp16) for each weight format
template <int FMT> constexpr int kXRow = FMT == kFmtNV4 ? 0 : 2;
template <int FMT> constexpr int kARow = FMT == kFmtNV4 ? 1 : 3;

// Pieces of 16 bytes (8 values) of n rows; piece idx of the flat [n][len/8] range goes to thread
// idx % NT; a batch covers kStage pieces per thread, issued together and committed together.
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

// Splitting commit: the 4 pieces of a 32-value block sit in 4 consecutive lanes, which agree on
// the block maximum through two lane swaps. NP = 2: bf16 source (x); NP = 3: fp16 source (the
// gated intermediate). With count_inf, ninf gains the number of infinite source values.
template <int NT, int NP>
MOEW2_DEV void stage_commit_split(const Stage& st, uint8_t* lds, int stride, int KR, int n, int base, int tid,
                                  bool count_inf, int& ninf) {
  const int per_row = KR / 8, total = n * per_row;
  if constexpr (MxRow<NP>::kRaw) {
    // 16-bit rows stored as they come (NP = 1: fp16, whose infinities are counted)
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int idx = base + i * NT + tid;
      if (idx < total) {
        const u32x4_t v = st.v[i];
        if (NP == 1 && count_inf) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ninf += (__builtin_isinf(f16_lo(v[q])) ? 1 : 0) + (__builtin_isinf(f16_hi(v[q])) ? 1 : 0);
        }
        const int m = idx / per_row, c8 = idx - m * per_row;
        *reinterpret_cast<u32x4_t*>(lds + (size_t)m * stride + 16 * c8) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int idx = base + i * NT + tid;
    const bool ok = idx < total;
    const u32x4_t v = st.v[i];
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = NP == 2 ? bf16_lo(v[q]) : f16_lo(v[q]);
      f[2 * q + 1] = NP == 2 ? bf16_hi(v[q]) : f16_hi(v[q]);
    }
    float a = 0.f;
    if (ok) {
#pragma unroll
      for (int q = 0; q < 8; ++q) a = __builtin_fmaxf(a, __builtin_fabsf(f[q]));
    }
    a = __builtin_fmaxf(a, __shfl_xor(a, 1, 64));
    a = __builtin_fmaxf(a, __shfl_xor(a, 2, 64));
    if (ok) {
      if (count_inf) {
#pragma unroll
        for (int q = 0; q < 8; ++q) ninf += __builtin_isinf(f[q]) ? 1 : 0;
      }
      const int m = idx / per_row, c8 = idx - m * per_row;
      const uint32_t sx = x_scale_byte(a);
      uint8_t* row = lds + (size_t)m * stride;
      uint32_t p0a, p0b, p1a, p1b, p2a = 0, p2b = 0;
      if (NP == 2) {
        x_split4(f[0], f[1], f[2], f[3], sx, p0a, p1a);
        x_split4(f[4], f[5], f[6], f[7], sx, p0b, p1b);
      } else {
        a_split4(f[0], f[1], f[2], f[3], sx, p0a, p1a, p2a);
        a_split4(f[4], f[5], f[6], f[7], sx, p0b, p1b, p2b);
      }
      *reinterpret_cast<u32x2_t*>(row + 8 * c8) = u32x2_t{p0a, p0b};
      *reinterpret_cast<u32x2_t*>(row + KR + 8 * c8) = u32x2_t{p1a, p1b};
      if (NP == 3) *reinterpret_cast<u32x2_t*>(row + 2 * KR + 8 * c8) = u32x2_t{p2a, p2b};
      if ((c8 & 3) == 0) {
        const int b = c8 >> 2, kt = b >> 3, d = b & 7, g = d & 3, c = d >> 2;
        uint8_t* sw = row + NP * KR + (kt * 4 + g) * MxRow<NP>::kSW;
        sw[c] = (uint8_t)sx;
        sw[2 + c] = (uint8_t)(NP == 2 ? x_lo_scale_byte(sx) : a_part_scale(sx, 1));
        if (NP == 3) sw[4 + c] = (uint8_t)a_part_scale(sx, 2);
      }
    }
    // one piece at a time: interleaving the pieces' conversions would raise the register peak
    // while the weight ring is in flight
    __builtin_amdgcn_sched_barrier(0);
  }
}

MOEW2_DEV i32x8_t a_operand(const uint8_t* part, int c, int g) {
  const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(part + 128 * c + 16 * g);
  const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(part + 128 * c + 64 + 16 * g);
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Instruction C (0, 1) of one k-tile for the NB row groups, all NP parts.
template <int C, int NP, int NB, int FMT>
MOEW2_DEV void mma_chunk(const TileRegs<NB, FMT>& r, const uint8_t* kbase, int KR, uint32_t w0, uint32_t w1, int g,
                         f32x4_t* acc) {
  const i32x8_t a0 = a_operand(kbase, C, g);
  const i32x8_t a1 = a_operand(kbase + KR, C, g);
  i32x8_t a2;
  if (NP == 3) a2 = a_operand(kbase + 2 * KR, C, g);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const i32x8_t bo = b_operand<FMT, C>(r.c[b]);
    acc[b] = mx_mfma<C, C>(a0, bo, acc[b], w0, r.s[b][0]);
    acc[b] = mx_mfma<2 + C, C>(a1, bo, acc[b], w0, r.s[b][0]);
    if (NP == 3) acc[b] = mx_mfma<C, C>(a2, bo, acc[b], w1, r.s[b][0]);
  }
}

// One k-tile of NVFP4 planes from a 16-bit staged row: per half c and instruction j, lane group g
// supplies row values 256kt + 128c + 32j + 8g .. + 7 (one 16-byte LDS read) and the B values at
// the same reduction positions (NV4 tile layout in common.h); NP = 0: bf16 rows, 1: fp16.
template <int NP, int NB>
MOEW2_DEV void mma_tile_nv4(const TileRegs<NB, kFmtNV4>& r, const uint8_t* arow, int kt, int g, f32x4_t* acc) {
  const uint8_t* kb = arow + 2 * (kt * kTileK + 8 * g);
  static_for<0, 2>([&](auto cc) {
    constexpr int C = decltype(cc)::value;
    static_for<0, 4>([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kb + 2 * (128 * C + 32 * J));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (NP == 0) acc[b] = mfma32_bf16(a, nv4_b_bf16<J>(r.c[b][C][J], r.s[b][C]), acc[b]);
        else acc[b] = mfma32_f16(a, nv4_b_f16<J>(r.c[b][C][J], r.s[b][C]), acc[b]);
      }
    });
  });
}

// One k-tile from the lane's staged row `arow`.
template <int NP, int NB, int FMT>
MOEW2_DEV void mma_tile(const TileRegs<NB, FMT>& r, const uint8_t* arow, int KR, int kt, int g, f32x4_t* acc) {
  if constexpr (FMT == kFmtNV4) {
    static_assert(MxRow<NP>::kRaw, "NVFP4 planes take 16-bit activation rows");
    mma_tile_nv4<NP, NB>(r, arow, kt, g, acc);
    return;
  } else {
  const uint8_t* kbase = arow + kt * kTileK;
  const uint8_t* sw = arow + NP * KR + (kt * 4 + g) * MxRow<NP>::kSW;
  const uint32_t w0 = *reinterpret_cast<const uint32_t*>(sw);
  const uint32_t w1 = NP == 3 ? *reinterpret_cast<const uint32_t*>(sw + 4) : 0u;
  mma_chunk<0, NP, NB, FMT>(r, kbase, KR, w0, w1, g, acc);
  mma_chunk<1, NP, NB, FMT>(r, kbase, KR, w0, w1, g, acc);
  }
}

// ring[i] <- k-tile kb + i for i in [I0, I1) (out-of-range requests past ke)
template <int NB, int FMT, int I0 = 0, int I1 = kRing>
MOEW2_DEV void prime_ring(TileRegs<NB, FMT> (&ring)[kRing], const WaveTiles& wt, int kb, int ke, int lane) {
#pragma unroll
  for (int i = I0; i < I1; ++i) load_tile<NB, FMT>(ring[i], wt, kb + i, kb + i < ke, lane);
}

// Consume k-tiles [kb, ke) from the primed ring; each consumed slot is refilled with the tile
// kRing further on (or an out-of-range request), so every iteration issues the same loads. The
// staged rows hold the reduction from k-tile koff on.
template <int NP, int NB, int FMT>
MOEW2_DEV void stream_k(TileRegs<NB, FMT> (&ring)[kRing], const WaveTiles& wt, int kb, int ke, const uint8_t* arow,
                        int KR, int g, f32x4_t* acc, int lane, int koff = 0) {
  for (int k0 = kb; k0 < ke; k0 += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kt = k0 + i;
      if (kt < ke) mma_tile<NP, NB, FMT>(ring[i], arow, KR, kt - koff, g, acc);
      load_tile<NB, FMT>(ring[i], wt, kt + kRing, kt + kRing < ke, lane);
    }
  }
}

// R row pairs of one wave as one continuous stream (KS = 1, nk a multiple of kRing): the slot
// that held k-tile kt of row pair r is refilled with step r * nk + kt + kRing of the sequence,
// which past the pair's last k-tile is the next pair's first, so the ring never drains between
// pairs. Row pair r accumulates into acc[r]. The stream covers k-tiles koff .. koff + nk - 1 of
// rows with nkt k-tiles each (rows of pair r + 1 start at tile 2 * nkt further); the staged rows
// hold the reduction from k-tile koff on.
template <int NP, int NB, int FMT, int R>
MOEW2_DEV void stream_rows(TileRegs<NB, FMT> (&ring)[kRing], const WaveTiles& wt, int nk, const uint8_t* arow,
                           int KR, int g, f32x4_t (&acc)[R][NB], int lane, int nkt, int koff = 0) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    for (int k0 = 0; k0 < nk; k0 += kRing) {
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        const int kt = k0 + i;
        mma_tile<NP, NB, FMT>(ring[i], arow, KR, kt, g, acc[r]);
        const int kn = kt + kRing;
        const bool wrap = kn >= nk;
        const int rn = wrap ? r + 1 : r;
        load_tile<NB, FMT>(ring[i], wt, 2 * rn * nkt + koff + (wrap ? kn - nk : kn), rn < R, lane);
      }
    }
  }
}

// Stage n rows (split into NP parts) while the weight ring is primed. Batches beyond the first
// go first, one round trip each; the first batch is issued just before the prime and committed
// after it, so every path reaches the streaming loop with the same loads outstanding (the
// compiler's waits inside the loop stay exact). The thread index is passed through an empty asm
// so that the staging addresses are recomputed per call instead of being hoisted out of an
// enclosing loop and held in registers across the stream. With count_inf, ninf gains the number
// of infinite staged values.
// SPLIT: ring slots primed before the staged rows are committed (the rest after). For a kernel
// whose every workgroup starts at once and reads the same few rows (the tiny-batch organisation),
// priming the whole ring first puts the entire weight volume in the memory queues ahead of those
// row loads; committing first leaves the memory idle while every workgroup waits for the same
// rows. Priming part of the ring first keeps weights streaming while the rows arrive: measured
// best at one slot of four for the tiny-batch gate_up (T=1 gate_up 9.7 -> 9.3 us against two;
// all four: 10.2; none: 10.8) and two for the tiny-batch down (one: within noise; four: 9.1 us
// against 8.4).
template <int NT, int NP, int NB, int FMT, int SPLIT = kRing, class RowOff>
MOEW2_DEV void stage_and_prime(TileRegs<NB, FMT> (&ring)[kRing], const WaveTiles& wt, int kb, int ke, int lane,
                               uint8_t* lds, int stride, const uint16_t* src, int KR, int n, RowOff row_off,
                               int tid, bool count_inf, int& ninf) {
  int st_tid = tid;
  asm volatile("" : "+v"(st_tid));
  Stage st;
  for (int base = kStage * NT; base < n * (KR / 8); base += kStage * NT) {
    stage_issue<NT>(st, src, KR, n, base, row_off, st_tid);
    stage_commit_split<NT, NP>(st, lds, stride, KR, n, base, st_tid, count_inf, ninf);
  }
  stage_issue<NT>(st, src, KR, n, 0, row_off, st_tid);
  prime_ring<NB, FMT, 0, SPLIT>(ring, wt, kb, ke, lane);
  __builtin_amdgcn_sched_barrier(0);   // the first ring loads go out before the commit waits
  stage_commit_split<NT, NP>(st, lds, stride, KR, n, 0, st_tid, count_inf, ninf);
  prime_ring<NB, FMT, SPLIT, kRing>(ring, wt, kb, ke, lane);
}

// Cross-wave sum of split-K partial accumulators (KS waves per row pair) into the ks == 0 wave.
template <int KS>
MOEW2_DEV void reduce_split_k(f32x4_t* acc, float* red, int w, int ks, int lane) {
  if (KS == 1) return;
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

// The same for accumulators of up to 16 token rows (all 64 lanes). `red` may alias the staged
// rows: every wave is past its stream before any partial is written.
template <int KS>
MOEW2_DEV void reduce_split_k16(f32x4_t* acc, float* red, int w, int ks, int lane) {
  if (KS == 1) return;
  __syncthreads();
  if (ks > 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((w * 2 + b) * 4 + r) * 64 + lane] = acc[b][r];
  }
  __syncthreads();
  if (ks == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[b][r];
        for (int kk = 1; kk < KS; ++kk) v += red[(((w + kk) * 2 + b) * 4 + r) * 64 + lane];
        acc[b][r] = v;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Routing inside the decode kernels (8 < P <= kDecodeMaxPairs, no routing pass): workgroup row p
// (blockIdx.y) finds all pairs of expert e = ids[p] in ascending pair order with wave ballots over
// the ids - the order of the routing pass's stable sort ("The v0.24.0 port", bullet
// "Deterministic unpermute") - and takes the kChunk of them that start at p when p's rank among
// them is a multiple of kChunk. Other rows, and rows whose id is outside [0, E), exit at once.
// Pair p's gated row is act[p].
// ---------------------------------------------------------------------------------------------
constexpr int kScanBallots = kDecodeMaxPairs / 64;   // 64 pairs per ballot
static_assert(kDecodeMaxPairs == 2 * kThreads, "two ids per thread");

struct ScanLds {
  uint64_t ball[kScanBallots];    // pairs of the selected expert, ballot i = pairs 64i .. 64i+63
  int bad[kWaves];                // invalid ids seen by each wave
};

// Index of the k-th (from 0) set bit of v (v has more than k set bits).
MOEW2_DEV int select_bit64(uint64_t v, int k) {
  int pos = 0;
#pragma unroll
  for (int width = 32; width >= 1; width >>= 1) {
    const int c = __popcll(v & ((1ull << width) - 1ull));
    if (k >= c) { k -= c; v >>= width; pos += width; }
  }
  return pos;
}

// Selects the chunk of workgroup row p: its expert e, the expert's pair count n and the rank c0
// of pair p among them; true (for the whole workgroup) when p starts a chunk, i.e. c0 is a
// multiple of kChunk - so the kChunk-pair chunks of a popular expert run on separate rows in
// parallel instead of one after another. With `counters` non-null the workgroup also records
// the invalid pair count and clears the overflow count.
MOEW2_DEV bool pair_group(const int32_t* ids, int P, int E, int p, ScanLds& sh, int tid, int lane, int w,
                          long long* counters, int& e, int& n, int& c0) {
  e = ids[p];
  const int id0 = tid < P ? ids[tid] : -1;
  const int id1 = tid + kThreads < P ? ids[tid + kThreads] : -1;
  const uint64_t b0 = __ballot(id0 == e), b1 = __ballot(id1 == e);
  int bad = 0;
  if (counters)
    bad = __popcll(__ballot(tid < P && (id0 < 0 || id0 >= E))) +
          __popcll(__ballot(tid + kThreads < P && (id1 < 0 || id1 >= E)));
  if (lane == 0) {
    sh.ball[w] = b0;
    sh.ball[kWaves + w] = b1;
    sh.bad[w] = bad;
  }
  __syncthreads();
  if (counters && tid == 0) {
    int total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) total += sh.bad[i];
    counters[0] = total;
    counters[1] = 0;
  }
  if (e < 0 || e >= E) return false;
  const int word = p >> 6;
  c0 = __popcll(sh.ball[word] & ((1ull << (p & 63)) - 1ull));
  n = 0;
#pragma unroll
  for (int i = 0; i < kScanBallots; ++i) {
    if (i < word) c0 += __popcll(sh.ball[i]);
    n += __popcll(sh.ball[i]);
  }
  return c0 % kChunk == 0;
}

// Pair index of the m-th pair (from 0) of the selected group.
MOEW2_DEV int pair_at(const ScanLds& sh, int m) {
#pragma unroll
  for (int i = 0; i < kScanBallots; ++i) {
    const int c = __popcll(sh.ball[i]);
    if (m < c) return 64 * i + select_bit64(sh.ball[i], m);
    m -= c;
  }
  return 0;
}

// Chunk of the sorted organisation: workgroup row ti takes the ti-th entry of the routing pass's
// chunk list, in expert order: (expert, value). value = first sorted row rs of a group | slice cs
// << 20 | (slices - 1) << 22. A group of at most kChunk rows is one entry (cs = 0, one slice);
// with the wide list (forwards of at most kWideMaxPairs pairs) an expert's rows form groups of
// kWideRows, each entry of a larger group one of its ceil(rows / kChunk) slices. The down stage
// takes such a group as halves of kDownRows rows, one per even entry.
constexpr int kWideRows = kWideSlices * kChunk;   // 16: one full MFMA row tile
struct SortedChunk {
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tiles;
  const int32_t* meta;
};
struct ChunkEntry {
  int e, rs, cs, ncs;
};
MOEW2_DEV bool chunk_entry(const SortedChunk& sc, int ti, ChunkEntry& c) {
  if (ti >= sc.meta[1]) return false;
  c.e = sc.tiles[2 * ti];
  const int v = sc.tiles[2 * ti + 1];
  c.rs = v & 0xFFFFF;
  c.cs = (v >> 20) & 3;
  c.ncs = ((v >> 22) & 3) + 1;
  return true;
}
static_assert(kChunk == kDecodeChunk, "the routing pass cuts chunks of the decode kernels' size");

// ---------------------------------------------------------------------------------------------
// gate_up: grid (I / (16*NP), groups). Wave w handles row-pair q = blockIdx.x*NP + w/KS (gate row
// group 2q, up row group 2q+1) over the reduction slice w%KS of KS = 4/NP.
// kDecodeDirect: group = pair blockIdx.y (expert ids[p]). kDecodeRouted: group = the kChunk pairs
// of expert ids[blockIdx.y] from blockIdx.y on, when blockIdx.y starts such a chunk (pair_group).
// The gated row of pair p is act[p] in both.
// ---------------------------------------------------------------------------------------------
template <int NPW, int MODE, int FMT>
__global__ void __launch_bounds__(kThreads)
decode_gate_up_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                      const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                      _Float16* __restrict__ act, long long* __restrict__ counters,
                      int P, int E, int K, int I, int top_k, const float* __restrict__ scale2) {
  constexpr int KS = kWaves / NPW;
  constexpr bool DIRECT = MODE == kDecodeDirect;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ ScanLds sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  int e, n;
  int pr[kChunk];   // pair and token of each staged row (the same in every lane)
  bool valid = true;
  if constexpr (MODE == kDecodeDirect) {
    // no early exit: the x row is requested together with the id (an invalid pair streams no
    // weights and gets a row of zeros, which the down stage stages like any other)
    const int id = ids[blockIdx.y];
    valid = id >= 0 && id < E;
    e = valid ? id : 0;
    n = 1;
#pragma unroll
    for (int m = 0; m < kChunk; ++m) pr[m] = (int)blockIdx.y;
  } else {
    static_assert(MODE == kDecodeRouted, "the sorted organisation has its own gate_up kernel");
    long long* cnt = blockIdx.x == 0 && blockIdx.y == 0 ? counters : nullptr;
    int n_total, first;
    if (!pair_group(ids, P, E, blockIdx.y, sh, tid, lane, w, cnt, e, n_total, first)) return;
    n = min(kChunk, n_total - first);
#pragma unroll
    for (int m = 0; m < kChunk; ++m) pr[m] = pair_at(sh, first + min(m, n - 1));
  }
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int pw = w / KS, ks = w % KS;
  const int q = blockIdx.x * NPW + pw;
  WaveTiles wt = wave_tiles<FMT>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * q * nkt);
  wt.tile[1] = (uint32_t)((2 * q + 1) * nkt);
  const int kb = ks * nkt / KS, ke = valid ? (ks + 1) * nkt / KS : kb;
  // NVFP4: scale_2 of the expert's gate and up tensors, applied to the fp32 results
  const float sg = FMT == kFmtNV4 ? scale2[3 * e] : 1.f, su = FMT == kFmtNV4 ? scale2[3 * e + 1] : 1.f;
  constexpr int XR = kXRow<FMT>;
  const int stride = MxRow<XR>::stride(K);
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][2][4][16]
  TileRegs<2, FMT> ring[kRing];
  {
    auto row_off = [&](int m) -> size_t {
      const int pp = m == 0 ? pr[0] : m == 1 ? pr[1] : m == 2 ? pr[2] : pr[3];
      return (size_t)(pp / top_k) * K;
    };
    int ninf = 0;
    stage_and_prime<kThreads, XR, 2, FMT, DIRECT ? 1 : kRing>(ring, wt, kb, ke, lane, lds, stride, x, K, n,
                                                                row_off, tid, false, ninf);
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    stream_k<XR, 2, FMT>(ring, wt, kb, ke, lds + (size_t)ma * stride, K, lane >> 4, acc, lane);
    reduce_split_k<KS>(acc, red, w, ks, lane);
    if (ks == 0 && lane < 16) {
      // accumulator register r of lanes 0..15 holds token row r, column lane
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        if (r < n) {
          const int pp = r == 0 ? pr[0] : r == 1 ? pr[1] : r == 2 ? pr[2] : pr[3];
          act[(size_t)pp * I + 16 * q + lane] = valid ? (_Float16)silu_mul(acc[0][r] * sg, acc[1][r] * su) : (_Float16)0.f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// gate_up of the sorted organisation: grid (I / (16*NP), chunk entries). An entry of one slice
// is the routed kernel's work for its <= kChunk rows (the same arithmetic, bit for bit). An entry
// cs of a group of up to kWideRows rows split into ncs slices stages those rows over its share
// [k0, k1) of the reduction only (the same LDS as kChunk whole rows), so one weight pass serves
// up to 16 rows instead of 4, and writes the gate and up partial sums (times scale_2 for NVFP4
// planes) to gu_part[cs][pair]; wide_finish_kernel sums the slices and forms the gated rows.
// ---------------------------------------------------------------------------------------------
template <int NPW, int FMT, int NW>
__global__ void __launch_bounds__(64 * NW)
decode_gate_up_sorted_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                             const uint16_t* __restrict__ x, _Float16* __restrict__ act, float* __restrict__ gu_part,
                             int32_t* __restrict__ pair_ncs, int P, int K, int I, int top_k, SortedChunk sc,
                             const float* __restrict__ scale2) {
  constexpr int KS = NW / NPW;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int row_pair[kWideRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  ChunkEntry c;
  if (!chunk_entry(sc, blockIdx.y, c)) return;
  const int e = c.e;
  const bool wide = c.ncs > 1;
  const int n = min(wide ? kWideRows : kChunk, sc.offsets[e + 1] - c.rs);
  if (tid < kWideRows) row_pair[tid] = sc.perm[c.rs + min(tid, n - 1)];
  const int nkt = K / kTileK, nrg = 2 * I / kTileRows;
  const int k0 = c.cs * nkt / c.ncs, nk = (c.cs + 1) * nkt / c.ncs - k0;
  const int pw = w / KS, ks = w % KS;
  const int q = blockIdx.x * NPW + pw;
  WaveTiles wt = wave_tiles<FMT>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * q * nkt);
  wt.tile[1] = (uint32_t)((2 * q + 1) * nkt);
  const int kb = k0 + ks * nk / KS, ke = k0 + (ks + 1) * nk / KS;
  const float sg = FMT == kFmtNV4 ? scale2[3 * e] : 1.f, su = FMT == kFmtNV4 ? scale2[3 * e + 1] : 1.f;
  constexpr int XR = kXRow<FMT>;
  const int KR = nk * kTileK;
  const int stride = MxRow<XR>::stride(KR);
  __syncthreads();   // row_pair
  TileRegs<2, FMT> ring[kRing];
  auto row_off = [&](int m) -> size_t { return (size_t)(row_pair[m] / top_k) * K + (size_t)k0 * kTileK; };
  int ninf = 0;
  stage_and_prime<64 * NW, XR, 2, FMT>(ring, wt, kb, ke, lane, lds, stride, x, KR, n, row_off, tid, false, ninf);
  __syncthreads();
  const int ma = min(lane & 15, n - 1);
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  stream_k<XR, 2, FMT>(ring, wt, kb, ke, lds + (size_t)ma * stride, KR, lane >> 4, acc, lane, k0);
  reduce_split_k16<KS>(acc, reinterpret_cast<float*>(lds), w, ks, lane);
  if (ks != 0) return;
  // accumulator register r of lane l holds token row 4 (l / 16) + r, column l % 16
  const int col = 16 * q + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * (lane >> 4) + r;
    if (row < n) {
      const int pp = row_pair[row];
      if (!wide) {
        act[(size_t)pp * I + col] = (_Float16)silu_mul(acc[0][r] * sg, acc[1][r] * su);
      } else {
        float* gp = gu_part + ((size_t)c.cs * P + pp) * 2 * I;
        gp[col] = acc[0][r] * sg;
        gp[I + col] = acc[1][r] * su;
      }
    }
  }
  // the slice count of each pair's group, for wide_finish_kernel (one writer per pair). Last, after
  // every use of blockIdx.x: under a blockIdx.x == 0 test the compiler substitutes 0 for it, and a
  // use past the test's lane-divergent join then takes a vector register, which turns every weight
  // offset derived from it into a per-load loop over the lanes' values.
  if (blockIdx.x == 0 && c.cs == 0 && w == 0 && lane < n) pair_ncs[row_pair[lane]] = c.ncs;
}

// Gated rows of the split groups: for pair blockIdx.x whose group has more than one slice (its
// slice count written by the gate_up kernel this forward), a = silu(sum of the gate slices) *
// (sum of the up slices), slices added in order, rounded to fp16 into act[pair]. Other pairs, and
// pairs whose id is outside [0, E) (never written), return at once.
__global__ void __launch_bounds__(256)
wide_finish_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ pair_ncs,
                   const float* __restrict__ gu_part, _Float16* __restrict__ act, int P, int E, int I) {
  const int p = blockIdx.x;
  const int id = ids[p], ncs = pair_ncs[p];
  if (id < 0 || id >= E || ncs < 2) return;
  for (int i = 4 * (int)threadIdx.x; i < I; i += 4 * 256) {
    f32x4_t gs = *reinterpret_cast<const f32x4_t*>(gu_part + (size_t)p * 2 * I + i);
    f32x4_t us = *reinterpret_cast<const f32x4_t*>(gu_part + (size_t)p * 2 * I + I + i);
    for (int cs = 1; cs < ncs; ++cs) {
      const float* gp = gu_part + ((size_t)cs * P + p) * 2 * I;
      gs += *reinterpret_cast<const f32x4_t*>(gp + i);
      us += *reinterpret_cast<const f32x4_t*>(gp + I + i);
    }
    const _Float16 h0 = (_Float16)silu_mul(gs[0], us[0]), h1 = (_Float16)silu_mul(gs[1], us[1]);
    const _Float16 h2 = (_Float16)silu_mul(gs[2], us[2]), h3 = (_Float16)silu_mul(gs[3], us[3]);
    *reinterpret_cast<u32x2_t*>(act + (size_t)p * I + i) =
        u32x2_t{(uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16)};
  }
}

// ---------------------------------------------------------------------------------------------
// routed down: grid (K / (32*NPW*R), P). The group is that of the gate_up stage (pair_group);
// wave w handles the R row pairs rq .. rq + R - 1, rq = (blockIdx.x*NPW + w/KS) * R (row groups
// 2*rq and 2*rq + 1 of each), over the reduction slice w%KS; with R = 2 (whole reduction per
// wave) the two pairs are one continuous weight stream, which halves the workgroups and the
// per-workgroup costs (group scan, staging, ring start) per byte. Per-pair rows go to pair_out at
// the pair index (bijective);
// combine_kernel then sums them per token in j order. The blockIdx.x == 0 workgroups count the
// gated intermediates that overflowed fp16 (each pair belongs to one group).
// ---------------------------------------------------------------------------------------------
template <int NPW, int FMT, int R>
__global__ void __launch_bounds__(kThreads)
decode_down_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                   const _Float16* __restrict__ act, const int32_t* __restrict__ ids,
                   float* __restrict__ pair_out, long long* __restrict__ counters, int P, int E, int K,
                   int I, const float* __restrict__ scale2) {
  constexpr int KS = kWaves / NPW;
  static_assert(R == 1 || KS == 1, "row pairs per wave need the whole reduction in each wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ ScanLds sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  int e, n_e, first;
  if (!pair_group(ids, P, E, blockIdx.y, sh, tid, lane, w, nullptr, e, n_e, first)) return;
  const int n = min(kChunk, n_e - first);
  int pr[kChunk];
#pragma unroll
  for (int m = 0; m < kChunk; ++m) pr[m] = pair_at(sh, first + min(m, n - 1));
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int pw = w / KS, ks = w % KS;
  const int rq = (blockIdx.x * NPW + pw) * R;   // the wave's first row pair
  WaveTiles wt = wave_tiles<FMT>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * rq * nkt);
  wt.tile[1] = (uint32_t)((2 * rq + 1) * nkt);
  const int kb = ks * nkt / KS, ke = (ks + 1) * nkt / KS;
  constexpr int AR = kARow<FMT>;
  const int stride = MxRow<AR>::stride(I);
  float* red = reinterpret_cast<float*>(lds + (size_t)kChunk * stride);  // [kWaves][2][4][16]
  const uint16_t* act16 = reinterpret_cast<const uint16_t*>(act);
  const float sd = FMT == kFmtNV4 ? scale2[3 * e + 2] : 1.f;   // NVFP4: the down tensor's scale_2
  TileRegs<2, FMT> ring[kRing];
  {
    auto row_off = [&](int m) -> size_t {
      const int pp = m == 0 ? pr[0] : m == 1 ? pr[1] : m == 2 ? pr[2] : pr[3];
      return (size_t)pp * I;
    };
    int ninf = 0;
    stage_and_prime<kThreads, AR, 2, FMT>(ring, wt, kb, ke, lane, lds, stride, act16, I, n, row_off, tid,
                                    blockIdx.x == 0, ninf);
    if (ninf) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)ninf);
    __syncthreads();
    const int ma = min(lane & 15, n - 1);
    f32x4_t acc[R][2];
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q][0] = acc[q][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (R == 1) {
      stream_k<AR, 2, FMT>(ring, wt, kb, ke, lds + (size_t)ma * stride, I, lane >> 4, acc[0], lane);
      reduce_split_k<KS>(acc[0], red, w, ks, lane);
    } else {
      stream_rows<AR, 2, FMT, R>(ring, wt, nkt, lds + (size_t)ma * stride, I, lane >> 4, acc, lane, nkt);
    }
    if (ks == 0 && lane < 16) {
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int col = 16 * (2 * (rq + q) + b) + lane;
#pragma unroll
          for (int r = 0; r < kChunk; ++r) {
            if (r < n) {
              const int pp = r == 0 ? pr[0] : r == 1 ? pr[1] : r == 2 ? pr[2] : pr[3];
              pair_out[(size_t)pp * K + col] = acc[q][b][r] * sd;
            }
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// down of the sorted organisation: grid (K / (32*NPW*R), chunk entries), NW waves per workgroup.
// With the wide list a group of at most kDownRows rows is taken by its entry 0 over the whole
// reduction (its other entry exits); a larger group (three or four entries) by its entries 0 and
// 1, each over all its rows and one half of the reduction (k-tiles [0, nkt/2) and [nkt/2, nkt)),
// writing fp32 partial rows to pair_out and pair_out2 (summed by the combine), so one weight pass
// serves up to 16 rows; entries 2 and 3 exit. With the plain list an entry is its 4-row chunk.
// Per-row arithmetic of an unsplit group as in the routed kernel (bit-identical rows).
// ---------------------------------------------------------------------------------------------
constexpr int kDownRows = 2 * kChunk;
template <int NPW, int FMT, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
decode_down_sorted_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                          const _Float16* __restrict__ act, float* __restrict__ pair_out, float* __restrict__ pair_out2,
                          long long* __restrict__ counters, int K, int I, int wide, SortedChunk sc,
                          const float* __restrict__ scale2) {
  constexpr int KS = NW / NPW;
  static_assert(R == 1 || KS == 1, "row pairs per wave need the whole reduction in each wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int row_pair[kWideRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  ChunkEntry c;
  if (!chunk_entry(sc, blockIdx.y, c)) return;
  const bool split = wide && c.ncs > 2;                      // more than kDownRows rows
  if (wide && c.cs >= (split ? 2 : 1)) return;
  const int e = c.e;
  const int h = split ? c.cs : 0;                            // reduction half of a split group
  const int row0 = c.rs + kChunk * c.cs * !wide;
  const int n = min(wide ? (split ? kWideRows : kDownRows) : kChunk, sc.offsets[e + 1] - row0);
  if (tid < kWideRows) row_pair[tid] = sc.perm[row0 + min(tid, n - 1)];
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int k0 = h * (nkt / 2), nk = split ? (h ? nkt - nkt / 2 : nkt / 2) : nkt;   // this entry's k-tiles
  const int pw = w / KS, ks = w % KS;
  const int rq = (blockIdx.x * NPW + pw) * R;   // the wave's first row pair
  WaveTiles wt = wave_tiles<FMT>(codes, scales, e, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(2 * rq * nkt);
  wt.tile[1] = (uint32_t)((2 * rq + 1) * nkt);
  const int kb = k0 + ks * nk / KS, ke = k0 + (ks + 1) * nk / KS;
  constexpr int AR = kARow<FMT>;
  const int KR = nk * kTileK;
  const int stride = MxRow<AR>::stride(KR);
  const uint16_t* act16 = reinterpret_cast<const uint16_t*>(act);
  const float sd = FMT == kFmtNV4 ? scale2[3 * e + 2] : 1.f;   // NVFP4: the down tensor's scale_2
  __syncthreads();   // row_pair
  TileRegs<2, FMT> ring[kRing];
  auto row_off = [&](int m) -> size_t { return (size_t)row_pair[m] * I + (size_t)k0 * kTileK; };
  int ninf = 0;
  // every staged value is counted once: by the first column slice, in each half of a split group
  stage_and_prime<64 * NW, AR, 2, FMT>(ring, wt, kb, ke, lane, lds, stride, act16, KR, n, row_off, tid,
                                       blockIdx.x == 0, ninf);
  if (ninf) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)ninf);
  __syncthreads();
  const int ma = min(lane & 15, n - 1);
  f32x4_t acc[R][2];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q][0] = acc[q][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (R == 1) {
    stream_k<AR, 2, FMT>(ring, wt, kb, ke, lds + (size_t)ma * stride, KR, lane >> 4, acc[0], lane, k0);
    reduce_split_k16<KS>(acc[0], reinterpret_cast<float*>(lds), w, ks, lane);
  } else {
    stream_rows<AR, 2, FMT, R>(ring, wt, nk, lds + (size_t)ma * stride, KR, lane >> 4, acc, lane, nkt, k0);
  }
  if (ks != 0) return;
  float* out = h ? pair_out2 : pair_out;
  // accumulator register r of lane l holds token row 4 (l / 16) + r, column l % 16
#pragma unroll
  for (int q = 0; q < R; ++q)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = 16 * (2 * (rq + q) + b) + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * (lane >> 4) + r;
        if (row < n) out[(size_t)row_pair[row] * K + col] = acc[q][b][r] * sd;
      }
    }
}

// ---------------------------------------------------------------------------------------------
// direct down + combine for tiny batches: grid (K/16). The workgroup covers one row group (16
// output columns) for every pair; wave w takes pair w/2 and half w%2 of the reduction; per-pair
// results meet in LDS and are combined per token in j order. Block 0 also records the two
// counters (single writer).
// ---------------------------------------------------------------------------------------------
constexpr int kDirectWaves = 2 * kDirectMaxPairs;   // two reduction halves per pair
constexpr int kDirectThreads = 64 * kDirectWaves;

template <int FMT>
__global__ void __launch_bounds__(kDirectThreads)
decode_down_direct_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                          const _Float16* __restrict__ act, const int32_t* __restrict__ ids,
                          const float* __restrict__ wts, void* __restrict__ y, long long* __restrict__ counters,
                          int out_dtype, int T, int E, int K, int I, int top_k, const float* __restrict__ scale2) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int P = T * top_k;                         // <= kDirectMaxPairs
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform in the wave)
  const int nkt = I / kTileK, nrg = K / kTileRows;
  const int rg = blockIdx.x;
  constexpr int AR = kARow<FMT>;
  const int stride = MxRow<AR>::stride(I);
  float* o = reinterpret_cast<float*>(lds + (size_t)kDirectMaxPairs * stride);  // [P][16]
  float* red = o + kDirectMaxPairs * 16;                                        // [P][16]
  // wave w: pair p = w / 2, reduction half w % 2
  const int p = w >> 1, hk = w & 1;
  const int id = p < P ? ids[p] : -1;
  const bool valid = id >= 0 && id < E;
  WaveTiles wt = wave_tiles<FMT>(codes, scales, valid ? id : 0, (uint32_t)(nrg * nkt));
  wt.tile[0] = (uint32_t)(rg * nkt);
  wt.tile[1] = 0;
  const int kb = hk * nkt / 2, ke = valid ? (hk + 1) * nkt / 2 : kb;
  // ids and router weights of the combine, read now rather than after the stream
  __shared__ int cid[kDirectMaxPairs];
  __shared__ float cw[kDirectMaxPairs];
  __shared__ int cnt[2];
  if (tid < P) {
    cid[tid] = ids[tid];
    cw[tid] = wts[tid];
  }
  if (tid < 2) cnt[tid] = 0;
  // gated rows of all pairs (rows of invalid pairs are staged but never read); block 0 counts the
  // infinite ones while staging them
  const uint16_t* act16 = reinterpret_cast<const uint16_t*>(act);
  auto row_off = [&](int m) -> size_t { return (size_t)m * I; };
  TileRegs<1, FMT> ring[kRing];
  int ninf = 0;
  stage_and_prime<kDirectThreads, AR, 1, FMT, kRing / 2>(ring, wt, kb, ke, lane, lds, stride, act16, I, P, row_off,
                                                   tid, blockIdx.x == 0, ninf);
  __syncthreads();
  if (blockIdx.x == 0) {
    // counters: invalid pairs, and infinite gated intermediates (the rows of invalid pairs are
    // zeros, written by the gate_up stage)
    if (ninf) atomicAdd(&cnt[1], ninf);
    if (tid < P && (cid[tid] < 0 || cid[tid] >= E)) atomicAdd(&cnt[0], 1);
  }
  f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
  stream_k<AR, 1, FMT>(ring, wt, kb, ke, lds + (size_t)(p < P ? p : 0) * stride, I, lane >> 4, acc, lane);
  if (valid && hk == 1 && lane < 16) red[p * 16 + lane] = acc[0][0];
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) {
    counters[0] = cnt[0];
    counters[1] = cnt[1];
  }
  if (valid && hk == 0 && lane < 16)
    o[p * 16 + lane] = (acc[0][0] + red[p * 16 + lane]) * (FMT == kFmtNV4 ? scale2[3 * id + 2] : 1.f);
  __syncthreads();
  // combine: y[t][16*rg + c] = sum_j w[t,j] * o[t*top_k+j][c]
  for (int idx = tid; idx < T * 16; idx += kDirectThreads) {
    const int t = idx / 16, c = idx - t * 16;
    float sum = 0.f;
    for (int j = 0; j < top_k; ++j) {
      const int pp = t * top_k + j;
      const int ii = cid[pp];
      if (ii < 0 || ii >= E) continue;
      sum += cw[pp] * o[pp * 16 + c];
    }
    const size_t yo = (size_t)t * K + 16 * rg + c;
    if (out_dtype == MOE_W2_OUT_F32) reinterpret_cast<float*>(y)[yo] = sum;
    else reinterpret_cast<uint16_t*>(y)[yo] = f32_to_bf16_rne(sum);
  }
}

// y[t] = sum_j (ascending) w[t, j] * o[t*top_k + j]; ids outside [0, E) contribute nothing.
// One thread per 4 output columns of one token. A group of up to 8 pairs has its ids, weights and
// pair rows requested together (rows of invalid pairs are read but not used), so a token costs
// one memory round trip per 8 pairs; the sum itself runs in ascending j. With pair_ncs (the
// sorted decode organisation's wide list), a pair of a group of more than kDownRows rows has its
// down output in two reduction halves, o = pair_out[p] + pair_out2[p], added before weighting.
__global__ void combine_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wts,
                               const float* __restrict__ pair_out, const int32_t* __restrict__ pair_ncs,
                               const float* __restrict__ pair_out2, void* __restrict__ y,
                               int T, int top_k, int E, int K, int out_dtype) {
  constexpr int G = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = K / 4;
  if (gid >= (long long)T * q) return;
  const int t = (int)(gid / q), c = (int)(gid - (long long)t * q) * 4;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int j0 = 0; j0 < top_k; j0 += G) {
    int id[G], ns[G];
    float w[G];
    float4 o[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (j0 + i < top_k) {
        const int p = t * top_k + j0 + i;
        id[i] = ids[p];
        w[i] = wts[p];
        ns[i] = pair_ncs ? pair_ncs[p] : 0;
        // each per-pair row is read once: nontemporal keeps it from evicting L2 lines
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pair_out + (size_t)p * K + c));
        o[i] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    if (pair_ncs) {
      // second halves, requested only for the pairs whose group was split (a second round trip
      // for those tokens; reading every pair's would cost batches without split groups as much)
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (j0 + i < top_k && id[i] >= 0 && id[i] < E && ns[i] > 2) {
          const int p = t * top_k + j0 + i;
          const f32x4_t v =
              __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pair_out2 + (size_t)p * K + c));
          o[i].x += v[0]; o[i].y += v[1]; o[i].z += v[2]; o[i].w += v[3];
        }
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

// The sorted organisation's gate_up runs 8-wave workgroups where its LDS would fit fewer than four
// 4-wave workgroups per CU (160 KB of LDS): the same waves per CU in fewer, wider workgroups whose
// staged rows serve twice the columns (Zipf T=64 batch at K=6144: gate_up 202 -> 192 us).
constexpr size_t kLdsPerCu = 160 * 1024;
inline bool sorted_wide8(size_t lds) { return lds > kLdsPerCu / 4; }

}  // namespace

size_t decode_direct_lds(int I) {
  return (size_t)kDirectMaxPairs * MxRow<3>::stride(I) + (size_t)kDirectMaxPairs * 2 * 16 * 4;
}

static SortedChunk sorted_chunks(const Workspace& ws, const uint8_t* wsb) {
  return SortedChunk{(const int32_t*)(wsb + ws.offsets), (const int32_t*)(wsb + ws.perm),
                     (const int32_t*)(wsb + ws.tiles), (const int32_t*)(wsb + ws.meta)};
}

template <int FMT>
static hipError_t decode_gate_up_fmt(const moe_w2_planes* p, int T, int top_k, const void* x,
                                     const int32_t* ids, const Workspace& ws, uint8_t* wsb, int mode,
                                     hipStream_t s) {
  const int P = T * top_k;
  const size_t lds = (size_t)kChunk * MxRow<2>::stride(p->K) + (size_t)kWaves * 2 * 4 * 16 * 4;
  const uint16_t* xb = (const uint16_t*)x;
  _Float16* act = (_Float16*)(wsb + ws.act);
  long long* cnt = (long long*)(wsb + ws.counters);
  if (mode == kDecodeDirect) {
    hipLaunchKernelGGL((decode_gate_up_kernel<1, kDecodeDirect, FMT>), dim3(p->I / 16, P), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, act, cnt, P, p->E, p->K, p->I, top_k, p->scale2);
  } else if (mode == kDecodeSorted) {
    // one workgroup row per chunk entry of the routing pass (at most max_chunks; rows past meta[1]
    // exit); the same split of the reduction over waves as the routed organisation, so that
    // entries of one slice give bit-identical results. LDS: the staged rows of the largest entry
    // (kChunk whole rows, or 4 ncs rows of a 1/ncs share of the reduction) - the reduction of the
    // waves' partial sums reuses it.
    const bool wide = P <= kWideMaxPairs;
    const int nkt = p->K / kTileK;
    size_t lds_s = 0;
    for (int ncs = 1; ncs <= (wide ? kWideSlices : 1); ++ncs) {
      const size_t rows = ncs == 1 ? kChunk : (size_t)kChunk * ncs;
      lds_s = std::max(lds_s, rows * MxRow<kXRow<FMT>>::stride((nkt + ncs - 1) / ncs * kTileK));
    }
    lds_s = std::max(lds_s, (size_t)kWaves * 2 * 4 * 64 * 4);
    float* gu_part = (float*)(wsb + ws.gu_part);
    int32_t* pair_ncs = (int32_t*)(wsb + ws.pair_ncs);
    const SortedChunk sc = sorted_chunks(ws, wsb);
    if (pick_np(min(p->E, P)) == 4 && sorted_wide8(lds_s))
      hipLaunchKernelGGL((decode_gate_up_sorted_kernel<8, FMT, 8>), dim3(p->I / 128, ws.max_chunks), dim3(512),
                         lds_s, s, p->gu_codes, p->gu_scales, xb, act, gu_part, pair_ncs, P, p->K, p->I, top_k, sc, p->scale2);
    else if (pick_np(min(p->E, P)) == 4)
      hipLaunchKernelGGL((decode_gate_up_sorted_kernel<4, FMT, kWaves>), dim3(p->I / 64, ws.max_chunks),
                         dim3(kThreads), lds_s, s, p->gu_codes, p->gu_scales, xb, act, gu_part, pair_ncs, P, p->K,
                         p->I, top_k, sc, p->scale2);
    else
      hipLaunchKernelGGL((decode_gate_up_sorted_kernel<1, FMT, kWaves>), dim3(p->I / 16, ws.max_chunks),
                         dim3(kThreads), lds_s, s, p->gu_codes, p->gu_scales, xb, act, gu_part, pair_ncs, P, p->K,
                         p->I, top_k, sc, p->scale2);
    if (wide)
      hipLaunchKernelGGL(wide_finish_kernel, dim3(P), dim3(256), 0, s, ids, pair_ncs, gu_part, act, P, p->E, p->I);
  } else if (pick_np(min(p->E, P)) == 4) {   // at most this many workgroup rows do work
    hipLaunchKernelGGL((decode_gate_up_kernel<4, kDecodeRouted, FMT>), dim3(p->I / 64, P), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, act, cnt, P, p->E, p->K, p->I, top_k, p->scale2);
  } else {
    hipLaunchKernelGGL((decode_gate_up_kernel<1, kDecodeRouted, FMT>), dim3(p->I / 16, P), dim3(kThreads), lds, s,
                       p->gu_codes, p->gu_scales, xb, ids, act, cnt, P, p->E, p->K, p->I, top_k, p->scale2);
  }
  return hipGetLastError();
}

hipError_t launch_decode_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                                 const int32_t* ids, const Workspace& ws, uint8_t* wsb, int mode,
                                 hipStream_t s) {
  if (T * top_k == 0) return hipSuccess;
  if (p->fmt == kFmtNV4) return decode_gate_up_fmt<kFmtNV4>(p, T, top_k, x, ids, ws, wsb, mode, s);
  return p->fmt == kFmtW4 ? decode_gate_up_fmt<kFmtW4>(p, T, top_k, x, ids, ws, wsb, mode, s)
                          : decode_gate_up_fmt<kFmtW2>(p, T, top_k, x, ids, ws, wsb, mode, s);
}

template <int FMT>
static hipError_t decode_down_routed(const moe_w2_planes* p, int rows, int P, const int32_t* ids, const Workspace& ws,
                                     uint8_t* wsb, hipStream_t s) {
  const int groups = min(p->E, P);   // both organisations split the reduction alike (bit-identical results)
  const size_t lds = (size_t)kChunk * MxRow<3>::stride(p->I) + (size_t)kWaves * 2 * 4 * 16 * 4;
  const _Float16* act = (const _Float16*)(wsb + ws.act);
  long long* cnt = (long long*)(wsb + ws.counters);
  float* po = (float*)(wsb + ws.pair_out);
  const bool two_pairs = FMT == kFmtW2 && (p->I / kTileK) % kRing == 0 && p->K % 256 == 0;
  if (pick_np(groups) == 4 && two_pairs)
    hipLaunchKernelGGL((decode_down_kernel<4, FMT, 2>), dim3(p->K / 256, rows), dim3(kThreads), lds, s,
                       p->dn_codes, p->dn_scales, act, ids, po, cnt, P, p->E, p->K, p->I, p->scale2);
  else if (pick_np(groups) == 4)
    hipLaunchKernelGGL((decode_down_kernel<4, FMT, 1>), dim3(p->K / 128, rows), dim3(kThreads), lds, s,
                       p->dn_codes, p->dn_scales, act, ids, po, cnt, P, p->E, p->K, p->I, p->scale2);
  else
    hipLaunchKernelGGL((decode_down_kernel<1, FMT, 1>), dim3(p->K / 32, rows), dim3(kThreads), lds, s,
                       p->dn_codes, p->dn_scales, act, ids, po, cnt, P, p->E, p->K, p->I, p->scale2);
  return hipGetLastError();
}

// down of the sorted organisation: one workgroup row per chunk entry; the same kernel shapes as the
// routed organisation (two row pairs per wave for 2-bit planes). 4-wave workgroups even where the
// 8 staged rows limit them to three per CU: measured against 8-wave ones (two per CU) on T=64
// batches, uniform and Zipf(1.1) at K=4096 and 6144, they were faster in all four (down 91 vs
// 100 us uniform at K=4096), the wider workgroups' fewer, longer rows of work balancing worse.
template <int FMT>
static hipError_t decode_down_sorted(const moe_w2_planes* p, int P, const Workspace& ws, uint8_t* wsb, hipStream_t s) {
  const int wide = P <= kWideMaxPairs ? 1 : 0;
  const int groups = min(p->E, P);
  const int nkt = p->I / kTileK;
  constexpr int AR = kARow<FMT>;
  // staged rows: kChunk whole rows (plain list), or kDownRows whole rows / kWideRows rows over the
  // larger reduction half (wide list)
  const size_t rows_lds =
      wide ? std::max((size_t)kDownRows * MxRow<AR>::stride(p->I),
                      (size_t)kWideRows * MxRow<AR>::stride((nkt - nkt / 2) * kTileK))
           : (size_t)kChunk * MxRow<AR>::stride(p->I);
  const float* sc2 = p->scale2;
  const _Float16* act = (const _Float16*)(wsb + ws.act);
  long long* cnt = (long long*)(wsb + ws.counters);
  float* po = (float*)(wsb + ws.pair_out);
  float* po2 = wide ? (float*)(wsb + ws.gu_part) : nullptr;   // the gate_up partials are summed by now
  const SortedChunk sc = sorted_chunks(ws, wsb);
  const unsigned rows = (unsigned)ws.max_chunks;
  // two row pairs per wave stream whole multiples of the ring: nkt, and with the wide list its halves
  const bool two_pairs = FMT == kFmtW2 && nkt % (wide ? 2 * kRing : kRing) == 0;
  if (pick_np(groups) == 4 && two_pairs)
    hipLaunchKernelGGL((decode_down_sorted_kernel<4, FMT, 2, kWaves>), dim3(p->K / 256, rows), dim3(kThreads),
                       rows_lds, s, p->dn_codes, p->dn_scales, act, po, po2, cnt, p->K, p->I, wide, sc, sc2);
  else if (pick_np(groups) == 4)
    hipLaunchKernelGGL((decode_down_sorted_kernel<4, FMT, 1, kWaves>), dim3(p->K / 128, rows), dim3(kThreads),
                       rows_lds, s, p->dn_codes, p->dn_scales, act, po, po2, cnt, p->K, p->I, wide, sc, sc2);
  else
    hipLaunchKernelGGL((decode_down_sorted_kernel<1, FMT, 1, kWaves>), dim3(p->K / 32, rows), dim3(kThreads),
                       std::max(rows_lds, (size_t)kWaves * 2 * 4 * 64 * 4), s, p->dn_codes, p->dn_scales, act, po,
                       po2, cnt, p->K, p->I, wide, sc, sc2);
  return hipGetLastError();
}

template <int FMT>
static hipError_t decode_down_fmt(const moe_w2_planes* p, int T, int top_k, const int32_t* ids, const float* w,
                                  void* y, int out_dtype, const Workspace& ws, uint8_t* wsb, int mode,
                                  hipStream_t s) {
  const int P = T * top_k;
  if (mode == kDecodeDirect) {
    const _Float16* act = (const _Float16*)(wsb + ws.act);
    long long* cnt = (long long*)(wsb + ws.counters);
    hipLaunchKernelGGL(decode_down_direct_kernel<FMT>, dim3(p->K / 16), dim3(kDirectThreads), decode_direct_lds(p->I),
                       s, p->dn_codes, p->dn_scales, act, ids, w, y, cnt, out_dtype, T, p->E, p->K, p->I, top_k, p->scale2);
    return hipGetLastError();
  }
  return mode == kDecodeSorted ? decode_down_sorted<FMT>(p, P, ws, wsb, s)
                               : decode_down_routed<FMT>(p, P, P, ids, ws, wsb, s);
}

hipError_t launch_decode_down(const moe_w2_planes* p, int T, int top_k, const int32_t* ids, const float* w,
                              void* y, int out_dtype, const Workspace& ws, uint8_t* wsb, int mode,
                              hipStream_t s) {
  if (T * top_k == 0) return hipSuccess;
  if (p->fmt == kFmtNV4) return decode_down_fmt<kFmtNV4>(p, T, top_k, ids, w, y, out_dtype, ws, wsb, mode, s);
  return p->fmt == kFmtW4 ? decode_down_fmt<kFmtW4>(p, T, top_k, ids, w, y, out_dtype, ws, wsb, mode, s)
                          : decode_down_fmt<kFmtW2>(p, T, top_k, ids, w, y, out_dtype, ws, wsb, mode, s);
}

hipError_t launch_combine(int T, int top_k, int E, int K, const int32_t* ids, const float* w,
                          const float* pair_out, void* y, int out_dtype, hipStream_t s, const int32_t* pair_ncs,
                          const float* pair_out2) {
  const long long n = (long long)T * (K / 4);
  if (n == 0) return hipSuccess;
  const int B = 256;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + B - 1) / B)), dim3(B), 0, s, ids, w, pair_out, pair_ncs,
                     pair_out2, y, T, top_k, E, K, out_dtype);
  return hipGetLastError();
}

}  // namespace moew2
