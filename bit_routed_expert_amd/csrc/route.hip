// Token-sort / expert-offset pass: a stable counting sort of the pairs p = t*top_k + j by
// expert id. Valid sorted ids form a permutation of token*top_k+j ("The v0.24.0 port",
// section "Our hooks", bullet "Deterministic unpermute"); ids outside [0, E) are placed last.
//
// The rank of a pair among the pairs of its expert is computed without atomics on counts:
// within a round of 256 pairs every pair sets its bit in a 256-bit mask of its expert (LDS),
// and its rank is the popcount of the mask bits below it. This keeps the sort stable and the
// output independent of scheduling.
#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

constexpr int kRoundThreads = 256;   // pairs per round
constexpr int kMaskWords = kRoundThreads / 32;
constexpr int kChunkRounds = 4;      // rounds per chunk in the multi-kernel path
constexpr int kChunkPairs = kRoundThreads * kChunkRounds;
constexpr int kSmallMaxPairs = 4096; // single-workgroup path

__device__ __forceinline__ int bin_of(int id, int E) { return (id >= 0 && id < E) ? id : E; }

// Entry m of the tile list of an expert with c pairs from sorted row s0: tiles of bm rows (value =
// first row), or with `wide` (the sorted decode organisation) groups of 4*bm rows, each split into
// ceil(rows / bm) reduction slices, entry m = slice m % 4 of group m / 4 (value = the group's first
// row | slice << 20 | (slices - 1) << 22). The entry count is ceil(c / bm) either way, and a group
// of at most bm rows is one entry with value = its first row.
__device__ __forceinline__ int32_t tile_value(int s0, int c, int m, int bm, int wide) {
  if (!wide) return s0 + m * bm;
  const int g = m >> 2, ks = m & 3;
  const int ng = min(4 * bm, c - 4 * bm * g);
  const int nks = (ng + bm - 1) / bm;
  return (s0 + 4 * bm * g) | (ks << 20) | ((nks - 1) << 22);
}

// In-place exclusive scan of n ints in LDS by the whole block; returns the total.
__device__ int block_exclusive_scan(int* data, int n, int* scratch /* blockDim ints */) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) if (b0 + i < n) local += data[b0 + i];
  scratch[tid] = local;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    int v = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += v;
    __syncthreads();
  }
  int run = scratch[tid] - local;  // exclusive prefix of this thread's segment
  for (int i = 0; i < per; ++i) {
    if (b0 + i < n) { int v = data[b0 + i]; data[b0 + i] = run; run += v; }
  }
  int total = scratch[nt - 1];
  __syncthreads();
  return total;
}

// Offsets, active-expert list, GEMM M-tile list and counters from per-bin totals held in LDS
// (`cnt` has E+1 entries and is overwritten by its exclusive scan). Shared by both paths.
__device__ void finish_routing(int* cnt, int E, int P, int* scratch, int* tmp,
                               int32_t* offsets, int32_t* active, int32_t* meta, int32_t* tiles,
                               long long* counters, int max_tiles, int bm, int wide) {
  const int tid = threadIdx.x, nt = blockDim.x;
  // per-expert activity and tile counts
  for (int b = tid; b < E; b += nt) tmp[b] = cnt[b] > 0 ? 1 : 0;
  __syncthreads();
  int n_active = block_exclusive_scan(tmp, E, scratch);
  for (int b = tid; b < E; b += nt) {
    int n = cnt[b];
    if (n > 0) active[tmp[b]] = b;  // tmp[b] = slot
  }
  __syncthreads();
  for (int b = tid; b < E; b += nt) tmp[b] = (cnt[b] + bm - 1) / bm;
  __syncthreads();
  int n_tiles = block_exclusive_scan(tmp, E, scratch);
  // offsets: exclusive scan of the E+1 bins (the last bin holds the invalid pairs)
  int tot = block_exclusive_scan(cnt, E + 1, scratch);
  (void)tot;
  for (int b = tid; b <= E; b += nt) offsets[b] = b < E ? cnt[b] : cnt[E];
  if (tid == 0) offsets[E] = cnt[E];  // = number of valid pairs
  for (int b = tid; b < E; b += nt) {
    int n = cnt[b + 1] - cnt[b];
    int t0 = tmp[b];
    for (int m = 0; m * bm < n; ++m) {
      if (t0 + m < max_tiles) { tiles[2 * (t0 + m)] = b; tiles[2 * (t0 + m) + 1] = tile_value(cnt[b], n, m, bm, wide); }
    }
  }
  if (tid == 0) {
    meta[0] = n_active;
    meta[1] = n_tiles < max_tiles ? n_tiles : max_tiles;
    if (counters) { counters[0] = (long long)(P - cnt[E]); counters[1] = 0; }
  }
}

// ---------------------------------------------------------------------------------------
// Single-workgroup routing for P <= kSmallMaxPairs.
// LDS: masks[(E+1)][8] words, running[E+1], cnt[E+1], tmp[E], rank[P], scratch[256].
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(kRoundThreads)
route_small_kernel(const int32_t* __restrict__ ids, int E, int P, int32_t* __restrict__ offsets,
                   int32_t* __restrict__ perm, int32_t* active, int32_t* meta, int32_t* tiles,
                   long long* counters, int max_tiles, int bm, int wide) {
  extern __shared__ int lds[];
  const int nb = E + 1;
  uint32_t* masks = reinterpret_cast<uint32_t*>(lds);
  int* running = lds + nb * kMaskWords;
  int* cnt = running + nb;
  int* tmp = cnt + nb;
  int* rank = tmp + nb;
  int* scratch = rank + kSmallMaxPairs;
  const int tid = threadIdx.x;
  for (int b = tid; b < nb; b += kRoundThreads) running[b] = 0;
  const int rounds = (P + kRoundThreads - 1) / kRoundThreads;
  for (int r = 0; r < rounds; ++r) {
    for (int i = tid; i < nb * kMaskWords; i += kRoundThreads) masks[i] = 0;
    __syncthreads();
    const int p = r * kRoundThreads + tid;
    int bin = -1;
    if (p < P) {
      bin = bin_of(ids[p], E);
      atomicOr(&masks[bin * kMaskWords + tid / 32], 1u << (tid % 32));
    }
    __syncthreads();
    if (bin >= 0) {
      const uint32_t* m = masks + bin * kMaskWords;
      int rk = running[bin];
      for (int w = 0; w < tid / 32; ++w) rk += __popc(m[w]);
      rk += __popc(m[tid / 32] & ((1u << (tid % 32)) - 1u));
      rank[p] = rk;
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kRoundThreads) {
      int c = 0;
      for (int w = 0; w < kMaskWords; ++w) c += __popc(masks[b * kMaskWords + w]);
      running[b] += c;
    }
    __syncthreads();
  }
  for (int b = tid; b < nb; b += kRoundThreads) cnt[b] = running[b];
  __syncthreads();
  finish_routing(cnt, E, P, scratch, tmp, offsets, active, meta, tiles, counters, max_tiles, bm, wide);
  __syncthreads();
  // cnt now holds the exclusive scan over bins (bin start positions)
  for (int p = tid; p < P; p += kRoundThreads) {
    const int bin = bin_of(ids[p], E);
    perm[cnt[bin] + rank[p]] = p;
  }
}

// ---------------------------------------------------------------------------------------
// One-round routing for P <= 1024 pairs and E <= 256 experts (decode batches): one thread per
// pair, a 1024-bit mask per expert, and a single block scan of three packed prefix sums per
// expert (pair count, GEMM M-tiles, active flag).
// ---------------------------------------------------------------------------------------
constexpr int kFastThreads = 1024;
constexpr int kFastWords = kFastThreads / 32;

__global__ void __launch_bounds__(kFastThreads)
route_fast_kernel(const int32_t* __restrict__ ids, int E, int P, int32_t* __restrict__ offsets,
                  int32_t* __restrict__ perm, int32_t* active, int32_t* meta, int32_t* tiles,
                  long long* counters, int max_tiles, int bm, int wide) {
  extern __shared__ int lds[];
  const int nb = E + 1;
  uint32_t* masks = reinterpret_cast<uint32_t*>(lds);     // [nb][32]
  int* pre = lds + nb * kFastWords;                        // [nb][32] pairs of the bin in earlier words
  int* cntb = pre + nb * kFastWords;                       // [nb] pairs of the bin
  int* start = cntb + nb;                                  // [nb]
  int* wsum = start + nb;                                  // [16]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < nb * kFastWords; i += kFastThreads) masks[i] = 0;
  __syncthreads();
  const int bin = tid < P ? bin_of(ids[tid], E) : -1;
  if (bin >= 0) atomicOr(&masks[bin * kFastWords + tid / 32], 1u << (tid % 32));
  __syncthreads();
  // per (bin, word): the word's pair count and the exclusive prefix over the bin's words, one
  // bin per 32 lanes (kFastWords = 32 words per bin, and 1024 % 32 == 0 keeps a segment on one bin)
  for (int i = tid; i < nb * kFastWords; i += kFastThreads) {
    const int pc = __popc(masks[i]);
    int inc = pc;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int o = __shfl_up(inc, d, 32);
      if ((lane & 31) >= d) inc += o;
    }
    pre[i] = inc - pc;
    if ((i & 31) == 31) cntb[i >> 5] = inc;
  }
  __syncthreads();
  int rank = 0;
  if (bin >= 0) {
    const int wi = bin * kFastWords + tid / 32;
    rank = pre[wi] + __popc(masks[wi] & ((1u << (tid % 32)) - 1u));
  }
  int c = 0;
  uint32_t v = 0;
  if (tid < nb) {
    c = cntb[tid];
    v = (uint32_t)c << 20;
    if (tid < E && c > 0) v |= ((uint32_t)((c + bm - 1) / bm) << 10) | 1u;
  }
  // block exclusive scan of the packed values (fields never carry into each other)
  uint32_t incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wv] = (int)incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < kFastThreads / 64; ++i) { int t = wsum[i]; wsum[i] = run; run += t; }
  }
  __syncthreads();
  const uint32_t excl = incl - v + (uint32_t)wsum[wv];
  if (tid < nb) {
    const int s0 = (int)(excl >> 20), t0 = (int)((excl >> 10) & 1023u), a0 = (int)(excl & 1023u);
    start[tid] = s0;
    offsets[tid] = s0;
    if (tid < E && c > 0) {
      active[a0] = tid;
      for (int m = 0; m * bm < c; ++m)
        if (t0 + m < max_tiles) { tiles[2 * (t0 + m)] = tid; tiles[2 * (t0 + m) + 1] = tile_value(s0, c, m, bm, wide); }
    }
    if (tid == E) {
      meta[0] = a0;
      meta[1] = t0 < max_tiles ? t0 : max_tiles;
      if (counters) { counters[0] = (long long)(P - s0); counters[1] = 0; }
    }
  }
  __syncthreads();
  if (bin >= 0) perm[start[bin] + rank] = tid;
}

// ---------------------------------------------------------------------------------------
// Multi-kernel routing for larger P: per-chunk ranks and counts, a scan, then the scatter.
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(kRoundThreads)
route_chunk_kernel(const int32_t* __restrict__ ids, int E, int P, int32_t* __restrict__ chunk_cnt,
                   int32_t* __restrict__ rank) {
  extern __shared__ int lds[];
  const int nb = E + 1;
  uint32_t* masks = reinterpret_cast<uint32_t*>(lds);
  int* running = lds + nb * kMaskWords;
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int b = tid; b < nb; b += kRoundThreads) running[b] = 0;
  for (int r = 0; r < kChunkRounds; ++r) {
    for (int i = tid; i < nb * kMaskWords; i += kRoundThreads) masks[i] = 0;
    __syncthreads();
    const int p = c * kChunkPairs + r * kRoundThreads + tid;
    int bin = -1;
    if (p < P) {
      bin = bin_of(ids[p], E);
      atomicOr(&masks[bin * kMaskWords + tid / 32], 1u << (tid % 32));
    }
    __syncthreads();
    if (bin >= 0) {
      const uint32_t* m = masks + bin * kMaskWords;
      int rk = running[bin];
      for (int w = 0; w < tid / 32; ++w) rk += __popc(m[w]);
      rk += __popc(m[tid / 32] & ((1u << (tid % 32)) - 1u));
      rank[p] = rk;
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kRoundThreads) {
      int cc = 0;
      for (int w = 0; w < kMaskWords; ++w) cc += __popc(masks[b * kMaskWords + w]);
      running[b] += cc;
    }
    __syncthreads();
  }
  for (int b = tid; b < nb; b += kRoundThreads) chunk_cnt[(long long)c * nb + b] = running[b];
}

// One workgroup: per-bin exclusive prefix over chunks (in place) and the routing summary.
__global__ void __launch_bounds__(1024)
route_scan_kernel(int E, int P, int nchunks, int32_t* __restrict__ chunk_cnt,
                  int32_t* __restrict__ offsets, int32_t* active, int32_t* meta, int32_t* tiles,
                  long long* counters, int max_tiles, int bm, int wide) {
  extern __shared__ int lds[];
  const int nb = E + 1;
  int* cnt = lds;
  int* tmp = cnt + nb;
  int* scratch = tmp + nb;
  const int tid = threadIdx.x;
  for (int b = tid; b < nb; b += blockDim.x) {
    int run = 0;
    int c = 0;
    for (; c + 8 <= nchunks; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = chunk_cnt[(long long)(c + u) * nb + b];
#pragma unroll
      for (int u = 0; u < 8; ++u) { chunk_cnt[(long long)(c + u) * nb + b] = run; run += v[u]; }
    }
    for (; c < nchunks; ++c) {
      int v = chunk_cnt[(long long)c * nb + b];
      chunk_cnt[(long long)c * nb + b] = run;
      run += v;
    }
    cnt[b] = run;
  }
  __syncthreads();
  finish_routing(cnt, E, P, scratch, tmp, offsets, active, meta, tiles, counters, max_tiles, bm, wide);
  __syncthreads();
  // keep the bin start positions for the scatter in offsets' spare copy: chunk_cnt row nchunks
  for (int b = tid; b < nb; b += blockDim.x) chunk_cnt[(long long)nchunks * nb + b] = cnt[b];
}

__global__ void __launch_bounds__(kRoundThreads)
route_scatter_kernel(const int32_t* __restrict__ ids, int E, int P, int nchunks,
                     const int32_t* __restrict__ chunk_cnt, const int32_t* __restrict__ rank,
                     int32_t* __restrict__ perm) {
  const int nb = E + 1;
  const int c = blockIdx.x;
  for (int r = 0; r < kChunkRounds; ++r) {
    const int p = c * kChunkPairs + r * kRoundThreads + threadIdx.x;
    if (p >= P) return;
    const int bin = bin_of(ids[p], E);
    const int pos = chunk_cnt[(long long)nchunks * nb + bin] + chunk_cnt[(long long)c * nb + bin] + rank[p];
    perm[pos] = p;
  }
}

}  // namespace

size_t route_scratch_bytes(int E, int P) {
  const int nb = E + 1;
  const int nchunks = (P + kChunkPairs - 1) / kChunkPairs;
  return align_up((size_t)(nchunks + 1) * nb * sizeof(int32_t)) + align_up((size_t)P * sizeof(int32_t));
}

hipError_t launch_route(int E, int T, int top_k, const int32_t* ids, const RouteOut& o, hipStream_t s) {
  const int P = T * top_k;
  const int nb = E + 1;
  if (P <= kFastThreads && E <= 256) {
    size_t lds = (size_t)2 * nb * kFastWords * 4 + (size_t)2 * nb * 4 + 16 * 4;
    hipLaunchKernelGGL(route_fast_kernel, dim3(1), dim3(kFastThreads), lds, s, ids, E, P, o.offsets, o.perm,
                       o.active, o.meta, o.tiles, o.counters, o.max_tiles, o.tile_rows, o.wide);
    return hipGetLastError();
  }
  if (P <= kSmallMaxPairs) {
    size_t lds = (size_t)nb * kMaskWords * 4 + (size_t)3 * nb * 4 + (size_t)kSmallMaxPairs * 4 +
                 kRoundThreads * 4;
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(kRoundThreads), lds, s, ids, E, P,
                       o.offsets, o.perm, o.active, o.meta, o.tiles, o.counters, o.max_tiles, o.tile_rows, o.wide);
    return hipGetLastError();
  }
  const int nchunks = (P + kChunkPairs - 1) / kChunkPairs;
  size_t lds1 = (size_t)nb * kMaskWords * 4 + (size_t)nb * 4;
  hipLaunchKernelGGL(route_chunk_kernel, dim3(nchunks), dim3(kRoundThreads), lds1, s, ids, E, P,
                     o.chunk_cnt, o.rank);
  size_t lds2 = (size_t)2 * nb * 4 + 1024 * 4;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), lds2, s, E, P, nchunks, o.chunk_cnt,
                     o.offsets, o.active, o.meta, o.tiles, o.counters, o.max_tiles, o.tile_rows, o.wide);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(kRoundThreads), 0, s, ids, E, P,
                     nchunks, o.chunk_cnt, o.rank, o.perm);
  return hipGetLastError();
}

// Slot forward: each pair's expert id becomes its slot index through the device map; a pair
// whose expert sits in no slot (a miss) or whose id is outside [0, E) gets -1, which every
// forward path treats as a pair that contributes nothing. One workgroup, so the miss count has a
// single writer and needs no clearing beforehand (the call can be captured in a graph).
// Source: the README paragraph on the base cache (a missing expert's contribution is zeroed and
// an in-graph miss counter bumped).
namespace {
constexpr int kSlotThreads = 1024;
__global__ void __launch_bounds__(kSlotThreads)
slot_ids_kernel(int P, int E, int S, const int32_t* __restrict__ ids, const int32_t* __restrict__ slot_of_expert,
                int32_t* __restrict__ slot_ids, long long* __restrict__ counters) {
  __shared__ int part[kSlotThreads / 64];
  int miss = 0;
  for (int p = threadIdx.x; p < P; p += kSlotThreads) {
    const int id = ids[p];
    int sl = -1;
    if (id >= 0 && id < E) {
      sl = slot_of_expert[id];
      if (sl < 0 || sl >= S) { sl = -1; ++miss; }
    }
    slot_ids[p] = sl;
  }
  // wave sums, then one thread writes the total
  for (int off = 32; off > 0; off >>= 1) miss += __shfl_down(miss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = miss;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long total = 0;
    for (int i = 0; i < kSlotThreads / 64; ++i) total += part[i];
    counters[2] = total;
  }
}
}  // namespace

hipError_t launch_slot_ids(int P, int E, int S, const int32_t* ids, const int32_t* slot_of_expert,
                           int32_t* slot_ids, long long* counters, hipStream_t s) {
  hipLaunchKernelGGL(slot_ids_kernel, dim3(1), dim3(kSlotThreads), 0, s, P, E, S, ids, slot_of_expert, slot_ids,
                     counters);
  return hipGetLastError();
}

}  // namespace moew2
