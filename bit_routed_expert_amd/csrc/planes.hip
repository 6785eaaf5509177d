// moe_w2_pack / moe_w2_unpack kernels: canonical 2-bit planes <-> native tiled planes.
// Planes are built once when the layer's weights are processed after loading ("The v0.24.0
// port", section "Our hooks"); the native layout is described in common.h.
#include "common.h"
#include "internal.h"

namespace moew2 {
namespace {

// Canonical row of native row `nr` in a matrix. Gate_up matrices interleave gate and up rows in
// groups of 16; down matrices keep the canonical order.
__device__ __forceinline__ int canonical_row(int nr, int I, bool gate_up) {
  if (!gate_up) return nr;
  int rg = nr >> 4, j = nr & 15;
  int q = rg >> 1;
  return (rg & 1) ? I + 16 * q + j : 16 * q + j;
}

// Row k of value slot 0 of dword j, sub-slot s, for lane group g in k-tile kt (the two tile
// layouts of the planes; gate_up matrices use the block layout, down matrices the k-group one).
__device__ __forceinline__ int slot_k0(int kt, int j, int s, int g, bool block_layout) {
  return kt * kTileK + (block_layout ? 32 * ((j >> 1) * 4 + g) + 16 * (j & 1) + 8 * s
                                     : 32 * (2 * j + s) + 8 * g);
}

// code c (0..3, value {-4,-1,1,4}[c]) -> (sign, |value|==4) bit pair
__device__ __forceinline__ uint32_t code_sign(uint32_t c) { return (c >> 1) ^ 1u; }
__device__ __forceinline__ uint32_t code_mag4(uint32_t c) { return ((c >> 1) ^ (c & 1u)) ^ 1u; }

// One thread per (matrix, tile, lane): writes the lane's 8 native dwords.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                  int nmat, int NR, int KR, int I, int gate_up) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const long long total = (long long)nmat * nrg * nkt * 64;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  long long t = gid >> 6;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int nr = rg * kTileRows + (lane & 15), g = lane >> 4;
  const int cr = canonical_row(nr, I, gate_up != 0);
  const uint8_t* row = canon + ((long long)e * NR + cr) * (KR / 4);
  uint32_t dw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k0 = slot_k0(kt, j, s, g, gate_up != 0);  // multiple of 8
      const uint32_t bits = (uint32_t)row[k0 / 4] | ((uint32_t)row[k0 / 4 + 1] << 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = (bits >> (2 * i)) & 3u;
        v |= code_sign(c) << (4 * i + 3 - 2 * s);
        v |= code_mag4(c) << (4 * i + 2 - 2 * s);
      }
    }
    dw[j] = v;
  }
  uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileCodeBytes;
  u32x4_t v4 = {dw[0], dw[1], dw[2], dw[3]};
  *reinterpret_cast<u32x4_t*>(tile + 16 * lane) = v4;
}

__global__ void unpack_codes_kernel(const uint8_t* __restrict__ native, uint8_t* __restrict__ canon,
                                    int nmat, int NR, int KR, int I, int gate_up) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const long long total = (long long)nmat * nrg * nkt * 64;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  long long t = gid >> 6;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int nr = rg * kTileRows + (lane & 15), g = lane >> 4;
  const int cr = canonical_row(nr, I, gate_up != 0);
  const uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileCodeBytes;
  u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(tile + 16 * lane);
  uint32_t dw[4] = {v4[0], v4[1], v4[2], v4[3]};
  uint8_t* row = canon + ((long long)e * NR + cr) * (KR / 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k0 = slot_k0(kt, j, s, g, gate_up != 0);
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sg = (dw[j] >> (4 * i + 3 - 2 * s)) & 1u;
        const uint32_t m4 = (dw[j] >> (4 * i + 2 - 2 * s)) & 1u;
        const uint32_t c = sg ? (m4 ? 0u : 1u) : (m4 ? 3u : 2u);
        bits |= c << (2 * i);
      }
      row[k0 / 4] = (uint8_t)(bits & 0xff);
      row[k0 / 4 + 1] = (uint8_t)(bits >> 8);
    }
  }
}

// Down rows: per-row offset E0 so that every weight of the row is exact in fp16.
// Native byte nb = b - E0 must lie in [103, 140]: +-1 * 2^(nb-127) >= 2^-24 (smallest fp16
// subnormal) and 4 * 2^(nb-127) <= 2^15.
__global__ void down_offset_kernel(const uint8_t* __restrict__ scales, int32_t* __restrict__ e0,
                                   int nrows, int nblk, int32_t* __restrict__ flag) {
  int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= nrows) return;
  const uint8_t* s = scales + (long long)r * nblk;
  int mn = 255, mx = 0;
  for (int b = 0; b < nblk; ++b) { int v = s[b]; mn = v < mn ? v : mn; mx = v > mx ? v : mx; }
  int off = 0;
  if (mx > 254) atomicOr(flag, kFlagDnScale);
  if (mn < 103 || mx > 140) {
    off = mx - 140;
    if (mn - off < 103) atomicOr(flag, kFlagDnSpan);
  }
  e0[r] = off;
}

// One thread per (matrix, tile, row): 8 scale bytes.
__global__ void pack_scales_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                   const int32_t* __restrict__ e0, int nmat, int NR, int KR, int I,
                                   int gate_up, int32_t* __restrict__ flag) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows, nblk = KR / 32;
  const long long total = (long long)nmat * nrg * nkt * kTileRows;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & (kTileRows - 1));
  long long t = gid >> 4;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int nr = rg * kTileRows + j;
  const int cr = canonical_row(nr, I, gate_up != 0);
  const uint8_t* src = canon + ((long long)e * NR + cr) * nblk + kt * 8;
  const int off = gate_up ? 0 : e0[(long long)e * NR + cr];
  uint8_t out[8];
  int bad = 0;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    int b = src[d];
    if (gate_up && b > 252) bad = 1;
    out[d] = (uint8_t)(b - off);
  }
  if (bad) atomicOr(flag, kFlagGuScale);
  uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileScaleBytes;
  if (gate_up) {
    // block layout: byte 2*(16g + j) + c holds block 4c + g
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint16_t*>(tile + 2 * (16 * g + j)) = (uint16_t)(out[g] | (out[4 + g] << 8));
  } else {
    u32x2_t v = {(uint32_t)out[0] | ((uint32_t)out[1] << 8) | ((uint32_t)out[2] << 16) | ((uint32_t)out[3] << 24),
                 (uint32_t)out[4] | ((uint32_t)out[5] << 8) | ((uint32_t)out[6] << 16) | ((uint32_t)out[7] << 24)};
    *reinterpret_cast<u32x2_t*>(tile + 8 * j) = v;
  }
}

__global__ void unpack_scales_kernel(const uint8_t* __restrict__ native, uint8_t* __restrict__ canon,
                                     const int32_t* __restrict__ e0, int nmat, int NR, int KR, int I,
                                     int gate_up) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows, nblk = KR / 32;
  const long long total = (long long)nmat * nrg * nkt * kTileRows;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & (kTileRows - 1));
  long long t = gid >> 4;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int nr = rg * kTileRows + j;
  const int cr = canonical_row(nr, I, gate_up != 0);
  const int off = gate_up ? 0 : e0[(long long)e * NR + cr];
  const uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileScaleBytes;
  uint8_t* dst = canon + ((long long)e * NR + cr) * nblk + kt * 8;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int at = gate_up ? 2 * (16 * (d & 3) + j) + (d >> 2) : 8 * j + d;
    dst[d] = (uint8_t)(tile[at] + off);
  }
}

inline unsigned grid_for(long long n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

hipError_t launch_pack(const moe_w2_planes* p, const uint8_t* gu_codes, const uint8_t* gu_scales,
                       const uint8_t* dn_codes, const uint8_t* dn_scales, hipStream_t s) {
  const int E = p->E, K = p->K, I = p->I;
  const int B = 256;
  hipError_t err = hipMemsetAsync(p->flag, 0, sizeof(int32_t), s);
  if (err != hipSuccess) return err;
  long long n_dn_rows = (long long)E * K;
  hipLaunchKernelGGL(down_offset_kernel, dim3(grid_for(n_dn_rows, B)), dim3(B), 0, s,
                     dn_scales, p->dn_e0, (int)n_dn_rows, I / 32, p->flag);
  long long n1 = (long long)E * (2 * I / kTileRows) * (K / 256) * 64;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(n1, B)), dim3(B), 0, s,
                     gu_codes, p->gu_codes, E, 2 * I, K, I, 1);
  long long n2 = (long long)E * (K / kTileRows) * (I / 256) * 64;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(n2, B)), dim3(B), 0, s,
                     dn_codes, p->dn_codes, E, K, I, I, 0);
  long long n3 = (long long)E * (2 * I / kTileRows) * (K / 256) * kTileRows;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(n3, B)), dim3(B), 0, s,
                     gu_scales, p->gu_scales, p->dn_e0, E, 2 * I, K, I, 1, p->flag);
  long long n4 = (long long)E * (K / kTileRows) * (I / 256) * kTileRows;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(n4, B)), dim3(B), 0, s,
                     dn_scales, p->dn_scales, p->dn_e0, E, K, I, I, 0, p->flag);
  return hipGetLastError();
}

hipError_t launch_unpack(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales,
                         uint8_t* dn_codes, uint8_t* dn_scales, hipStream_t s) {
  const int E = p->E, K = p->K, I = p->I;
  const int B = 256;
  long long n1 = (long long)E * (2 * I / kTileRows) * (K / 256) * 64;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(n1, B)), dim3(B), 0, s,
                     p->gu_codes, gu_codes, E, 2 * I, K, I, 1);
  long long n2 = (long long)E * (K / kTileRows) * (I / 256) * 64;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(n2, B)), dim3(B), 0, s,
                     p->dn_codes, dn_codes, E, K, I, I, 0);
  long long n3 = (long long)E * (2 * I / kTileRows) * (K / 256) * kTileRows;
  hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(n3, B)), dim3(B), 0, s,
                     p->gu_scales, gu_scales, p->dn_e0, E, 2 * I, K, I, 1);
  long long n4 = (long long)E * (K / kTileRows) * (I / 256) * kTileRows;
  hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(n4, B)), dim3(B), 0, s,
                     p->dn_scales, dn_scales, p->dn_e0, E, K, I, I, 0);
  return hipGetLastError();
}

}  // namespace moew2
