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

// Row k of value slot 0 of dword j, sub-slot s, for lane group g in k-tile kt (block layout).
__device__ __forceinline__ int slot_k0(int kt, int j, int s, int g) {
  return kt * kTileK + 32 * ((j >> 1) * 4 + g) + 16 * (j & 1) + 8 * s;
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
      const int k0 = slot_k0(kt, j, s, g);  // multiple of 8
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
      const int k0 = slot_k0(kt, j, s, g);
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

// FP4 codes (canonical: two e2m1 codes per byte, low nibble = even element): one thread per
// (matrix, tile, instruction c, lane); the lane's 16 operand bytes are the 32 codes of block
// 8kt + 4c + g of its row, i.e. 16 consecutive canonical bytes (W4 tile layout in common.h).
__global__ void pack_codes4_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                   int nmat, int NR, int KR, int I, int gate_up, int unpack) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const long long total = (long long)nmat * nrg * nkt * 128;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63), c = (int)((gid >> 6) & 1);
  long long t = gid >> 7;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int cr = canonical_row(rg * kTileRows + (lane & 15), I, gate_up != 0);
  uint8_t* row = const_cast<uint8_t*>(canon) + ((long long)e * NR + cr) * (KR / 2) + 16 * (8 * kt + 4 * c + (lane >> 4));
  uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileCodeBytesW4 + 1024 * c + 16 * lane;
  if (unpack)
    *reinterpret_cast<u32x4_t*>(row) = *reinterpret_cast<const u32x4_t*>(tile);
  else
    *reinterpret_cast<u32x4_t*>(tile) = *reinterpret_cast<const u32x4_t*>(row);
}

// One thread per (matrix, tile, row): the row's 8 scale bytes of the k-tile. Byte 2*(16g + j) + c
// of the tile holds block 4c + g of row j (block layout). A byte above 252 is flagged: its
// weights (up to 4 * 2^(b-127)) would not be finite in fp32.
__global__ void pack_scales_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                   int nmat, int NR, int KR, int I, int gate_up, int32_t* __restrict__ flag) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows, nblk = KR / 32;
  const long long total = (long long)nmat * nrg * nkt * kTileRows;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & (kTileRows - 1));
  long long t = gid >> 4;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int cr = canonical_row(rg * kTileRows + j, I, gate_up != 0);
  const uint8_t* src = canon + ((long long)e * NR + cr) * nblk + kt * 8;
  uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileScaleBytes;
  int bad = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int b0 = src[g], b1 = src[4 + g];
    bad |= (b0 > 252) | (b1 > 252);
    *reinterpret_cast<uint16_t*>(tile + 2 * (16 * g + j)) = (uint16_t)(b0 | (b1 << 8));
  }
  if (bad) atomicOr(flag, kFlagScale);
}

__global__ void unpack_scales_kernel(const uint8_t* __restrict__ native, uint8_t* __restrict__ canon,
                                     int nmat, int NR, int KR, int I, int gate_up) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows, nblk = KR / 32;
  const long long total = (long long)nmat * nrg * nkt * kTileRows;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & (kTileRows - 1));
  long long t = gid >> 4;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int cr = canonical_row(rg * kTileRows + j, I, gate_up != 0);
  const uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileScaleBytes;
  uint8_t* dst = canon + ((long long)e * NR + cr) * nblk + kt * 8;
#pragma unroll
  for (int d = 0; d < 8; ++d) dst[d] = tile[2 * (16 * (d & 3) + j) + (d >> 2)];
}

// NVFP4 codes (canonical: two e2m1 codes per byte, low nibble = even element; NV4 tile layout in
// common.h): one thread per (matrix, tile, half c, lane); dword j of the lane's 16 bytes holds the
// 8 codes of values 128c + 32j + 8g .. + 7 of its row, i.e. 4 consecutive canonical bytes.
__global__ void pack_codes_nv4_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                      int nmat, int NR, int KR, int I, int gate_up, int unpack) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows;
  const long long total = (long long)nmat * nrg * nkt * 128;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63), c = (int)((gid >> 6) & 1);
  long long t = gid >> 7;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int cr = canonical_row(rg * kTileRows + (lane & 15), I, gate_up != 0);
  uint8_t* row = const_cast<uint8_t*>(canon) + ((long long)e * NR + cr) * (KR / 2) + 128 * kt + 64 * c + 4 * (lane >> 4);
  uint32_t* tile = reinterpret_cast<uint32_t*>(native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) *
                                               kTileCodeBytesW4 + 1024 * c + 16 * lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t* src = reinterpret_cast<uint32_t*>(row + 16 * j);
    if (unpack) *src = tile[j];
    else tile[j] = *src;
  }
}

// NVFP4 scales (canonical: one E4M3FN byte per 16 values along the reduction axis): one thread
// per (matrix, tile, 16-block parity h, row n); byte 128h + 8n + 4c + j of the tile is the scale
// of 16-block 16kt + 8c + 2j + h of row n. A NaN encoding (0x7F, 0xFF) is flagged.
__global__ void pack_scales_nv4_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ native,
                                       int nmat, int NR, int KR, int I, int gate_up, int32_t* __restrict__ flag,
                                       int unpack) {
  const int nkt = KR / kTileK, nrg = NR / kTileRows, nsc = KR / 16;
  const long long total = (long long)nmat * nrg * nkt * 32;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int n = (int)(gid & 15), h = (int)((gid >> 4) & 1);
  long long t = gid >> 5;
  const int kt = (int)(t % nkt); t /= nkt;
  const int rg = (int)(t % nrg);
  const int e = (int)(t / nrg);
  const int cr = canonical_row(rg * kTileRows + n, I, gate_up != 0);
  uint8_t* row = const_cast<uint8_t*>(canon) + ((long long)e * NR + cr) * nsc + 16 * kt + h;
  uint8_t* tile = native + ((long long)e * nrg * nkt + (long long)rg * nkt + kt) * kTileScaleBytesNV4 + 128 * h + 8 * n;
  int bad = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (unpack) {
        row[8 * c + 2 * j] = tile[4 * c + j];
      } else {
        const uint8_t b = row[8 * c + 2 * j];
        bad |= (b & 0x7F) == 0x7F;
        tile[4 * c + j] = b;
      }
    }
  if (bad) atomicOr(flag, kFlagNaN);
}

// scale_2 of experts [e0, e0 + n): gate and up from gu [n][2], down from dn [n], into planes [E][3]
// (or back, with unpack); a non-finite value is flagged.
__global__ void copy_scale2_kernel(const float* __restrict__ gu, const float* __restrict__ dn, float* __restrict__ planes,
                                   int n, int32_t* __restrict__ flag, int unpack) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (unpack) {
    const_cast<float*>(gu)[2 * i] = planes[3 * i];
    const_cast<float*>(gu)[2 * i + 1] = planes[3 * i + 1];
    const_cast<float*>(dn)[i] = planes[3 * i + 2];
    return;
  }
  const float a = gu[2 * i], b = gu[2 * i + 1], c = dn[i];
  planes[3 * i] = a;
  planes[3 * i + 1] = b;
  planes[3 * i + 2] = c;
  if (!__builtin_isfinite(a) || !__builtin_isfinite(b) || !__builtin_isfinite(c)) atomicOr(flag, kFlagNaN);
}

inline unsigned grid_for(long long n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

// Packs experts [e0, e0 + n) of the planes from canonical planes holding those n experts.
hipError_t launch_pack_experts(const moe_w2_planes* p, int e0, int n, const uint8_t* gu_codes,
                               const uint8_t* gu_scales, const uint8_t* dn_codes, const uint8_t* dn_scales,
                               hipStream_t s) {
  const int K = p->K, I = p->I;
  const int B = 256;
  const size_t gu = (size_t)2 * I * K, dn = (size_t)K * I;   // weights per expert
  const int cb = code_bits(p->fmt);                           // code bits per weight
  hipError_t err = hipMemsetAsync(p->flag, 0, sizeof(int32_t), s);
  if (err != hipSuccess) return err;
  long long n1 = (long long)n * (2 * I / kTileRows) * (K / 256) * 64;
  long long n2 = (long long)n * (K / kTileRows) * (I / 256) * 64;
  uint8_t* guc = p->gu_codes + (size_t)e0 * gu * cb / 8;
  uint8_t* dnc = p->dn_codes + (size_t)e0 * dn * cb / 8;
  if (p->fmt == kFmtW4) {
    hipLaunchKernelGGL(pack_codes4_kernel, dim3(grid_for(2 * n1, B)), dim3(B), 0, s, gu_codes, guc, n, 2 * I, K, I, 1, 0);
    hipLaunchKernelGGL(pack_codes4_kernel, dim3(grid_for(2 * n2, B)), dim3(B), 0, s, dn_codes, dnc, n, K, I, I, 0, 0);
  } else {
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(n1, B)), dim3(B), 0, s, gu_codes, guc, n, 2 * I, K, I, 1);
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(n2, B)), dim3(B), 0, s, dn_codes, dnc, n, K, I, I, 0);
  }
  long long n3 = (long long)n * (2 * I / kTileRows) * (K / 256) * kTileRows;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(n3, B)), dim3(B), 0, s,
                     gu_scales, p->gu_scales + (size_t)e0 * gu / 32, n, 2 * I, K, I, 1, p->flag);
  long long n4 = (long long)n * (K / kTileRows) * (I / 256) * kTileRows;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(n4, B)), dim3(B), 0, s,
                     dn_scales, p->dn_scales + (size_t)e0 * dn / 32, n, K, I, I, 0, p->flag);
  return hipGetLastError();
}

hipError_t launch_pack(const moe_w2_planes* p, const uint8_t* gu_codes, const uint8_t* gu_scales,
                       const uint8_t* dn_codes, const uint8_t* dn_scales, hipStream_t s) {
  return launch_pack_experts(p, 0, p->E, gu_codes, gu_scales, dn_codes, dn_scales, s);
}

// NVFP4 planes, both directions (unpack = native -> canonical; the flag is cleared and set on
// packing only).
hipError_t launch_pack_nv4(const moe_w2_planes* p, const uint8_t* gu_codes, const uint8_t* gu_scales,
                           const float* gu_scale2, const uint8_t* dn_codes, const uint8_t* dn_scales,
                           const float* dn_scale2, int unpack, hipStream_t s) {
  const int E = p->E, K = p->K, I = p->I;
  const int B = 256;
  if (!unpack) {
    hipError_t err = hipMemsetAsync(p->flag, 0, sizeof(int32_t), s);
    if (err != hipSuccess) return err;
  }
  const long long t_gu = (long long)E * (2 * I / kTileRows) * (K / kTileK);
  const long long t_dn = (long long)E * (K / kTileRows) * (I / kTileK);
  hipLaunchKernelGGL(pack_codes_nv4_kernel, dim3(grid_for(t_gu * 128, B)), dim3(B), 0, s, gu_codes, p->gu_codes, E,
                     2 * I, K, I, 1, unpack);
  hipLaunchKernelGGL(pack_codes_nv4_kernel, dim3(grid_for(t_dn * 128, B)), dim3(B), 0, s, dn_codes, p->dn_codes, E, K,
                     I, I, 0, unpack);
  hipLaunchKernelGGL(pack_scales_nv4_kernel, dim3(grid_for(t_gu * 32, B)), dim3(B), 0, s, gu_scales, p->gu_scales, E,
                     2 * I, K, I, 1, p->flag, unpack);
  hipLaunchKernelGGL(pack_scales_nv4_kernel, dim3(grid_for(t_dn * 32, B)), dim3(B), 0, s, dn_scales, p->dn_scales, E,
                     K, I, I, 0, p->flag, unpack);
  hipLaunchKernelGGL(copy_scale2_kernel, dim3(grid_for(E, B)), dim3(B), 0, s, gu_scale2, dn_scale2, p->scale2, E,
                     p->flag, unpack);
  return hipGetLastError();
}

hipError_t launch_unpack(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales,
                         uint8_t* dn_codes, uint8_t* dn_scales, hipStream_t s) {
  const int E = p->E, K = p->K, I = p->I;
  const int B = 256;
  long long n1 = (long long)E * (2 * I / kTileRows) * (K / 256) * 64;
  long long n2 = (long long)E * (K / kTileRows) * (I / 256) * 64;
  if (p->fmt == kFmtW4) {
    hipLaunchKernelGGL(pack_codes4_kernel, dim3(grid_for(2 * n1, B)), dim3(B), 0, s, gu_codes, p->gu_codes, E, 2 * I,
                       K, I, 1, 1);
    hipLaunchKernelGGL(pack_codes4_kernel, dim3(grid_for(2 * n2, B)), dim3(B), 0, s, dn_codes, p->dn_codes, E, K, I,
                       I, 0, 1);
  } else {
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(n1, B)), dim3(B), 0, s, p->gu_codes, gu_codes, E, 2 * I, K,
                       I, 1);
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(n2, B)), dim3(B), 0, s, p->dn_codes, dn_codes, E, K, I, I,
                       0);
  }
  long long n3 = (long long)E * (2 * I / kTileRows) * (K / 256) * kTileRows;
  hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(n3, B)), dim3(B), 0, s,
                     p->gu_scales, gu_scales, E, 2 * I, K, I, 1);
  long long n4 = (long long)E * (K / kTileRows) * (I / 256) * kTileRows;
  hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(n4, B)), dim3(B), 0, s,
                     p->dn_scales, dn_scales, E, K, I, I, 0);
  return hipGetLastError();
}

}  // namespace moew2
