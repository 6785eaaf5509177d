// Device-side building blocks shared by the kernels of libmoew2 (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

#define MOEW2_DEV __device__ __forceinline__

// ------------------------------------------------------------------------------------------
// Native plane layout (built by moe_w2_pack), in the operand order of the block-scaled matrix
// instruction described below:
//   A weight matrix of NR rows (output features) and reduction length KR is stored as tiles of
//   16 rows x 256 reduction elements; tile (rg, kt) holds 1024 code bytes at
//   (rg * (KR/256) + kt) * 1024 and 128 scale bytes at (rg * (KR/256) + kt) * 128. Lane l
//   (0..63) of a wave owns row 16*rg + l%16 and reads the 16 code bytes at tile + 16*l, so one
//   16-byte load per lane is one fully coalesced 1 KiB wave load. With g = l/16, the lane's dwords
//   0,1 hold block 8kt + g of its row and dwords 2,3 block 8kt + 4 + g; dword j holds values
//   16*(j%2) .. 16*(j%2) + 15 of its block as bit pairs: value 8s + i (i = 0..7, s = 0, 1) has its
//   sign at bit 4i+3-2s and |value|==4 at bit 4i+2-2s. So (dw & 0xCCCCCCCC) | 0x22222222 is the
//   eight e2m1 codes (+-1 = 0b?010, +-4 = 0b?110) of values 0..7 of the dword and
//   ((dw << 2) & 0xCCCCCCCC) | 0x22222222 those of values 8..15, value i in nibble i.
//   Scale byte 2*l + c of a tile = UE8M0 byte of block 8kt + 4c + g of row l%16.
//   Gate_up matrices interleave rows in groups of 16: row group 2q = gate rows 16q..16q+15,
//   row group 2q+1 = up rows 16q..16q+15.
// ------------------------------------------------------------------------------------------
constexpr int kTileRows = 16;
constexpr int kTileK = 256;
constexpr int kTileCodeBytes = 1024;
constexpr int kTileScaleBytes = 128;

// FP4 planes (e2m1 codes with UE8M0 block-32 scales, the instruction's own B format) use the same
// tiles with 2048 code bytes: instruction c's operands at bytes [1024c, 1024c + 1024), lane l's
// 16 bytes at 1024c + 16l holding the 32 e2m1 values of block 8kt + 4c + l/16 of row l%16 in
// order (value i in nibble i, low nibble first) - one fully coalesced 1 KiB wave load per
// instruction. Scale tiles are the 2-bit planes' (byte 2l + c).
constexpr int kTileCodeBytesW4 = 2048;

// NVFP4 planes (e2m1 codes, one E4M3FN scale per 16 values along the reduction axis and one fp32
// scale_2 per tensor: W = e2m1 x e4m3 x scale_2) feed the 16 x 16 x 32 bf16 / fp16 matrix
// instructions, with W's e2m1 x e4m3 part formed exactly in registers (at most 2 + 4 significant
// bits) and scale_2 applied to the fp32 result. Tiles of 16 rows x 256 values hold 2048 code
// bytes: half c (values 128c .. 128c + 127 of the tile) at [1024c, 1024c + 1024), lane l's 16
// bytes at 1024c + 16l; with n = l % 16 (row) and g = l / 16, dword j of them holds values
// 128c + 32j + 8g .. + 7 of row n (value i in nibble i, low nibble first): the B operand of
// instruction j of half c, whose 32 reduction values are exactly one 32-block. Scale tiles are
// 256 bytes: byte 128h + 8n + 4c + j is the e4m3 scale of 16-block 16kt + 8c + 2j + h of row n,
// so lane l reads its two scale words (c = 0, 1; byte j = instruction j) at 128 (g / 2) + 8n.
constexpr int kTileScaleBytesNV4 = 256;

template <int FMT>
struct WFmt {
  static constexpr int kCodeBytes = FMT ? kTileCodeBytesW4 : kTileCodeBytes;
  static constexpr int kLoads = FMT ? 2 : 1;   // 16-byte code loads per lane per tile
  static constexpr int kScaleBytes = FMT == 2 ? kTileScaleBytesNV4 : 128;   // per tile
  static constexpr int kScaleWords = FMT == 2 ? 2 : 1;                      // per lane per tile
};

template <int I, int N, class F>
MOEW2_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// Two e2m1 words (values 0..7 and 8..15 of a native dword, 8 codes each).
MOEW2_DEV void native_to_fp4(uint32_t dw, uint32_t& blk0, uint32_t& blk1) {
  blk0 = (dw & 0xCCCCCCCCu) | 0x22222222u;
  blk1 = ((dw << 2) & 0xCCCCCCCCu) | 0x22222222u;
}

// ------------------------------------------------------------------------------------------
// Block-scaled (MX) matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4 with A = fp8 (OCP
// e4m3) and B = fp4 (e2m1); layout checked on the device. With g = l/16, one instruction covers
// 128 k = 4 blocks of 32:
//   B lane l: column l%16, all 32 values of block g in k order (nibble i of the 128-bit operand
//             = value i; low nibble first).
//   A lane l: row l%16; operand bytes 0..15 = k 16g .. 16g+15, bytes 16..31 = k 64+16g .. +15.
//   scales: lane l supplies the E8M0 byte of (row/column l%16, block g), selected from its
//           32-bit scale register by op_sel (0..3).
//   accumulator register r (0..3) of lane l: row 4*(l/16) + r, column l%16.
// The planes use this operand order (layout note above): in k-tile kt, lane l holds blocks
// 8kt + g (instruction 0) and 8kt + 4 + g (instruction 1) of its row.
// ------------------------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4e_t __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0;   // A operand format: OCP e4m3
constexpr int kFmtFp4 = 4;   // B operand format: e2m1

// B operand of one instruction from the lane's two native dwords of a block (values 0..15 and
// 16..31): four e2m1 words.
MOEW2_DEV i32x8_t mx_b_operand(uint32_t d0, uint32_t d1) {
  uint32_t a0, a1, b0, b1;
  native_to_fp4(d0, a0, a1);
  native_to_fp4(d1, b0, b1);
  i32x8_t v = {(int)a0, (int)a1, (int)b0, (int)b1, 0, 0, 0, 0};
  return v;
}

// The same expansion as one bit-field insert per output dword (plus a shift for the second):
// v_bfi_b32 takes the selector mask from a scalar register. Make the masks once per kernel with
// fp4_masks().
struct Fp4Masks {
  uint32_t sel;   // scalar register: 0xCCCCCCCC
  uint32_t one;   // 0x22222222
};
MOEW2_DEV Fp4Masks fp4_masks() {
  Fp4Masks f;
  asm volatile("s_mov_b32 %0, 0xcccccccc" : "=s"(f.sel));
  f.one = 0x22222222u;
  return f;
}
MOEW2_DEV uint32_t bfi_sel(uint32_t sel, uint32_t a, uint32_t b) {   // (a & sel) | (b & ~sel)
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(sel), "v"(a), "v"(b));
  return r;
}
MOEW2_DEV i32x8_t mx_b_operand(uint32_t d0, uint32_t d1, const Fp4Masks& f) {
  const uint32_t a0 = bfi_sel(f.sel, d0, f.one);
  const uint32_t a1 = bfi_sel(f.sel, d0 << 2, f.one);
  const uint32_t b0 = bfi_sel(f.sel, d1, f.one);
  const uint32_t b1 = bfi_sel(f.sel, d1 << 2, f.one);
  i32x8_t v = {(int)a0, (int)a1, (int)b0, (int)b1, 0, 0, 0, 0};
  return v;
}

// B operand of instruction C of a tile from the lane's code registers: the 2-bit codes expand to
// e2m1 (W2), the fp4 codes are the operand (W4).
template <int FMT, int C>
MOEW2_DEV i32x8_t b_operand(const u32x4_t (&cr)[WFmt<FMT>::kLoads], const Fp4Masks& f) {
  if constexpr (FMT == 0) {
    return mx_b_operand(cr[0][2 * C], cr[0][2 * C + 1], f);
  } else {
    const u32x4_t& v = cr[C];
    return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
  }
}

template <int FMT, int C>
MOEW2_DEV i32x8_t b_operand(const u32x4_t (&cr)[WFmt<FMT>::kLoads]) {
  if constexpr (FMT == 0) {
    return mx_b_operand(cr[0][2 * C], cr[0][2 * C + 1]);
  } else {
    const u32x4_t& v = cr[C];
    return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
  }
}

template <int OPA, int OPB>
MOEW2_DEV f32x4_t mx_mfma(const i32x8_t& a, const i32x8_t& b, f32x4_t c, uint32_t sa, uint32_t sb) {
  const f32x4e_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      a, b, __builtin_bit_cast(f32x4e_t, c), kFmtFp8, kFmtFp4, OPA, (int)sa, OPB, (int)sb);
  return __builtin_bit_cast(f32x4_t, r);
}

// x as two e4m3 parts for the A operand. Per 32-element block with |x| <= amax: scale byte
// sx = max(0, exponent field of amax - 7), so |x| / 2^(sx-127) < 256 fits e4m3 (max 448);
// hi = RNE_e4m3(x / 2^(sx-127)); lo = RNE_e4m3(16 * (x / 2^(sx-127) - hi)) with scale byte sx - 4.
// A bf16 value (8 significant bits) is the exact sum of the two parts whenever it is at least
// 2^-11 of the block maximum (hi holds the top 4 bits, the remainder has at most 4); smaller
// values keep an error below 2^-21 of the block maximum. sx < 4 (a block maximum below 2^-116)
// drops the lo part.
MOEW2_DEV uint32_t x_scale_byte(float amax) {
  const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 255u);
  return (uint32_t)(ef > 7 ? ef - 7 : 0);
}
MOEW2_DEV uint32_t x_lo_scale_byte(uint32_t sx) { return sx >= 4 ? sx - 4 : 0; }

// Four values -> four hi bytes and four lo bytes (one dword each), given the block's scale byte.
MOEW2_DEV void x_split4(float v0, float v1, float v2, float v3, uint32_t sx, uint32_t& hi, uint32_t& lo) {
  const int sh = 127 - (int)sx, sl = 131 - (int)sx;
  const float t0 = __builtin_ldexpf(v0, sh), t1 = __builtin_ldexpf(v1, sh);
  const float t2 = __builtin_ldexpf(v2, sh), t3 = __builtin_ldexpf(v3, sh);
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, h, true);
  const float r0 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 0), -16.f, __builtin_ldexpf(v0, sl));
  const float r1 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 1), -16.f, __builtin_ldexpf(v1, sl));
  const float r2 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 2), -16.f, __builtin_ldexpf(v2, sl));
  const float r3 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 3), -16.f, __builtin_ldexpf(v3, sl));
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, l, true);
  hi = (uint32_t)h;
  lo = sx >= 4 ? (uint32_t)l : 0u;
}

// The gated intermediate (fp16, 11 significant bits) as three e4m3 parts with scale bytes sa,
// sa - 4 and sa - 8 (sa = x_scale_byte of the block maximum): p0 = RNE(t), p1 = RNE(16 (t - p0)),
// p2 = RNE(16 (16 (t - p0) - p1)) with t = a / 2^(sa-127). Each remainder has at most 4
// significant bits left, so the three parts are exact for every value at least 2^-10 of the block
// maximum; smaller values keep an error below 2^-24 of the block maximum. sa < 8 drops the parts
// whose scale would go below 0.
MOEW2_DEV void a_split4(float v0, float v1, float v2, float v3, uint32_t sa, uint32_t& p0, uint32_t& p1,
                        uint32_t& p2) {
  const int sh = 127 - (int)sa, sm = 131 - (int)sa;
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v0, sh), __builtin_ldexpf(v1, sh), 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(v2, sh), __builtin_ldexpf(v3, sh), h, true);
  const float r0 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 0), -16.f, __builtin_ldexpf(v0, sm));
  const float r1 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 1), -16.f, __builtin_ldexpf(v1, sm));
  const float r2 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 2), -16.f, __builtin_ldexpf(v2, sm));
  const float r3 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(h, 3), -16.f, __builtin_ldexpf(v3, sm));
  int m = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
  m = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, m, true);
  const float q0 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(m, 0), -16.f, 16.f * r0);
  const float q1 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(m, 1), -16.f, 16.f * r1);
  const float q2 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(m, 2), -16.f, 16.f * r2);
  const float q3 = __builtin_fmaf(__builtin_amdgcn_cvt_f32_fp8(m, 3), -16.f, 16.f * r3);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, l, true);
  p0 = (uint32_t)h;
  p1 = sa >= 4 ? (uint32_t)m : 0u;
  p2 = sa >= 8 ? (uint32_t)l : 0u;
}
// scale word pair of one (row, k-tile, lane group) for the three parts: word 0 = (p0 c0, p0 c1,
// p1 c0, p1 c1), word 1 = (p2 c0, p2 c1, 0, 0); c = chunk (instruction 0 or 1 of the k-tile)
MOEW2_DEV uint32_t a_part_scale(uint32_t sa, int part) {
  const int v = (int)sa - 4 * part;
  return v > 0 ? (uint32_t)v : 0u;
}

// ------------------------------------------------------------------------------------------
// Three-part fp6 (OCP e2m3) expansion of an activation block for the A operand of the same
// instruction with A = fp6: v_mfma_scale_f32_16x16x128_f8f6f4 with A in e2m3 runs at the fp4
// rate, twice the fp8 rate (measured: 9.0 vs 4.7 PFLOP/s on the chip). Lane l of a wave then
// supplies the 32 values of the block that B lane group l/16 holds, value j in bits 6j..6j+5 of
// its six operand dwords, with its own scale byte (layout measured with one-hot probes).
// Per 32-value block with maximum M, scale byte b = max(9, min(254, exponent field of M - 1)),
// so t = v / 2^(b-127) has |t| < 4 (|t| < 2 when clamped at 9). With RNE to the e2m3 grid:
//   p0 = RNE(t), p1 = RNE(16 (t - p0)), p2 = RNE(16 (16 (t - p0) - p1)),
// each residual exact in fp32; parts p use scale bytes b - 4p. |t - p0| <= 1/8, every later
// residual <= 1/16 of its part's unit, so |v - sum| <= 2^-12 * 2^(b-127) <= 2^-13 * M.
// The hardware conversion (v_cvt_scalef32_2xpk16_fp6_f32) rounds v / scale to nearest even
// (checked against a host model over every grid point, every midpoint and random values) and
// interleaves its two 16-value sources: source 0 value i -> field 2i, source 1 value i ->
// field 2i + 1; the reverse conversion returns the fields in order, times the scale.
// ------------------------------------------------------------------------------------------
constexpr int kFmtFp6 = 2;   // A operand format: OCP e2m3
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));

// Split record of one (row, k-tile) of 256 values (8 blocks d = 4c + g, c = instruction of the
// k-tile, g = lane group), 608 bytes:
//   [0, 384)   part p, block d: operand dwords 0..3 at 16 * (8p + d)
//   [384, 576) part p, block d: operand dwords 4..5 at 384 + 8 * (8p + d)
//   [576, 608) block d: scale word at 576 + 4d, bytes (b, b - 4, b - 8, 0)
// A row stride of 608 bytes (152 dwords, 8 mod 16) keeps the lane pattern of an operand read
// (16 rows x 4 consecutive 16-byte pieces) free of LDS bank conflicts.
constexpr int kA6Bytes = 608;
constexpr int kA6Hi = 384;
constexpr int kA6Scale = 576;

MOEW2_DEV uint32_t a6_scale_byte(float amax) {
  const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 255u);
  const int b = ef - 1;
  return (uint32_t)(b < 9 ? 9 : (b > 254 ? 254 : b));
}

// 32 values (natural order) -> three parts of six operand dwords each.
MOEW2_DEV void a6_split(const float (&v)[32], uint32_t b, u32x6_t (&part)[3]) {
  f32x16_t ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) { ev[i] = v[2 * i]; od[i] = v[2 * i + 1]; }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const float sc = __builtin_bit_cast(float, (b - 4u * (uint32_t)p) << 23);
    part[p] = __builtin_bit_cast(u32x6_t, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc));
    if (p < 2) {
      const f32x32_t back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(
          __builtin_bit_cast(__attribute__((ext_vector_type(6))) unsigned, part[p]), sc);
#pragma unroll
      for (int i = 0; i < 16; ++i) { ev[i] -= back[2 * i]; od[i] -= back[2 * i + 1]; }
    }
  }
}

// Writes block d of a split record (see kA6Bytes).
MOEW2_DEV void a6_store(uint8_t* rec, int d, const u32x6_t (&part)[3], uint32_t b) {
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    *reinterpret_cast<u32x4_t*>(rec + 16 * (8 * p + d)) = u32x4_t{part[p][0], part[p][1], part[p][2], part[p][3]};
    *reinterpret_cast<u32x2_t*>(rec + kA6Hi + 8 * (8 * p + d)) = u32x2_t{part[p][4], part[p][5]};
  }
  *reinterpret_cast<uint32_t*>(rec + kA6Scale + 4 * d) = b | ((b - 4u) << 8) | ((b - 8u) << 16);
}

template <int OPA, int OPB>
MOEW2_DEV f32x4_t mx6_mfma(const i32x8_t& a, const i32x8_t& b, f32x4_t c, uint32_t sa, uint32_t sb) {
  const f32x4e_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      a, b, __builtin_bit_cast(f32x4e_t, c), kFmtFp6, kFmtFp4, OPA, (int)sa, OPB, (int)sb);
  return __builtin_bit_cast(f32x4_t, r);
}

// fp16 bits -> float
MOEW2_DEV float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
MOEW2_DEV float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// bf16 bits -> float
MOEW2_DEV float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
MOEW2_DEV float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

MOEW2_DEV float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// 16-byte global load helper
MOEW2_DEV u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Raw buffer view of one expert's weight plane (at most 2^31 - 1 bytes). A load at offset
// kOutOfRange lies past the buffer's size and returns zeros without a memory access: issuing it
// instead of branching around the load keeps every wave's load sequence fixed, so the compiler's
// wait counts stay exact while a ring of tiles is in flight. Weight loads carry the nontemporal
// policy (each byte is read once per call).
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped) buffer, gfx9-family descriptor word 3
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kPolicyNT = 2;               // cache policy bits: nt
MOEW2_DEV __amdgpu_buffer_rsrc_t buffer_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
// voffset (per lane, range-checked) + soffset (wave-uniform byte offset added to the base)
MOEW2_DEV u32x4_t buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kPolicyNT));
}
MOEW2_DEV uint32_t buf_ld2_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, kPolicyNT);
}

// ------------------------------------------------------------------------------------------
// NVFP4 B operands and the 16 x 16 x 32 instructions. Operand layout (both A and B): lane l
// supplies row / column l % 16 and reduction values 8(l/16) .. 8(l/16) + 7 of the instruction;
// accumulator register r of lane l holds row 4(l/16) + r, column l % 16 (as for the block-scaled
// instruction above).
// ------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2e_t __attribute__((ext_vector_type(2)));

// 8 e2m1 codes (value i in nibble i) times e4m3 byte J of `sw`, as 8 bf16 values. Exact: the
// e2m1 value (from the conversion with scale 1) times the e4m3 value is exact in fp32 and has at
// most 6 significant bits, so its bf16 rounding changes nothing.
template <int J>
MOEW2_DEV bf16x8_t nv4_b_bf16(uint32_t codes, uint32_t sw) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)sw, J);
  bf16x8_t r;
  static_for<0, 4>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const f32x2e_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, q);
    r[2 * q] = (__bf16)(f[0] * s);
    r[2 * q + 1] = (__bf16)(f[1] * s);
  });
  return r;
}

// The same as 8 fp16 values: the conversion applies the power-of-two part 2^E of |s| for the
// e4m3 value s (it uses only its scale operand's exponent), a packed fp16 multiply the signed
// mantissa factor f = s / 2^E, |f| in [1, 2) (3 fraction bits at most). Both steps are exact:
// |e2m1 x 2^E| lies in [2^-10, 1536] and the product in [2^-10, 2688], inside fp16's normal
// range, with at most 6 significant bits. 2^E and 2^-E are formed from s's exponent field
// (E in [-9, 8]); a zero scale takes 2^E = 2^-126 and f = 0, which gives zeros.
template <int J>
MOEW2_DEV f16x8_t nv4_b_f16(uint32_t codes, uint32_t sw) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)sw, J);
  const uint32_t eb = __builtin_bit_cast(uint32_t, s) & 0x7F800000u;
  const float p2 = __builtin_bit_cast(float, eb > 0x00800000u ? eb : 0x00800000u);
  const _Float16 m = (_Float16)(s * __builtin_bit_cast(float, 0x7F000000u - eb));
  const f16x2_t mm = {m, m};
  f16x8_t r;
  static_for<0, 4>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, p2, q) * mm;
    r[2 * q] = h[0];
    r[2 * q + 1] = h[1];
  });
  return r;
}

MOEW2_DEV f32x4_t mfma32_bf16(const u32x4_t& a, const bf16x8_t& b, f32x4_t c) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b,
                                                                             __builtin_bit_cast(f32x4e_t, c), 0, 0, 0));
}
MOEW2_DEV f32x4_t mfma32_f16(const u32x4_t& a, const f16x8_t& b, f32x4_t c) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), b,
                                                                            __builtin_bit_cast(f32x4e_t, c), 0, 0, 0));
}

MOEW2_DEV u32x2_t buf_ld8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kPolicyNT));
}

// Round-to-nearest-even fp32 -> bf16 bits (finite and infinite inputs; NaN stays NaN).
MOEW2_DEV uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
