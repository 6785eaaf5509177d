// Device-side building blocks shared by the kernels of libmoew2 (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

#define MOEW2_DEV __device__ __forceinline__

// ------------------------------------------------------------------------------------------
// Native plane layout (built by moe_w2_pack):
//   A weight matrix of NR rows (output features) and reduction length KR is stored as tiles of
//   16 rows x 256 reduction elements; tile (rg, kt) holds 1024 code bytes at
//   (rg * (KR/256) + kt) * 1024. Lane l (0..63) of a wave owns row 16*rg + l%16 and the
//   8-element group g = l/16 of every 32-element block; its 16 bytes sit at tile + 16*l, so one
//   16-byte load per lane is one fully coalesced 1 KiB wave load.
//   Dword j (0..3) of a lane covers blocks b = 2j and 2j+1 of the tile, elements
//   k = 256*kt + 32*b + 8*g + i (i = 0..7), as bit pairs: bit 4i+3 = sign (block 2j, i),
//   bit 4i+2 = |value|==4 (block 2j, i), bit 4i+1 = sign (block 2j+1, i), bit 4i+0 = |value|==4
//   (block 2j+1, i). So (dw & 0xCCCCCCCC) | 0x22222222 is eight e2m1 codes (+-1 = 0b?010,
//   +-4 = 0b?110) of block 2j and ((dw << 2) & 0xCCCCCCCC) | 0x22222222 those of block 2j+1; byte
//   q of such a word holds elements 2q (low nibble) and 2q+1, which is exactly the 8-element B
//   operand of v_mfma_f32_16x16x32 for lane l (column l%16, k = 8*(l/16) .. +7).
//   Scale tile (rg, kt): 128 bytes at (rg * (KR/256) + kt) * 128, row-major [16 rows][8 blocks].
//   Gate_up matrices interleave rows in groups of 16: row group 2q = gate rows 16q..16q+15,
//   row group 2q+1 = up rows 16q..16q+15. Down scale bytes are stored minus a per-row offset E0
//   (kept separately) so that every down weight is exact in fp16.
// ------------------------------------------------------------------------------------------
constexpr int kTileRows = 16;
constexpr int kTileK = 256;
constexpr int kTileCodeBytes = 1024;
constexpr int kTileScaleBytes = 128;

// Two e2m1 words (8 codes each, blocks 2j and 2j+1) from one native dword.
MOEW2_DEV void native_to_fp4(uint32_t dw, uint32_t& blk0, uint32_t& blk1) {
  blk0 = (dw & 0xCCCCCCCCu) | 0x22222222u;
  blk1 = ((dw << 2) & 0xCCCCCCCCu) | 0x22222222u;
}

// A float whose exponent field is byte D of `sw`. The MX conversion instructions scale by
// 2^(exponent field - 127) and ignore the sign and mantissa of their scale operand, so this is
// the UE8M0 scale 2^(b-127) for every byte b in 0..254 with one shift.
template <int D>
MOEW2_DEV float ue8m0_scale_operand(uint32_t sw) {
  uint32_t v = D == 0 ? (sw << 23) : D == 1 ? (sw << 15) : D == 2 ? (sw << 7) : (sw >> 1);
  return __builtin_bit_cast(float, v);
}

MOEW2_DEV bf16x8_t fp4x8_to_bf16(uint32_t f, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

MOEW2_DEV f16x8_t fp4x8_to_f16(uint32_t f, float scale) {
  f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(f, scale, 0);
  f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(f, scale, 1);
  f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(f, scale, 2);
  f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(f, scale, 3);
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Element type traits: gate_up runs in bf16, down in fp16.
struct Bf16Op {
  typedef bf16x8_t vec;
  MOEW2_DEV static vec dequant(uint32_t fp4, float scale) { return fp4x8_to_bf16(fp4, scale); }
  MOEW2_DEV static f32x4_t mfma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
struct F16Op {
  typedef f16x8_t vec;
  MOEW2_DEV static vec dequant(uint32_t fp4, float scale) { return fp4x8_to_f16(fp4, scale); }
  MOEW2_DEV static f32x4_t mfma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_16x16x32 operand layout (checked on the device): A lane l holds row l%16,
// k = 8*(l/16) .. +7; B lane l holds column l%16, the same k; accumulator register r (0..3) of
// lane l holds row 4*(l/16) + r, column l%16.

MOEW2_DEV float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// 16-byte global load / store helpers
MOEW2_DEV u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
MOEW2_DEV u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }

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
