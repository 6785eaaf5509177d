"""Number formats used by the method, written out plainly (test infrastructure; see oracle/__init__).

Sources:
* Codebook: vLLM-Moet README, bullet "2-bit expert planes - the sign-bias finding" (values
  {-4, -1, 1, 4}); code order from the starlog article, section "Technical Insight" (the
  illustrative kernel's LUT comment maps codes 0,1,2,3 to -4,-1,1,4).
* UE8M0 block-32 scales: "The v0.24.0 port" page, section "Our hooks", modelopt.py bullet.
  A UE8M0 byte b encodes 2**(b-127) for b in 0..254; 255 is not a number (OCP MX convention).
* NVFP4 element and scale formats (e2m1 codes, e4m3 block-16 scales): README opening paragraph
  and the same modelopt.py bullet name them; their bit-level definitions (the OCP / NVFP4
  e2m1 and E4M3FN formats) are not printed on the pages.

Canonical packing (a reading, the pages are silent): 4 codes per byte, element k of a row at bits
2*(k%4)..2*(k%4)+1 (LSB first), along the row's reduction axis. FP4 (MXFP4) expert planes: two
e2m1 codes per byte, low nibble = even element, with the same UE8M0 block-32 scales.
"""
from fractions import Fraction

import numpy as np

# code c -> value; c and 3-c are negatives of each other.
CODEBOOK = (-4.0, -1.0, 1.0, 4.0)

# e2m1 nibble -> value. Bit 3 is the sign; nibble 8 is -0.0.
E2M1_MAGNITUDE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(nibble):
    """Value of one e2m1 nibble as a Python float (exact). Nibble 8 gives -0.0."""
    nibble = int(nibble)
    if not 0 <= nibble < 16:
        raise ValueError("e2m1 nibble out of range")
    mag = E2M1_MAGNITUDE[nibble & 7]
    return -mag if nibble & 8 else mag


def e4m3_value(byte):
    """Value of one E4M3FN byte as a Python float (exact). Raises on the NaN encodings.

    E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities; exponent
    field 0 is subnormal ((m/8) * 2**-6); S.1111.111 is NaN.
    """
    byte = int(byte)
    if not 0 <= byte < 256:
        raise ValueError("e4m3 byte out of range")
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 0xF and m == 7:
        raise ValueError("e4m3 NaN")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_fraction(byte):
    """Exact rational value of an E4M3FN byte (sign carried separately by the caller)."""
    v = e4m3_value(byte)
    return Fraction(v)


def ue8m0_value(byte):
    """2**(byte-127) for byte in 0..254 (UE8M0). Raises on 255."""
    byte = int(byte)
    if not 0 <= byte <= 254:
        raise ValueError("UE8M0 byte 255 is not a number")
    return 2.0 ** (byte - 127)


def unpack_codes(packed):
    """Canonical packed codes [..., n/4] uint8 -> codes [..., n] uint8 in 0..3 (LSB first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    shifts = np.array([0, 2, 4, 6], dtype=np.uint8)
    codes = (packed[..., None] >> shifts) & np.uint8(3)
    return codes.reshape(packed.shape[:-1] + (packed.shape[-1] * 4,))


def pack_codes(codes):
    """codes [..., n] (values 0..3, n % 4 == 0) -> canonical packed bytes [..., n/4]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 4:
        raise ValueError("last axis must be a multiple of 4")
    if codes.size and codes.max() > 3:
        raise ValueError("codes must be in 0..3")
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 4, 4))
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def unpack_e2m1(packed):
    """Canonical FP4 bytes [..., n/2] -> e2m1 nibbles [..., n]: element 2i in the low nibble of
    byte i, element 2i+1 in the high nibble (the NVFP4 packing named for the re-quantizer input,
    used for the FP4 expert planes too)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & np.uint8(15)
    out[..., 1::2] = packed >> np.uint8(4)
    return out


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
