"""Offline round-to-nearest int4 weight encoding, group 128 along K (TEST INFRASTRUCTURE).

Page anchors: PhyAI reading ("PhyAI: Real-Time Physical AI at the Edge,
Scalable Rollouts in the Cloud"), Sec. 5.4 (offline round-to-nearest
quantisation prepares optional low-precision artifacts) and Figure 3 (the
quantizer as an offline service); VLA-HWBench abstract on the first page
(4-bit weights plus kernel fusion for pi0.5).

The pages say only "4-bit", "round-to-nearest" and "offline".  The encoding
read here, step by step, for a weight matrix W [N][K] (float32) and each row
and group G of 128 consecutive k:

1. amax = max |W_G| (exact in float32);
2. s = bf16 round-to-nearest-even of (amax / 7) computed as a float32 division;
   s = 0 when amax = 0;
3. q = round-half-even(W / s) (float32 division), clamped to [-8, 7]; q = 0 when s = 0;
4. q is stored as 4-bit two's complement; byte j of a row holds k = 2j in its
   low nibble and k = 2j+1 in its high nibble;
5. dequantisation is w = q * s (exact in float32 and float64).

The quantisation decision (steps 2-3) is taken in float32, the precision the
GPU quantiser uses, so both sides produce the same integers.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    Written from the definition: keep the top 16 bits of the float32 pattern
    after adding half an ulp of the 16-bit result, the half-ulp reduced by one
    when the kept part is even (so exact halves go to the even neighbour).
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_is_odd = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + keep_is_odd) >> 16
    return (rounded.astype(np.uint32) << 16).view(np.float32)


def quantize(w) -> tuple[np.ndarray, np.ndarray]:
    """Quantise W [N][K] (K a multiple of 128).

    Returns (packed uint8 [N][K/2], scales as bf16 bit patterns uint16 [N][K/128]).
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = w.reshape(n, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    s = _bf16_round((amax / np.float32(7.0)).astype(np.float32))
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    ratio = (g / safe[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -8, 7)
    q = np.where(s[:, :, None] > 0, q, 0).astype(np.int8).reshape(n, k)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    s_bits = (s.view(np.uint32) >> 16).astype(np.uint16)
    return packed, s_bits


def unpack_codes(packed) -> np.ndarray:
    """uint8 [N][K/2] -> signed codes int8 [N][K] (low nibble first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    n, half = packed.shape
    q = np.empty((n, 2 * half), dtype=np.int8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def scales_f64(s_bits) -> np.ndarray:
    return (np.asarray(s_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequantize(packed, s_bits) -> np.ndarray:
    """w = q * s in float64, [N][K]."""
    q = unpack_codes(packed).astype(np.float64)
    s = scales_f64(s_bits)
    n, k = q.shape
    return (q.reshape(n, k // GROUP, GROUP) * s[:, :, None]).reshape(n, k)


def quantize_stack(w) -> tuple[np.ndarray, np.ndarray]:
    """Quantise a stack [L][N][K] layer by layer."""
    w = np.asarray(w, dtype=np.float32)
    packs, scales = zip(*(quantize(w[i]) for i in range(w.shape[0])))
    return np.stack(packs), np.stack(scales)


def dequantize_stack(packed, s_bits) -> np.ndarray:
    return np.stack([dequantize(packed[i], s_bits[i]) for i in range(packed.shape[0])])
