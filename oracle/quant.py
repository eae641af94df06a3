"""INT4 / INT8 KV encodings, step by step in float32 (oracle; test infrastructure only).

Source: KV4-RL review, section 1 ("INT4 KV Cache Quantization", "Selective
Protection") and section 3 (full context stored as calibration-free paged
INT4; sink and recent positions in an INT8 side cache). The pages give no
numeric rule; the readings used here are:

INT4, per (token, kv head, K or V, group of 32 consecutive head_dim entries):
  mn, mx        = min and max of the 32 float32 values
  s32           = (mx - mn) / 15                      float32, round-to-nearest-even
  scale_h       = fp16(s32), min_h = fp16(mn)          RNE, saturated to +-65504
  inv           = 1 / float32(scale_h) if scale_h > 0 else 0   (float32 RNE)
  c_i           = clamp(rint((x_i - float32(min_h)) * inv), 0, 15)   (ties to even)
  decoded value = c_i * scale_h + min_h

INT8, per (token, kv head, K or V) over all head_dim entries:
  s   = max|x_i| / 127 (float32, stored as float32)
  inv = 1 / s if s >= 2**-126 else 0   (a scale below the smallest normal
        float32 counts as zero, so the reciprocal never overflows)
  c_i = clamp(rint(x_i * inv), -127, 127)
  decoded value = c_i * s

Every product and difference above is a separate float32 operation (NumPy
never contracts them into a fused multiply-add).
"""
from __future__ import annotations

import numpy as np

GROUP = 32
FP16_MAX = np.float32(65504.0)
FLT_MIN = np.float32(2.0 ** -126)


def int4_encode(x):
    """Encode ``x`` (float32 [..., D], D a multiple of 32).

    Returns (codes uint8 [..., D] in 0..15, scale fp16 [..., D/32], min fp16 [..., D/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    g = x.reshape(*x.shape[:-1], D // GROUP, GROUP)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s32 = (mx - mn) / np.float32(15.0)
    scale_h = np.clip(s32, -FP16_MAX, FP16_MAX).astype(np.float16)
    min_h = np.clip(mn, -FP16_MAX, FP16_MAX).astype(np.float16)
    sf = scale_h.astype(np.float32)
    mf = min_h.astype(np.float32)
    pos = sf > 0
    inv = np.where(pos, np.float32(1.0) / np.where(pos, sf, np.float32(1.0)), np.float32(0.0))
    inv = inv.astype(np.float32)
    diff = (g - mf[..., None]).astype(np.float32)
    t = (diff * inv[..., None]).astype(np.float32)
    c = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    return c.reshape(x.shape), scale_h, min_h


def int4_decode(codes, scale_h, min_h):
    """Decoded INT4 values in float64: c * scale + min per group of 32."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    c = codes.reshape(*codes.shape[:-1], D // GROUP, GROUP).astype(np.float64)
    v = c * np.asarray(scale_h, np.float64)[..., None] + np.asarray(min_h, np.float64)[..., None]
    return v.reshape(codes.shape)


def int8_encode(x):
    """Encode ``x`` (float32 [..., D]): (codes int8 [..., D] in -127..127, scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).max(axis=-1)
    s = (a / np.float32(127.0)).astype(np.float32)
    pos = s >= FLT_MIN
    inv = np.where(pos, np.float32(1.0) / np.where(pos, s, np.float32(1.0)), np.float32(0.0))
    inv = inv.astype(np.float32)
    t = (x * inv[..., None]).astype(np.float32)
    c = np.clip(np.rint(t), -127, 127).astype(np.int8)
    return c, s


def int8_decode(codes, scale):
    """Decoded INT8 values in float64: c * s."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[..., None]


def pack_nibbles(codes):
    """Pack 4-bit codes along the last axis: byte j = c[2j] | c[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of :func:`pack_nibbles`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((*packed.shape[:-1], packed.shape[-1] * 2), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out
