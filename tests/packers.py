"""Test-side packers: write known codes / scales into the byte formats.

These are written independently of both the oracle (which only unpacks) and
the GPU library.  The layouts they produce: affine-4 low nibble first, 8 codes
per little-endian 32-bit word; affine-8 one byte per code, least significant
byte first; Q4_K the public 144-byte GGUF block; Q6_K the public 210-byte GGUF
block.  The hand-packed pins in test_oracle_pins.py fix those layouts byte by
byte.
"""
import numpy as np


def pack_affine4_codes(q):
    """q: int array [N, K] with values 0..15 -> uint32 [N, K/8]."""
    q = np.asarray(q, dtype=np.uint64)
    N, K = q.shape
    assert K % 8 == 0
    q = q.reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), dtype=np.uint64)
    for i in range(8):
        words |= q[:, :, i] << np.uint64(4 * i)
    return words.astype(np.uint32)


def pack_affine8_codes(q):
    """q: int array [N, K] with values 0..255 -> uint32 [N, K/4]: the bytes laid out in order and
    read back as little-endian words (a byte view, no shifts)."""
    q = np.ascontiguousarray(np.asarray(q).astype(np.uint8))
    N, K = q.shape
    assert K % 4 == 0
    return q.view("<u4").reshape(N, K // 4).astype(np.uint32)


def pack_q4k_scales(sc, m):
    """sc, m: int arrays [..., 8] of 6-bit values -> uint8 [..., 12]."""
    sc = np.asarray(sc, dtype=np.uint8)
    m = np.asarray(m, dtype=np.uint8)
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.uint8)
    for j in range(4):
        out[..., j] = (sc[..., j] & 63) | ((sc[..., j + 4] >> 4) << 6)
        out[..., j + 4] = (m[..., j] & 63) | ((m[..., j + 4] >> 4) << 6)
        out[..., j + 8] = (sc[..., j + 4] & 15) | ((m[..., j + 4] & 15) << 4)
    return out


def pack_q4k_codes(q):
    """q: int array [..., 256] (codes of one block, in weight order) -> uint8 [..., 128]."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.zeros(q.shape[:-1] + (128,), dtype=np.uint8)
    for c in range(4):
        lo = q[..., 64 * c: 64 * c + 32]
        hi = q[..., 64 * c + 32: 64 * c + 64]
        out[..., 32 * c: 32 * c + 32] = (lo & 15) | ((hi & 15) << 4)
    return out


def q4k_block(d_bits, dmin_bits, sc, m, q):
    """Assemble Q4_K blocks. d_bits/dmin_bits: uint16 [...]; sc, m: [..., 8]; q: [..., 256]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    dmin_bits = np.asarray(dmin_bits, dtype=np.uint16)
    shape = d_bits.shape
    out = np.zeros(shape + (144,), dtype=np.uint8)
    out[..., 0] = d_bits & 0xFF
    out[..., 1] = d_bits >> 8
    out[..., 2] = dmin_bits & 0xFF
    out[..., 3] = dmin_bits >> 8
    out[..., 4:16] = pack_q4k_scales(sc, m)
    out[..., 16:144] = pack_q4k_codes(q)
    return out


def q6k_block(d_bits, sc, q):
    """Assemble Q6_K blocks (210 bytes). d_bits: uint16 [...]; sc: int8-valued [..., 16];
    q: [..., 256] with values -32..31.  Weight o = 128h + 32j + l sits in the low (j < 2) or
    high (j >= 2) nibble of ql[64h + 32(j%2) + l] and in bits 2j, 2j+1 of qh[32h + l]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    u = np.asarray(q, dtype=np.int64) + 32
    assert u.min() >= 0 and u.max() <= 63
    shape = d_bits.shape
    u = u.reshape(shape + (2, 4, 32))  # [..., h, j, l]
    lo, hi = u & 15, u >> 4
    ql = np.zeros(shape + (2, 2, 32), dtype=np.int64)  # [..., h, j%2, l]
    ql[..., 0, :] = lo[..., 0, :] | (lo[..., 2, :] << 4)
    ql[..., 1, :] = lo[..., 1, :] | (lo[..., 3, :] << 4)
    qh = hi[..., 0, :] | (hi[..., 1, :] << 2) | (hi[..., 2, :] << 4) | (hi[..., 3, :] << 6)  # [..., h, l]
    out = np.zeros(shape + (210,), dtype=np.uint8)
    out[..., 0:128] = ql.reshape(shape + (128,))
    out[..., 128:192] = qh.reshape(shape + (64,))
    out[..., 192:208] = np.asarray(sc, dtype=np.int64).astype(np.int8).view(np.uint8)
    out[..., 208] = d_bits & 0xFF
    out[..., 209] = d_bits >> 8
    return out
