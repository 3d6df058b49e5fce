"""Hand-built quantized blocks for the oracle pins.

Encoders written from the block layouts (the inverse of decoding): a test
chooses the quantized fields, encodes them to bytes here, and checks that the
oracle's decoder returns exactly the weights those fields define.  A wrong
nibble order, scale packing or field offset in the decoder fails the round trip.
"""
import numpy as np


def f16_bits(v: float) -> int:
    return int(np.float16(v).view(np.uint16))


def enc_q8_0(d_bits: int, q: np.ndarray) -> bytes:
    assert q.shape == (32,)
    return bytes([d_bits & 255, d_bits >> 8]) + q.astype(np.int8).tobytes()


def enc_q4_0(d_bits: int, q: np.ndarray) -> bytes:
    """q: 32 values in 0..15; element j < 16 is the low nibble of byte j, j+16 the high one."""
    assert q.shape == (32,) and q.min() >= 0 and q.max() <= 15
    qs = [(int(q[j]) | (int(q[j + 16]) << 4)) for j in range(16)]
    return bytes([d_bits & 255, d_bits >> 8]) + bytes(qs)


def enc_q4_k(d_bits: int, dmin_bits: int, sc: np.ndarray, mn: np.ndarray, q: np.ndarray) -> bytes:
    """sc, mn: 8 six-bit values; q: 256 values in 0..15."""
    assert sc.shape == (8,) and mn.shape == (8,) and q.shape == (256,)
    s = [0] * 12
    for i in range(4):
        s[i] |= int(sc[i]) & 63
        s[i + 4] |= int(mn[i]) & 63
    for i in range(4, 8):
        s[i + 4] = (int(sc[i]) & 15) | ((int(mn[i]) & 15) << 4)
        s[i - 4] |= (int(sc[i]) >> 4) << 6
        s[i] |= (int(mn[i]) >> 4) << 6
    qs = [0] * 128
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = int(q[64 * c + l]) | (int(q[64 * c + 32 + l]) << 4)
    return (bytes([d_bits & 255, d_bits >> 8, dmin_bits & 255, dmin_bits >> 8]) + bytes(s) + bytes(qs))


def enc_q6_k(d_bits: int, sc: np.ndarray, q: np.ndarray) -> bytes:
    """sc: 16 int8 scales; q: 256 values in 0..63."""
    assert sc.shape == (16,) and q.shape == (256,)
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        n, k, l = e // 128, (e % 128) // 32, e % 32
        lo, hi = int(q[e]) & 15, int(q[e]) >> 4
        bi = 64 * n + 32 * (k % 2) + l
        ql[bi] |= lo << (4 * (k // 2))
        qh[32 * n + l] |= hi << (2 * k)
    return bytes(ql) + bytes(qh) + sc.astype(np.int8).tobytes() + bytes([d_bits & 255, d_bits >> 8])


def enc_q5_k(d_bits: int, dmin_bits: int, sc: np.ndarray, mn: np.ndarray, q: np.ndarray) -> bytes:
    """sc, mn: 8 six-bit values (packed as Q4_K); q: 256 values in 0..31.  The low four
    bits go in the nibbles as Q4_K's; the fifth bit of element 32 s + l is bit s of qh[l]."""
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 31
    q4 = enc_q4_k(d_bits, dmin_bits, sc, mn, q & 15)
    qh = [0] * 32
    for s in range(8):
        for l in range(32):
            qh[l] |= ((int(q[32 * s + l]) >> 4) & 1) << s
    return q4[:16] + bytes(qh) + q4[16:]


def enc_f16(v: np.ndarray) -> bytes:
    return np.asarray(v, np.float16).astype("<f2").tobytes()


def enc_f32(v: np.ndarray) -> bytes:
    return np.asarray(v, np.float32).astype("<f4").tobytes()
