"""Hand encoders for the canonical weight blocks (test side).

They write blocks from explicit (scale, code) values so that tests can build
matrices whose products are known in closed form.  They share no code with the
oracle's decoder.
"""
import struct

import numpy as np

F16, Q8_0, Q4_0, U8A_G32 = 0, 1, 2, 3


class M:
    def __init__(self, fmt, n, k, data):
        self.fmt, self.n, self.k = fmt, n, k
        self.data = np.frombuffer(bytes(data), np.uint8).copy() if not isinstance(data, np.ndarray) else data


def h16(v: float) -> bytes:
    return struct.pack("<e", v)


def enc_q8_0(d, q) -> M:
    """d: [n][k/32] floats (fp16-representable); q: int [n][k] in [-128, 127]."""
    q = np.asarray(q)
    n, k = q.shape
    out = bytearray()
    for r in range(n):
        for b in range(k // 32):
            out += h16(float(d[r][b]))
            out += bytes(int(v) & 0xFF for v in q[r, b * 32:(b + 1) * 32])
    return M(Q8_0, n, k, out)


def enc_q4_0(d, q) -> M:
    """d: [n][k/32]; q: int [n][k] codes in [0, 15] (value = (q - 8) * d)."""
    q = np.asarray(q)
    n, k = q.shape
    out = bytearray()
    for r in range(n):
        for b in range(k // 32):
            out += h16(float(d[r][b]))
            blk = q[r, b * 32:(b + 1) * 32]
            out += bytes(int(blk[j]) | (int(blk[j + 16]) << 4) for j in range(16))
    return M(Q4_0, n, k, out)


def enc_u8a(s, z, q) -> M:
    """s, z: [n][k/32]; q: int [n][k] in [0, 255] (value = s * (q - z))."""
    q = np.asarray(q)
    n, k = q.shape
    out = bytearray()
    for r in range(n):
        for b in range(k // 32):
            out += h16(float(s[r][b])) + h16(float(z[r][b]))
            out += bytes(int(v) for v in q[r, b * 32:(b + 1) * 32])
    return M(U8A_G32, n, k, out)


def enc_f16(w) -> M:
    w = np.asarray(w, np.float16)
    return M(F16, w.shape[0], w.shape[1], w.reshape(-1).view(np.uint8).copy())
