"""Byte layouts of the C ABI's buffers, as include/serq.h states them,
written out independently of the library for the tests."""

from __future__ import annotations

import numpy as np

from oracle import serq_oracle as O


def rq_row_bytes(r: int) -> int:
    """Q(R) rows: r codes padded with zero codes to a multiple of 32."""
    return -(-r // 32) * 16


def pad_rq(packed: np.ndarray, r: int) -> np.ndarray:
    """N x r/2 packed Q(R) rows -> the N x rq_row_bytes(r) buffer layout."""
    packed = np.asarray(packed, np.uint8).reshape(packed.shape[0], r // 2)
    return np.pad(packed, ((0, 0), (0, rq_row_bytes(r) - r // 2)))


def pack_rq(codes: np.ndarray) -> np.ndarray:
    """r x N int4 codes of Q(R) -> the N x rq_row_bytes(r) buffer layout."""
    r, n = codes.shape
    if r == 0:
        return np.zeros((n, 0), np.uint8)
    return pad_rq(O.pack_int4(codes.T), r)


def unpack_rq(buf: np.ndarray, r: int) -> np.ndarray:
    """The N x rq_row_bytes(r) buffer -> r x N int4 codes."""
    if r == 0:
        return np.zeros((0, buf.shape[0]), np.int8)
    return O.unpack_int4(np.ascontiguousarray(buf[:, : r // 2])).T.copy()


def bf6_value(field: np.ndarray) -> np.ndarray:
    """E3M2 six-bit patterns -> their values (sign bit 5, exponent bits 4..2
    with bias 3, mantissa bits 1..0; exponent 0 is subnormal)."""
    f = np.asarray(field, np.int64)
    sign = np.where(f & 0x20, -1.0, 1.0)
    e = (f >> 2) & 7
    m = f & 3
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -2, (1.0 + m / 4.0) * np.exp2(e - 3.0))
    return sign * mag


def bf6_decode(buf: np.ndarray, rows: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """The bf6 tile layout (include/serq.h, serq_prepack_bf6) -> (the padded
    Rp x Kp matrix of decoded values, the rows x k integer codes). Each
    24-byte lane fragment is read as one little-endian 192-bit integer whose
    six-bit field f is code k = 128 kt + 64 s + 32 (lane / 32) + f of row
    32 rb + lane % 32."""
    rp, kp = -(-rows // 128) * 128, -(-k // 128) * 128
    nkt, nrb = kp // 128, rp // 32
    b = np.asarray(buf, np.uint8).reshape(nkt, nrb, 2, 64, 24)
    bits = np.unpackbits(b, axis=-1, bitorder="little").reshape(nkt, nrb, 2, 64, 32, 6)
    fields = (bits.astype(np.int64) << np.arange(6)).sum(-1)          # [kt, rb, s, lane, f]
    vals = bf6_value(fields)
    lane = np.arange(64)
    full = np.zeros((rp, kp))
    for kt in range(nkt):
        for rb in range(nrb):
            for s in range(2):
                rows_l = rb * 32 + lane % 32
                k0 = kt * 128 + 64 * s + 32 * (lane // 32)
                full[rows_l[:, None], k0[:, None] + np.arange(32)[None, :]] = vals[kt, rb, s]
    codes = full[:rows, :k]
    assert np.array_equal(codes, np.round(codes)), "bf6 fields must decode to integers"
    return full, codes.astype(np.int8)
