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
