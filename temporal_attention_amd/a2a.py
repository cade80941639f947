"""Local pack / unpack around the P-way all-to-all between the two shardings of a layer pair.

ScaleFusion review, "Technical architecture" (layer table) and the algorithm
pseudocode: with P GPUs a rank holds its patch block [B, T, S/P, C] for the
temporal layer and a frame block [B, T/P, S, C] for the spatial layer; an
all-to-all converts between them.  A collective moves contiguous per-peer
chunks, so each direction is pack -> all-to-all -> unpack, and pack and unpack
are permutations that st_relayout performs.  This module only computes their
strides (argument marshalling); the exchange itself is the collective's.

Chunk layout on the wire, both directions: [P, B, T/P, S/P, C], chunk q
contiguous (one rank's share).

    s2t  (before the spatial layer)   x [B, T, S/P, C]  --pack-->  send[q] = frame block q
                                      recv[q] = patch block of rank q  --unpack-->  [B, T/P, S, C]
    t2s  (before the temporal layer)  x [B, T/P, S, C]  --pack-->  send[q] = patch block q
                                      recv[q] = frame block of rank q  --unpack-->  [B, T, S/P, C]
"""
from __future__ import annotations

from . import _lib as L


def _elem_bytes(t) -> int:
    return t.element_size()


def _copy(src, src_strides, dst, dst_strides, dims, stream):
    L.st_relayout(src, src_strides, dst, dst_strides, dims, len(dims), _elem_bytes(src), stream)


def _chunk_strides(B, tp, sp, C):
    """Contiguous strides of [P, B, T/P, S/P, C]."""
    return [B * tp * sp * C, tp * sp * C, sp * C, C, 1]


def pack_s2t(x, send, B, T, S_loc, C, P, stream=None):
    """x [B, T, S/P, C] (this rank's patches) -> send [P, B, T/P, S/P, C]: chunk q = frames q*T/P.."""
    tp = T // P
    dims = [P, B, tp, S_loc, C]
    _copy(x, [tp * S_loc * C, T * S_loc * C, S_loc * C, C, 1], send, _chunk_strides(B, tp, S_loc, C), dims, stream)


def unpack_s2t(recv, y, B, T, S_loc, C, P, stream=None):
    """recv [P, B, T/P, S/P, C] (chunk q from rank q) -> y [B, T/P, S, C] with rank q's patches at q*S/P.."""
    tp, S = T // P, S_loc * P
    dims = [P, B, tp, S_loc, C]
    _copy(recv, _chunk_strides(B, tp, S_loc, C), y, [S_loc * C, tp * S * C, S * C, C, 1], dims, stream)


def pack_t2s(x, send, B, T, S, C, P, stream=None):
    """x [B, T/P, S, C] (this rank's frames) -> send [P, B, T/P, S/P, C]: chunk q = patches q*S/P.."""
    tp, sp = T // P, S // P
    dims = [P, B, tp, sp, C]
    _copy(x, [sp * C, tp * S * C, S * C, C, 1], send, _chunk_strides(B, tp, sp, C), dims, stream)


def unpack_t2s(recv, y, B, T, S, C, P, stream=None):
    """recv [P, B, T/P, S/P, C] (chunk q = rank q's frames) -> y [B, T, S/P, C] with rank q's frames at q*T/P.."""
    tp, sp = T // P, S // P
    dims = [P, B, tp, sp, C]
    _copy(recv, _chunk_strides(B, tp, sp, C), y, [tp * sp * C, T * sp * C, sp * C, C, 1], dims, stream)
