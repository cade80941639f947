"""Local pack / unpack around the P-way all-to-all between the two shardings of a layer pair.

Argument marshalling for st_a2a_pack / st_a2a_unpack (include/st.h), which hold
the index maps.  ScaleFusion review, "Technical architecture" (layer table) and
the algorithm pseudocode: with P GPUs a rank holds its patch block
[B, T, S/P, C] for the temporal layer and a frame block [B, T/P, S, C] for the
spatial layer; an all-to-all converts between them.  Chunk layout on the wire,
both directions: [P, B, T/P, S/P, C], chunk q contiguous (one rank's share).
T and S are the global frame and patch counts.
"""
from __future__ import annotations

from . import _lib as L


def pack_s2t(x, send, B, T, S, C, P, stream=None):
    """x [B, T, S/P, C] (this rank's patches) -> send [P, B, T/P, S/P, C]: chunk q = frames q*T/P.."""
    L.st_a2a_pack(x, send, L.ST_A2A_S2T, B, T, S, C, P, x.element_size(), stream)


def unpack_s2t(recv, y, B, T, S, C, P, stream=None):
    """recv [P, B, T/P, S/P, C] (chunk r from rank r) -> y [B, T/P, S, C] with rank r's patches at r*S/P.."""
    L.st_a2a_unpack(recv, y, L.ST_A2A_S2T, B, T, S, C, P, recv.element_size(), stream)


def pack_t2s(x, send, B, T, S, C, P, stream=None):
    """x [B, T/P, S, C] (this rank's frames) -> send [P, B, T/P, S/P, C]: chunk q = patches q*S/P.."""
    L.st_a2a_pack(x, send, L.ST_A2A_T2S, B, T, S, C, P, x.element_size(), stream)


def unpack_t2s(recv, y, B, T, S, C, P, stream=None):
    """recv [P, B, T/P, S/P, C] (chunk r = rank r's frames) -> y [B, T, S/P, C] with rank r's frames at r*T/P.."""
    L.st_a2a_unpack(recv, y, L.ST_A2A_T2S, B, T, S, C, P, recv.element_size(), stream)
