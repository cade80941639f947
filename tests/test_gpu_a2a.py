"""Local pack / unpack around the P-way all-to-all, on the GPU against the oracle's exchange.

All P ranks are emulated on one GPU: each rank packs its shard with the library
(st_a2a_pack), the collective's block transpose is stood in for by plain device
copies (recv[q][r] = send[r][q]), and each rank unpacks.  Every element must
land where the oracle's all-to-all puts it (bit-exact), in both directions, up
to the 1080p per-GPU shape at P = 8 (T padded to 56 frames, 1020 patches per
rank).
"""
import numpy as np
import pytest

import oracle
import st_synth
from helpers import to_dev, to_host, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from temporal_attention_amd import a2a  # noqa: E402


def exchange(sends):
    """The collective's effect: rank q receives chunk q of every rank's send buffer, in rank order."""
    P = len(sends)
    return [t_.stack([sends[r][q] for r in range(P)]).contiguous() for q in range(P)]


@pytest.mark.parametrize("B,T,S,C,P,dt", [
    (2, 6, 12, 8, 3, "bf16"),
    (1, 8, 20, 4, 4, "f32"),
    (2, 4, 6, 16, 2, "bf16"),
    (1, 5, 7, 8, 1, "bf16"),
    (1, 56, 8160, 1152, 8, "bf16"),     # 1080p, P = 8: each rank 56 x 1020 x 1152
])
def test_pack_exchange_unpack_matches_oracle(B, T, S, C, P, dt):
    x = st_synth.bits((B, T, S, C), 60 + P + T, dt)
    tp, sp = T // P, S // P
    shards_s = oracle.shard(x, P, 2)                 # rank r: patches r*S/P..
    dev_s = [to_dev(np.ascontiguousarray(a)) for a in shards_s]
    sends = []
    for r in range(P):
        send = t_.empty((P, B, tp, sp, C), dtype=dev_s[r].dtype, device="cuda")
        a2a.pack_s2t(dev_s[r], send, B, T, S, C, P)
        sends.append(send)
    frames = []
    for q, recv in enumerate(exchange(sends)):
        y = t_.empty((B, tp, S, C), dtype=recv.dtype, device="cuda")
        a2a.unpack_s2t(recv, y, B, T, S, C, P)
        frames.append(y)
    t_.cuda.synchronize()
    want_t = oracle.a2a_s_to_t(shards_s)
    for q in range(P):
        assert np.array_equal(to_host(frames[q]), want_t[q]), f"s2t rank {q}"
    sends = []
    for r in range(P):
        send = t_.empty((P, B, tp, sp, C), dtype=frames[r].dtype, device="cuda")
        a2a.pack_t2s(frames[r], send, B, T, S, C, P)
        sends.append(send)
    back = []
    for q, recv in enumerate(exchange(sends)):
        y = t_.empty((B, T, sp, C), dtype=recv.dtype, device="cuda")
        a2a.unpack_t2s(recv, y, B, T, S, C, P)
        back.append(y)
    t_.cuda.synchronize()
    want_s = oracle.a2a_t_to_s(want_t)
    for q in range(P):
        got = to_host(back[q])
        assert np.array_equal(got, want_s[q]), f"t2s rank {q}"
        assert np.array_equal(got, shards_s[q]), f"round trip rank {q}"
