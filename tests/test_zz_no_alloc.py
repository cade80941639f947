"""st_block_sliced_noalloc (the allocation-free variant of st_block_sliced, for callers that
cannot allocate device memory) against st_block_sliced on the same inputs: bit-identical, on two
calls in a row, the second with a smaller input than the first."""
import numpy as np
import pytest

import st_synth
from helpers import empty, to_dev, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import temporal_attention_amd as st  # noqa: E402

EPS, BASE = st_synth.EPS, st_synth.ROPE_BASE


def case(seed, T, S, grid_w, C, H, d, dtype):
    sd = "bf16" if dtype == st.ST_BF16 else "f32"
    x = to_dev(st_synth.randn((1, T, S, C), seed, dtype=sd))
    wd = {}
    for i, tag in enumerate("st"):
        wd[tag] = dict(w_qkv=to_dev(st_synth.randn((3 * H * d, C), seed + 10 + i, std=0.02, dtype=sd)),
                       w_o=to_dev(st_synth.randn((C, H * d), seed + 20 + i, std=0.02, dtype=sd)),
                       g_q=t_.ones(d, device="cuda"), g_k=t_.ones(d, device="cuda"))
    lw = {k: st.layer_weights(v["w_qkv"], v["w_o"], v["g_q"], v["g_k"]) for k, v in wd.items()}
    return x, wd, lw


def with_workspace(x, lw, T, tv, S, grid_w, C, H, d, n_t, n_s, dtype):
    nb = st.st_block_sliced_workspace(1, T, S, grid_w, C, H, d, n_t, n_s, dtype)
    ws = t_.empty(nb, dtype=t_.uint8, device="cuda")
    y = empty((1, T, S, C), dtype == st.ST_BF16)
    st.st_block_sliced(x, 1, T, tv, S, grid_w, C, H, d, n_t, n_s, lw["s"], lw["t"], EPS, BASE, dtype, y, ws, nb)
    return y


@pytest.mark.parametrize("dtype", [st.ST_BF16, st.ST_F32])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    bf = dtype == st.ST_BF16
    shapes = ([(6, 960, 40, 1152, 16, 72, 2, 3), (4, 48, 8, 1152, 16, 72, 1, 1)] if bf
              else [(4, 64, 8, 128, 2, 64, 2, 2), (2, 16, 4, 128, 2, 64, 1, 1)])
    for i, (T, S, grid_w, C, H, d, n_t, n_s) in enumerate(shapes):   # the second call is smaller
        need = st.st_block_sliced_workspace(1, T, S, grid_w, C, H, d, n_t, n_s, dtype)
        assert 0 < need <= st.st_block_sliced_noalloc_max()
        x, wd, lw = case(70 + i, T, S, grid_w, C, H, d, dtype)
        y_ref = with_workspace(x, lw, T, T - 1, S, grid_w, C, H, d, n_t, n_s, dtype)
        y = empty((1, T, S, C), bf)
        y.fill_(7.0)
        st.st_block_sliced_noalloc(x, 1, T, T - 1, S, grid_w, C, H, d, n_t, n_s, lw["s"], lw["t"], EPS, BASE, dtype, y)
        t_.cuda.synchronize()
        assert t_.equal(y, y_ref), f"call {i}: noalloc differs from st_block_sliced"
        assert bool(t_.isfinite(y.float()).all())


def test_noalloc_rejects_shapes_beyond_its_scratch():
    T, S, grid_w, C, H, d = 24, 3600, 80, 1152, 16, 72      # the 720p layer pair: ~1 GB of workspace
    assert st.st_block_sliced_workspace(1, T, S, grid_w, C, H, d, 1, 1, st.ST_BF16) > st.st_block_sliced_noalloc_max()
    x = empty((1, T, S, C))
    y = empty((1, T, S, C))
    w = st.layer_weights(x, x, x, x)   # never read: validation fails first
    with pytest.raises(st.STError) as e:
        st.st_block_sliced_noalloc(x, 1, T, T, S, grid_w, C, H, d, 1, 1, w, w, EPS, BASE, st.ST_BF16, y)
    assert e.value.code == st.ST_EWORKSPACE
