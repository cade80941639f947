"""V-Major change detection on the GPU against the oracle.

The kernel sums |v_new - v_cache| in fp32 in its own order, the oracle in
fp64: a vector whose distance lies within a relative 1e-5 of the threshold may
fall either way (both answers are right for that precision); every other
mask entry must match exactly, the count must equal the mask's, the index list
must be exactly the set of active vectors (order unspecified), and the
refreshed cache must hold v_new exactly where the GPU marked a vector active.
"""
import numpy as np
import pytest

import oracle
import st_synth
from helpers import f64, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import temporal_attention_amd as st  # noqa: E402

BF, F32 = st.ST_BF16, st.ST_F32


def drifted(rows, H, d, seed, dt, frac=0.3, big=0.5, small=0.01):
    """v_new and a cached v that differs by a large step on about frac of the vectors, a small one elsewhere."""
    sd = "bf16" if dt == BF else "f32"
    vc = st_synth.randn((rows, H, d), seed, dtype="f32")
    r = np.random.default_rng(seed + 1)
    step = np.where(r.random((rows, H, 1)) < frac, big, small)
    vn = (vc + step * r.standard_normal((rows, H, d))).astype(np.float32)
    if sd == "bf16":
        return st_synth.f32_to_bf16_bits(vn), st_synth.f32_to_bf16_bits(vc)
    return vn, vc


def run(vn, vc, rows, H, d, thr, dt, update, with_idx=True):
    # buffers hold at least one row so that rows = 0 still passes real (non-null) pointers
    pad = lambda a: a if rows else np.zeros((1, H, d), a.dtype)   # noqa: E731
    vn_d, vc_d = to_dev(pad(vn)), to_dev(pad(vc))
    mask = t_.empty((max(rows, 1), H), dtype=t_.uint8, device="cuda")
    idx = t_.full((max(rows, 1) * H,), -1, dtype=t_.int32, device="cuda") if with_idx else None
    cnt = t_.full((1,), 7, dtype=t_.int64, device="cuda")
    st.st_v_change(vn_d, vc_d, rows, H, d, thr, dt, mask, idx, cnt, update)
    t_.cuda.synchronize()
    return (mask.cpu().numpy().astype(bool)[:rows], None if idx is None else idx.cpu().numpy()[:rows * H],
            int(cnt.item()), to_host(vc_d)[:rows])


@pytest.mark.parametrize("rows,H,d,thr,dt,update", [
    (300, 4, 72, 6.0, BF, 1),
    (257, 3, 64, 4.0, BF, 0),
    (100, 2, 128, 10.0, BF, 1),
    (90, 5, 72, 6.0, F32, 1),
    (77, 3, 40, 3.0, BF, 1),          # 5 pieces a row: 12 rows per wavefront pass, 4 idle lanes
    (41, 2, 128, 10.0, F32, 1),       # 32 pieces a row: 2 rows per pass
    (500, 1, 24, 2.0, BF, 0),         # 3 pieces a row
    (33, 7, 8, 0.0, BF, 1),           # threshold 0: every vector that changed at all
    (50, 2, 16, float("inf"), F32, 1),  # nothing is active
    (0, 4, 72, 1.0, BF, 1),           # no rows
])
def test_v_change_matches_oracle(rows, H, d, thr, dt, update):
    vn, vc = drifted(rows, H, d, 400 + rows + d, dt)
    mask, idx, cnt, cache = run(vn, vc, rows, H, d, thr, dt, update)
    dist, want, _, _ = oracle.v_change(f64(vn), f64(vc), thr)
    band = np.abs(dist - thr) <= 1e-5 * max(thr, 1e-30) if np.isfinite(thr) else np.zeros_like(want)
    assert np.array_equal(mask[~band], want[~band])
    assert cnt == int(mask.sum())
    got = np.sort(idx[:cnt])
    assert np.array_equal(got, np.flatnonzero(mask)) and np.all(idx[cnt:] == -1)
    expect_cache = np.where(mask[..., None], vn, vc) if update else vc
    assert np.array_equal(cache, expect_cache)


def test_v_change_without_index_list():
    vn, vc = drifted(200, 4, 72, 5, BF)
    mask, _, cnt, _ = run(vn, vc, 200, 4, 72, 6.0, BF, 0, with_idx=False)
    assert cnt == int(mask.sum()) and 0 < cnt < 800


def test_v_change_at_1080p_v_shape():
    rows, H, d, thr = 51 * 8160, 16, 72, 6.0
    vn, vc = drifted(rows, H, d, 9, BF, frac=0.2)
    mask, idx, cnt, cache = run(vn, vc, rows, H, d, thr, BF, 1)
    dist, want, _, _ = oracle.v_change(f64(vn), f64(vc), thr)
    band = np.abs(dist - thr) <= 1e-5 * thr
    assert np.array_equal(mask[~band], want[~band])
    assert cnt == int(mask.sum()) and 0.15 < cnt / mask.size < 0.25
    assert np.array_equal(np.sort(idx[:cnt]), np.flatnonzero(mask))
    assert np.array_equal(cache, np.where(mask[..., None], vn, vc))
