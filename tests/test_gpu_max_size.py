"""Parity past 2^31: every tensor below holds more than 2^31 elements (the relayout's, more than
2^32 bytes), so any element or byte offset the kernels computed in 32 bits would wrap.  The inputs are seeded
blocks (st_synth) repeated along one axis on the device, with a period that does not divide the
2^31-element wrap distance, so a wrapped offset reads other data and fails the check.  Outputs are
compared with the oracle on sampled rows, among them the ones on both sides of the wrap point
and the last ones.
"""
import math

import numpy as np
import pytest

import oracle
import st_synth
from helpers import assert_close, f64, to_dev, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import temporal_attention_amd as st  # noqa: E402

BF = st.ST_BF16
WRAP = 1 << 31


def sync():
    t_.cuda.synchronize()


def tiled(block, n, axis):
    """Device tensor: the storage-form block repeated along `axis` to length n."""
    blk = to_dev(block)
    p = blk.shape[axis]
    shape = list(blk.shape)
    shape[axis] = n
    out = t_.empty(shape, dtype=blk.dtype, device="cuda")
    for i0 in range(0, n, p):
        m = min(p, n - i0)
        out.narrow(axis, i0, m).copy_(blk.narrow(axis, 0, m))
    return out


def around(i, n, width=3):
    return [j for j in range(i - width, i + width + 1) if 0 <= j < n]


def free():
    sync()
    t_.cuda.empty_cache()


def test_relayout_past_4gb():
    """[1, 8, 250000, 288] int64 (4.6 GB, rows of 2304 bytes like a 1152-channel bf16 row) to
    [1, 250000, 8, 288]: byte offsets pass 2^31 and 2^32.  The source holds each element's own
    index, so every element is unique."""
    B, T, S, C = 1, 8, 250000, 288
    n = B * T * S * C
    assert n * 8 > 2 * WRAP
    src = t_.arange(n, dtype=t_.int64, device="cuda")
    dst = t_.full((n,), -1, dtype=t_.int64, device="cuda")
    st.st_relayout(src, [T * S * C, S * C, C, 1], dst, [S * T * C, C, T * C, 1], [B, T, S, C], 4, 8)
    sync()
    assert not bool((dst < 0).any()), "destination elements left unwritten"
    row_bytes = T * C * 8      # bytes of one destination patch
    rng = np.random.default_rng(7)
    s_idx = np.unique(np.concatenate([[0, S - 1], around(WRAP // row_bytes, S), around(2 * WRAP // row_bytes, S),
                                      rng.choice(S, 256, replace=False)]))
    si = t_.from_numpy(s_idx).cuda()
    got = dst.view(B, S, T, C).index_select(1, si).cpu().numpy()
    src_rows = src.view(B, T, S, C).index_select(2, si).cpu().numpy()
    assert np.array_equal(got, oracle.bt_to_bs(src_rows))
    del src, dst
    free()


def test_qkv_norm_rope_past_2g_rows_x_channels():
    """QKV projection + RMSNorm + 1D RoPE on 1,900,057 rows x 1152: q, k, v and x each hold
    2.19e9 elements."""
    rows, C, H, d, P = 1_900_057, 1152, 16, 72, 100_003
    assert rows * H * d > WRAP
    x_blk = st_synth.randn((P, C), 901, dtype="bf16")
    w = st_synth.randn((3 * H * d, C), 902, std=0.02, dtype="bf16")
    rng = np.random.default_rng(903)
    g_q = (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    g_k = (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    period = 51
    tab = t_.empty(st.st_rope_table_floats(d, st.ST_ROPE_1D, period), dtype=t_.float32, device="cuda")
    st.st_rope_table(d, st.ST_ROPE_1D, 10000.0, period, tab)
    x = tiled(x_blk, rows, 0)
    q, k, v = (t_.empty((rows, H, d), dtype=t_.bfloat16, device="cuda") for _ in range(3))
    st.st_qkv_norm_rope(x, rows, C, to_dev(w), to_dev(g_q), to_dev(g_k), 1e-6, 1.0, st.ST_ROPE_1D, tab, period,
                        None, period, 0, 0, H, d, BF, q, k, v)
    sync()
    wrap_r = WRAP // (H * d)
    r_idx = np.unique(np.concatenate([[0, rows - 1], around(wrap_r, rows), np.arange(rows - 64, rows),
                                      rng.choice(rows, 128, replace=False)]))
    ri = t_.from_numpy(r_idx).cuda()
    oq, ok, ov = oracle.qkv_norm_rope(f64(x_blk[r_idx % P]), f64(w), g_q, g_k, 1e-6, H, d, "1d", r_idx % period,
                                      10000.0)
    for name, got, ref in (("q", q, oq), ("k", k, ok), ("v", v, ov)):
        assert_close(f64(got.index_select(0, ri)), ref, what=name)
    del x, q, k, v
    free()


def test_out_proj_relayout_past_2g_outputs():
    """Output projection with the [n1, n2] -> [n2, n1] row store on 19 x 100003 rows x 1152:
    the input and the output each hold 2.19e9 elements."""
    n1, n2, K, N = 19, 100_003, 1152, 1152
    rows = n1 * n2
    assert rows * N > WRAP
    P = 65_537
    a_blk = st_synth.randn((P, K), 911, dtype="bf16")
    w = st_synth.randn((N, K), 912, std=0.02, dtype="bf16")
    a = tiled(a_blk, rows, 0)
    y = t_.full((rows, N), float("nan"), dtype=t_.bfloat16, device="cuda")
    st.st_out_proj_relayout(a, rows, K, to_dev(w), N, BF, n1, n2, y)
    sync()
    rng = np.random.default_rng(913)
    # output rows: around the wrap point, the last ones, random; input row r = i1 * n2 + i2 lands at i2 * n1 + i1
    o_idx = np.unique(np.concatenate([[0, rows - 1], around(WRAP // N, rows), np.arange(rows - 64, rows),
                                      rng.choice(rows, 128, replace=False)]))
    i2, i1 = o_idx // n1, o_idx % n1
    r_in = i1 * n2 + i2
    got = f64(y.index_select(0, t_.from_numpy(o_idx).cuda()))
    assert_close(got, oracle.linear(f64(a_blk[r_in % P]), f64(w)), what="y")
    del a, y
    free()


def test_attn_spatial_past_2g_elements():
    """Spatial attention over 300 frames of the 1080p frame (8160 patches, 16 heads x 72): q, k, v
    and the output each hold 2.82e9 elements; whole (frame, head) sequences are checked."""
    T, S, H, d, P = 300, 8160, 16, 72, 7
    assert T * S * H * d > WRAP
    blk = [st_synth.randn((1, P, S, H, d), 921 + i, dtype="bf16") for i in range(3)]
    q, k, v = (tiled(b, T, 1) for b in blk)
    out = t_.empty((1, T, S, H, d), dtype=t_.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(d)
    st.st_attn_spatial(q, k, v, 1, T, S, H, d, scale, BF, None, 0, out)
    sync()
    wrap_t = WRAP // (S * H * d)
    for t, h in ((wrap_t, 15), (wrap_t + 1, 0), (T - 1, 15), (0, 3)):
        got = f64(out[0, t, :, h])
        ref = oracle.attention(f64(blk[0][0, t % P, :, h]), f64(blk[1][0, t % P, :, h]), f64(blk[2][0, t % P, :, h]),
                               scale)
        assert_close(got, ref, what=f"O[t={t}, h={h}]")
    del q, k, v, out
    free()


def test_attn_temporal_past_2g_elements():
    """Temporal attention over 51 frames at 40000 patches, 16 heads x 72: q, k, v and the output
    each hold 2.35e9 elements; sampled patches before, across and after the wrap point."""
    S, T, H, d, P = 40_000, 51, 16, 72, 1009
    assert S * T * H * d > WRAP
    blk = [st_synth.randn((1, P, T, H, d), 931 + i, dtype="bf16") for i in range(3)]
    q, k, v = (tiled(b, S, 1) for b in blk)
    out = t_.empty((1, S, T, H, d), dtype=t_.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(d)
    st.st_attn_temporal(q, k, v, 1, S, T, T, H, d, scale, BF, None, 0, out)
    sync()
    wrap_s = WRAP // (T * H * d)
    s_idx = np.unique(np.concatenate([[0, S - 1], around(wrap_s, S), np.random.default_rng(933).choice(S, 32,
                                                                                                       replace=False)]))
    got = f64(out.index_select(1, t_.from_numpy(s_idx).cuda()))
    ref = oracle.attn_temporal(*(f64(b[:, s_idx % P]) for b in blk), scale)
    assert_close(got, ref, what="O")
    del q, k, v, out
    free()
