"""Chunk attention with log-sum-exp and the merge of chunk results, on the GPU against the fp64 oracle.

Ring and Torus attention compute attention over one key/value chunk at a time
and merge the partial results; on one GPU the identity that pins this is
chunked-then-merged == unchunked.  Inputs are seeded (st_synth), identical
bytes on both sides.

Tolerances: outputs use the bf16 / fp32 bars of the other kernels (max abs
2e-2 and rel L2 1e-2 in bf16, 1e-4 in fp32).  The log-sum-exp is a per-query
scalar of the same attention, held to the same max-abs figures: 2e-2 for the
bf16 path (fp32 arithmetic on the bf16 operands, which the oracle sees too) and
1e-4 for fp32.
"""
import math

import numpy as np
import pytest

import oracle
import st_synth
from helpers import assert_close, empty, f64, to_dev, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import temporal_attention_amd as st  # noqa: E402

BF, F32 = st.ST_BF16, st.ST_F32
LSE_BF16, LSE_F32 = 2e-2, 1e-4


def lse_tol(ref, dt):
    return LSE_BF16 if dt == BF else LSE_F32


def sync():
    t_.cuda.synchronize()


def tensors(shape_q, shape_kv, seed, dt, q_std=1.0):
    sd = "bf16" if dt == BF else "f32"
    return (st_synth.randn(shape_q, seed, std=q_std, dtype=sd), st_synth.randn(shape_kv, seed + 1, dtype=sd),
            st_synth.randn(shape_kv, seed + 2, dtype=sd))


def lse_buf(outer, H, L):
    return t_.empty((outer, H, L), dtype=t_.float32, device="cuda")


def check_lse(got, ref, dt, what="lse"):
    got = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= lse_tol(ref[fin], dt), f"{what}: max_abs={err:.3e}"


CHUNK_CASES = [
    # outer, Lq, Lk, kv_valid, H, d, q_std, dtype
    (3, 300, 500, 500, 2, 72, 1.0, BF),     # fewer queries than keys
    (2, 257, 100, 77, 3, 72, 3.0, BF),      # masked tail, peaked softmax (many rescales)
    (1, 300, 1000, 1000, 2, 72, 5.0, BF),   # q std 5: scores of std 5, up to ~20
    (1, 64, 1, 1, 2, 72, 1.0, BF),          # one key
    (2, 100, 130, 130, 2, 128, 1.0, BF),
    (2, 70, 200, 150, 2, 64, 2.0, BF),
    (2, 33, 40, 35, 2, 64, 1.0, F32),
    (2, 50, 20, 0, 2, 72, 1.0, BF),         # empty chunk: out 0, lse -inf
    (2, 10, 5, 0, 2, 64, 1.0, F32),
]


@pytest.mark.parametrize("outer,Lq,Lk,kv_valid,H,d,q_std,dt", CHUNK_CASES)
def test_attn_chunk_matches_oracle(outer, Lq, Lk, kv_valid, H, d, q_std, dt):
    q, k, v = tensors((outer, Lq, H, d), (outer, Lk, H, d), 700 + Lq + Lk + d, dt, q_std)
    out, lse = empty((outer, Lq, H, d), dt == BF), lse_buf(outer, H, Lq)
    scale = 1.0 / math.sqrt(d)
    st.st_attn_chunk(to_dev(q), to_dev(k), to_dev(v), outer, Lq, Lk, kv_valid, H, d, scale, dt, out, lse)
    sync()
    ro, rl = oracle.attn_chunk(f64(q), f64(k), f64(v), scale, kv_valid)
    if kv_valid == 0:
        assert np.all(f64(out) == 0.0)
    else:
        assert_close(f64(out), ro, bf16=dt == BF, what="O")
    check_lse(lse, rl, dt)


def test_attn_chunk_without_lse_path_matches_spatial_kernel():
    # Lq = Lk, all keys valid: the chunk entry point is spatial attention plus lse, bit for bit
    outer, L, H, d = 2, 333, 2, 72
    q, k, v = (to_dev(a) for a in tensors((outer, L, H, d), (outer, L, H, d), 901, BF))
    a, b = empty((outer, L, H, d)), empty((outer, L, H, d))
    st.st_attn_chunk(q, k, v, outer, L, L, L, H, d, 1 / math.sqrt(d), BF, a, lse_buf(outer, H, L))
    st.st_attn_spatial(q, k, v, 1, outer, L, H, d, 1 / math.sqrt(d), BF, None, 0, b)
    sync()
    assert t_.equal(a, b)


@pytest.mark.parametrize("dt,d,cuts,valid", [
    (BF, 72, (300, 301), 950),        # three chunks, one of a single key, masked tail
    (BF, 128, (64, 500), 700),
    (BF, 64, (1,), 1000),
    (F32, 64, (100, 450), 999),
])
def test_chunked_then_merged_equals_unchunked(dt, d, cuts, valid):
    outer, L, H = 2, 1000, 2
    q, k, v = tensors((outer, L, H, d), (outer, L, H, d), 1300 + d + len(cuts), dt, 2.0)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    bounds = [0, *cuts, L]
    acc_o, acc_l = empty((outer, L, H, d), dt == BF), lse_buf(outer, H, L)
    part_o, part_l = empty((outer, L, H, d), dt == BF), lse_buf(outer, H, L)
    for i, (a, b) in enumerate(zip(bounds, bounds[1:])):
        kc, vc = kd[:, a:b].contiguous(), vd[:, a:b].contiguous()
        nv = max(0, min(b, valid) - a)
        dst_o, dst_l = (acc_o, acc_l) if i == 0 else (part_o, part_l)
        st.st_attn_chunk(qd, kc, vc, outer, L, b - a, nv, H, d, scale, dt, dst_o, dst_l)
        if i > 0:   # running merge, in place into the accumulator
            st.st_attn_merge(acc_o, acc_l, part_o, part_l, outer, L, H, d, dt, acc_o, acc_l)
    sync()
    ro, rl = oracle.attn_chunk(f64(q), f64(k), f64(v), scale, valid)
    assert_close(f64(acc_o), ro, bf16=dt == BF, what="merged O")
    check_lse(acc_l, rl, dt, "merged lse")


# d = 40 (5 pieces a row, idle lanes in a pass), fp32 d = 72 (18 pieces), d = 520 (65 pieces: per-row lane
# groups), d = 5 (rows not 16-byte aligned: per-row lane groups, element by element)
@pytest.mark.parametrize("dt,d", [(BF, 72), (F32, 64), (BF, 40), (F32, 72), (BF, 520), (BF, 5)])
def test_merge_matches_oracle_including_empty_parts(dt, d):
    outer, L, H = 3, 77, 4
    sd = "bf16" if dt == BF else "f32"
    oa, ob = st_synth.randn((outer, L, H, d), 1500 + d, dtype=sd), st_synth.randn((outer, L, H, d), 1501 + d, dtype=sd)
    r = np.random.default_rng(1502 + d)
    la = r.normal(0.0, 4.0, (outer, H, L)).astype(np.float32)
    lb = r.normal(0.0, 4.0, (outer, H, L)).astype(np.float32)
    la[0, 0, :5] = -np.inf            # part a empty for some rows
    lb[1, 2, 3:9] = -np.inf           # part b empty for others
    la[2, 1, 10] = lb[2, 1, 10] = -np.inf   # both empty
    ta, tb = t_.from_numpy(la).cuda(), t_.from_numpy(lb).cuda()
    out, lse = empty((outer, L, H, d), dt == BF), lse_buf(outer, H, L)
    st.st_attn_merge(to_dev(oa), ta, to_dev(ob), tb, outer, L, H, d, dt, out, lse)
    sync()
    ro, rl = oracle.merge_chunks(f64(oa), la.astype(np.float64), f64(ob), lb.astype(np.float64))
    assert_close(f64(out), ro, bf16=dt == BF, what="merge O")
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(got[fin], rl[fin], rtol=1e-6, atol=1e-6)
    assert np.all(f64(out)[2, 10, 1] == 0.0)


def test_chunked_merge_at_1080p_frame_shape_sampled():
    # one 1080p frame (8160 patches x 16 heads x 72) in three uneven key chunks, merged;
    # checked against the oracle on a seeded sample of queries of every head
    L, H, d, outer = 8160, 16, 72, 1
    q, k, v = tensors((outer, L, H, d), (outer, L, H, d), 1700, BF)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    bounds = [0, 2000, 2001, L]
    acc_o, acc_l = empty((outer, L, H, d)), lse_buf(outer, H, L)
    part_o, part_l = empty((outer, L, H, d)), lse_buf(outer, H, L)
    for i, (a, b) in enumerate(zip(bounds, bounds[1:])):
        dst_o, dst_l = (acc_o, acc_l) if i == 0 else (part_o, part_l)
        st.st_attn_chunk(qd, kd[:, a:b].contiguous(), vd[:, a:b].contiguous(), outer, L, b - a, b - a, H, d, scale,
                         BF, dst_o, dst_l)
        if i > 0:
            st.st_attn_merge(acc_o, acc_l, part_o, part_l, outer, L, H, d, BF, acc_o, acc_l)
    sync()
    rows = np.random.default_rng(1701).choice(L, 48, replace=False)
    got_o, got_l = f64(acc_o), acc_l.cpu().numpy().astype(np.float64)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for h in range(H):
        ro, rl = oracle.attention_lse(qf[0, rows, h], kf[0, :, h], vf[0, :, h], scale)
        assert_close(got_o[0, rows, h], ro, what=f"head {h}")
        assert np.max(np.abs(got_l[0, h, rows] - rl)) <= lse_tol(rl, BF)


# --------------------------------------------------------------------------- #
# st_attn_chunk_acc: chunk attention merged into a running accumulator        #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dt,d,Lq,Lk,kv_valid", [(BF, 72, 300, 500, 480), (BF, 64, 70, 200, 150), (BF, 128, 100, 130, 130),
                                                 (F32, 64, 33, 40, 35)])
def test_chunk_acc_into_empty_accumulator_is_chunk(dt, d, Lq, Lk, kv_valid):
    # lse = -inf marks an empty accumulator: its rows are ignored, whatever they hold (NaN here)
    outer, H = 2, 2
    q, k, v = (to_dev(a) for a in tensors((outer, Lq, H, d), (outer, Lk, H, d), 1900 + d, dt))
    scale = 1.0 / math.sqrt(d)
    ref_o, ref_l = empty((outer, Lq, H, d), dt == BF), lse_buf(outer, H, Lq)
    st.st_attn_chunk(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dt, ref_o, ref_l)
    acc_o = t_.full((outer, Lq, H, d), float("nan"), dtype=ref_o.dtype, device="cuda")
    acc_l = t_.full((outer, H, Lq), -float("inf"), dtype=t_.float32, device="cuda")
    st.st_attn_chunk_acc(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dt, acc_o, acc_l)
    sync()
    assert t_.equal(acc_o, ref_o) and t_.equal(acc_l, ref_l)


@pytest.mark.parametrize("dt,d,cuts,valid", [
    (BF, 72, (300, 301), 950),        # three chunks, one of a single key, masked tail
    (BF, 128, (64, 500), 700),
    (BF, 64, (1,), 1000),
    (F32, 64, (100, 450), 999),
])
def test_chunk_acc_running_equals_unchunked(dt, d, cuts, valid):
    outer, L, H = 2, 1000, 2
    q, k, v = tensors((outer, L, H, d), (outer, L, H, d), 2000 + d + len(cuts), dt, 2.0)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    bounds = [0, *cuts, L]
    acc_o = empty((outer, L, H, d), dt == BF)
    acc_l = t_.full((outer, H, L), -float("inf"), dtype=t_.float32, device="cuda")
    # the same chunks through st_attn_chunk + st_attn_merge, for comparison
    m_o, m_l = empty((outer, L, H, d), dt == BF), lse_buf(outer, H, L)
    p_o, p_l = empty((outer, L, H, d), dt == BF), lse_buf(outer, H, L)
    for i, (a, b) in enumerate(zip(bounds, bounds[1:])):
        kc, vc = kd[:, a:b].contiguous(), vd[:, a:b].contiguous()
        nv = max(0, min(b, valid) - a)
        st.st_attn_chunk_acc(qd, kc, vc, outer, L, b - a, nv, H, d, scale, dt, acc_o, acc_l)
        dst_o, dst_l = (m_o, m_l) if i == 0 else (p_o, p_l)
        st.st_attn_chunk(qd, kc, vc, outer, L, b - a, nv, H, d, scale, dt, dst_o, dst_l)
        if i > 0:
            st.st_attn_merge(m_o, m_l, p_o, p_l, outer, L, H, d, dt, m_o, m_l)
    sync()
    ro, rl = oracle.attn_chunk(f64(q), f64(k), f64(v), scale, valid)
    assert_close(f64(acc_o), ro, bf16=dt == BF, what="accumulated O")
    check_lse(acc_l, rl, dt, "accumulated lse")
    # the fused merge rounds once per chunk where chunk + merge rounds twice: close, not identical
    assert_close(f64(acc_o), f64(m_o), bf16=dt == BF, what="fused vs chunk + merge")


def test_chunk_acc_empty_chunk_leaves_accumulator():
    outer, L, H, d = 2, 50, 2, 72
    q, k, v = (to_dev(a) for a in tensors((outer, L, H, d), (outer, 20, H, d), 2100, BF))
    acc_o, acc_l = empty((outer, L, H, d)), lse_buf(outer, H, L)
    st.st_attn_chunk(q, k, v, outer, L, 20, 20, H, d, 0.1, BF, acc_o, acc_l)
    before_o, before_l = acc_o.clone(), acc_l.clone()
    st.st_attn_chunk_acc(q, k, v, outer, L, 20, 0, H, d, 0.1, BF, acc_o, acc_l)   # kv_valid = 0
    sync()
    assert t_.equal(acc_o, before_o) and t_.equal(acc_l, before_l)


def test_chunk_acc_1080p_frame_sampled():
    # one 1080p frame in three uneven key chunks accumulated in place, checked on sampled queries
    L, H, d, outer = 8160, 16, 72, 1
    q, k, v = tensors((outer, L, H, d), (outer, L, H, d), 2200, BF)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    acc_o = empty((outer, L, H, d))
    acc_l = t_.full((outer, H, L), -float("inf"), dtype=t_.float32, device="cuda")
    for a, b in zip([0, 3000, 3001], [3000, 3001, L]):
        st.st_attn_chunk_acc(qd, kd[:, a:b].contiguous(), vd[:, a:b].contiguous(), outer, L, b - a, b - a, H, d, scale,
                             BF, acc_o, acc_l)
    sync()
    rows = np.random.default_rng(2201).choice(L, 48, replace=False)
    got_o, got_l = f64(acc_o), acc_l.cpu().numpy().astype(np.float64)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for h in range(H):
        ro, rl = oracle.attention_lse(qf[0, rows, h], kf[0, :, h], vf[0, :, h], scale)
        assert_close(got_o[0, rows, h], ro, what=f"head {h}")
        assert np.max(np.abs(got_l[0, h, rows] - rl)) <= lse_tol(rl, BF)
