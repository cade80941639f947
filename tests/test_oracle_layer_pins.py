"""Pins of the oracle's layer composition (CPU only).

oracle.spatial_layer, oracle.temporal_layer and oracle.block compose the step
functions that test_oracle_pins.py pins one by one.  Here each composition is
recomputed on tiny inputs by an independent formulation that shares no code
with the oracle and follows the pages' description of the layers directly:

  - ScaleFusion review, "Technical architecture" (layer table): the spatial
    layer attends over the S patches of each frame, the temporal layer over
    the T frames of each patch; the tensor goes [B,T,S,C] -> [B,S,T,C] between
    them and back afterwards.
  - CoCoDiff page, "V-First compute scheduling": linear projection to Q, K, V;
    RMSNorm then RoPE on Q and K only.

The formulation: projections as scalar dot products, the per-head RMS by an
explicit sum of squares, RoPE as complex multiplication of channel pairs with
the patch row h = s // W and column w = s % W (spatial) or the frame t
(temporal), softmax attention with the 1/sqrt(d) scale as explicit
exponentials without a max shift, relayouts as index loops.  It agrees with
the oracle to 1e-12.  The last section plants plausible mistakes in the
oracle (in its module, on the CPU) and checks that this pin catches each one.
"""
import cmath
import math

import numpy as np
import pytest

import oracle
from oracle import st_oracle

BASE, EPS = 10000.0, 1e-6


# --------------------------------------------------------------------------- #
# The independent formulation (pure Python loops)                              #
# --------------------------------------------------------------------------- #
def loop_project(xrow, w):
    """One token row times w^T: out[o] = sum_c w[o][c] * x[c]."""
    return [math.fsum(float(w[o, c]) * float(xrow[c]) for c in range(len(xrow))) for o in range(w.shape[0])]


def loop_rms(vec, g):
    ms = math.fsum(v * v for v in vec) / len(vec)
    inv = 1.0 / math.sqrt(ms + EPS)
    return [vec[j] * inv * float(g[j]) for j in range(len(vec))]


def complex_rotate(vec, p):
    """Pairs (2i, 2i+1) of one axis segment of length m, as complex numbers times exp(1j p base^(-2i/m))."""
    m = len(vec)
    out = []
    for i in range(m // 2):
        z = complex(vec[2 * i], vec[2 * i + 1]) * cmath.exp(1j * p * BASE ** (-2.0 * i / m))
        out += [z.real, z.imag]
    return out


def loop_qkv(xrow, w_qkv, g_q, g_k, H, d, positions):
    """q, k, v heads of one token; positions: one per axis segment ((t,) or (h, w))."""
    full = loop_project(xrow, w_qkv)
    nseg = len(positions)
    m = d // nseg
    heads = {}
    for part, name in enumerate("qkv"):
        hs = []
        for h in range(H):
            vec = full[part * H * d + h * d: part * H * d + (h + 1) * d]
            if name != "v":
                vec = loop_rms(vec, g_q if name == "q" else g_k)
                vec = sum((complex_rotate(vec[a * m:(a + 1) * m], positions[a]) for a in range(nseg)), [])
            hs.append(vec)
        heads[name] = hs
    return heads["q"], heads["k"], heads["v"]


def loop_attend(qs, ks, vs, d, n_valid):
    """softmax_j(q . k_j / sqrt(d)) v_j over keys j < n_valid, exponentials without a max shift."""
    out = []
    for q in qs:
        w = [math.exp(math.fsum(q[c] * k[c] for c in range(d)) / math.sqrt(d)) for k in ks[:n_valid]]
        tot = math.fsum(w)
        out.append([math.fsum(w[j] * vs[j][c] for j in range(n_valid)) / tot for c in range(d)])
    return out


def loop_layer(seqs, wts, H, d, n_valid):
    """seqs: list of sequences, each a list of (token row, positions); returns the output rows."""
    outs = []
    for seq in seqs:
        per_tok = [loop_qkv(row, wts["w_qkv"], wts["g_q"], wts["g_k"], H, d, pos) for row, pos in seq]
        o_rows = [[0.0] * (H * d) for _ in seq]
        for h in range(H):
            qs = [t[0][h] for t in per_tok]
            ks = [t[1][h] for t in per_tok]
            vs = [t[2][h] for t in per_tok]
            for i, o in enumerate(loop_attend(qs, ks, vs, d, n_valid)):
                o_rows[i][h * d:(h + 1) * d] = o
        outs.append([loop_project(o, wts["w_o"]) for o in o_rows])
    return outs


def loop_spatial(x, wts, H, d, W):
    """x [B,T,S,C] -> [B,T,S,C]: one sequence per (b, t) over the patches s, positions (s // W, s % W)."""
    B, T, S, C = x.shape
    y = np.zeros((B, T, S, wts["w_o"].shape[0]))
    for b in range(B):
        for t in range(T):
            seq = [(x[b, t, s], (s // W, s % W)) for s in range(S)]
            for s, row in enumerate(loop_layer([seq], wts, H, d, S)[0]):
                y[b, t, s] = row
    return y


def loop_temporal(x, wts, H, d, t_valid):
    """x [B,S,T,C] -> [B,S,T,C]: one sequence per (b, s) over the frames t, position t, keys t < t_valid."""
    B, S, T, C = x.shape
    y = np.zeros((B, S, T, wts["w_o"].shape[0]))
    for b in range(B):
        for s in range(S):
            seq = [(x[b, s, t], (t,)) for t in range(T)]
            for t, row in enumerate(loop_layer([seq], wts, H, d, t_valid)[0]):
                y[b, s, t] = row
    return y


def loop_swap_ts(x):
    """[B, A, Bx, C] -> [B, Bx, A, C] by index loops."""
    B, A, Bx, C = x.shape
    y = np.zeros((B, Bx, A, C))
    for b in range(B):
        for i in range(A):
            for j in range(Bx):
                for c in range(C):
                    y[b, j, i, c] = x[b, i, j, c]
    return y


def loop_block(x, ws, wt, H, d, W, t_valid):
    h = loop_spatial(x, ws, H, d, W)
    return loop_swap_ts(loop_temporal(loop_swap_ts(h), wt, H, d, t_valid))


# --------------------------------------------------------------------------- #
# Inputs: a non-square patch grid, two heads, non-uniform gains                #
# --------------------------------------------------------------------------- #
def inputs(seed, B=1, T=3, S=6, W=3, C=8, H=2, d=8, gain=1.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, S, C))
    mk = lambda: dict(w_qkv=0.4 * r.standard_normal((3 * H * d, C)), w_o=0.4 * r.standard_normal((C, H * d)),
                      g_q=gain * (1.0 + 0.2 * r.standard_normal(d)), g_k=gain * (1.0 + 0.2 * r.standard_normal(d)))
    return x, mk(), mk(), H, d, W


def close(a, b):
    return np.allclose(a, b, rtol=1e-12, atol=1e-12)


CASES = [dict(seed=300), dict(seed=301, B=2, T=2, S=6, W=2), dict(seed=302, T=4, S=4, W=4, d=4, H=3, C=12),
         dict(seed=303, gain=4.0)]


@pytest.mark.parametrize("case", CASES)
def test_spatial_layer_matches_loop_formulation(case):
    x, ws, _, H, d, W = inputs(**case)
    np.testing.assert_allclose(oracle.spatial_layer(x, ws, H, d, W, EPS, BASE), loop_spatial(x, ws, H, d, W),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("masked", [False, True])
def test_temporal_layer_matches_loop_formulation(case, masked):
    x, _, wt, H, d, _ = inputs(**case)
    xs = loop_swap_ts(x)
    T = x.shape[1]
    tv = T - 1 if masked else T
    got = oracle.temporal_layer(xs, wt, H, d, EPS, BASE, tv if masked else None)
    np.testing.assert_allclose(got, loop_temporal(xs, wt, H, d, tv), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES[:2])
def test_block_matches_loop_formulation(case):
    x, ws, wt, H, d, W = inputs(**case)
    T = x.shape[1]
    np.testing.assert_allclose(oracle.block(x, ws, wt, H, d, W, EPS, BASE, T - 1),
                               loop_block(x, ws, wt, H, d, W, T - 1), rtol=1e-12, atol=1e-12)


def test_loop_formulation_reduces_to_closed_forms():
    """The formulation itself: p = 0 leaves a pair alone, a pair at p rotates by p radians
    (first frequency), one key returns its value."""
    assert complex_rotate([1.0, 2.0, 3.0, 4.0], 0) == [1.0, 2.0, 3.0, 4.0]
    r = complex_rotate([1.0, 0.0], 0.5)
    assert abs(r[0] - math.cos(0.5)) < 1e-15 and abs(r[1] - math.sin(0.5)) < 1e-15
    assert loop_attend([[1.0, 2.0]], [[3.0, -1.0]], [[5.0, 6.0]], 2, 1) == [[5.0, 6.0]]


# --------------------------------------------------------------------------- #
# Planted mistakes: each one, put into the oracle module, fails the pins       #
# --------------------------------------------------------------------------- #
def spatial_mismatch(case):
    x, ws, _, H, d, W = inputs(**case)
    return not close(oracle.spatial_layer(x, ws, H, d, W, EPS, BASE), loop_spatial(x, ws, H, d, W))


def temporal_mismatch(case):
    x, _, wt, H, d, _ = inputs(**case)
    xs = loop_swap_ts(x)
    T = x.shape[1]
    return not close(oracle.temporal_layer(xs, wt, H, d, EPS, BASE, T - 1), loop_temporal(xs, wt, H, d, T - 1))


def test_unplanted_oracle_passes():
    assert not spatial_mismatch(CASES[0]) and not temporal_mismatch(CASES[0])


def test_planted_scale_one_over_d_is_caught(monkeypatch):
    sp, tp = st_oracle.attn_spatial, st_oracle.attn_temporal
    monkeypatch.setattr(st_oracle, "attn_spatial", lambda q, k, v, scale: sp(q, k, v, scale * scale))
    monkeypatch.setattr(st_oracle, "attn_temporal", lambda q, k, v, scale, tv=None: tp(q, k, v, scale * scale, tv))
    assert spatial_mismatch(CASES[0])
    assert temporal_mismatch(CASES[0])


def test_planted_1d_rope_in_spatial_layer_is_caught(monkeypatch):
    orig = st_oracle.qkv_norm_rope

    def one_d(x, w, gq, gk, eps, H, d, kind, pos, base):
        if kind == "2d":   # rotate by the token index s = h * W + w over all d channels
            W = int(pos[:, 1].max()) + 1
            return orig(x, w, gq, gk, eps, H, d, "1d", pos[:, 0] * W + pos[:, 1], base)
        return orig(x, w, gq, gk, eps, H, d, kind, pos, base)

    monkeypatch.setattr(st_oracle, "qkv_norm_rope", one_d)
    assert spatial_mismatch(CASES[0])


def test_planted_swapped_h_w_is_caught(monkeypatch):
    orig = st_oracle.positions_2d
    monkeypatch.setattr(st_oracle, "positions_2d", lambda S, W: orig(S, W)[:, ::-1].copy())
    assert spatial_mismatch(CASES[0])


def test_planted_row_major_over_height_is_caught(monkeypatch):
    """s = w * H_grid + h (column-major patch order) instead of s = h * W + w."""
    monkeypatch.setattr(st_oracle, "positions_2d",
                        lambda S, W: np.stack([np.arange(S) % (S // W), np.arange(S) // (S // W)], axis=1))
    assert spatial_mismatch(CASES[0])


def test_planted_repeat_instead_of_tile_positions_is_caught(monkeypatch):
    orig = st_oracle.qkv_norm_rope

    def repeated(x, w, gq, gk, eps, H, d, kind, pos, base):
        rows = x.shape[0]
        if kind == "2d":
            S = int(np.max(pos[:, 0] * (pos[:, 1].max() + 1) + pos[:, 1])) + 1
            base_pos = pos[:S]
            pos = np.repeat(base_pos, rows // S, axis=0)
        elif kind == "1d":
            T = int(pos.max()) + 1
            pos = np.repeat(np.arange(T), rows // T)
        return orig(x, w, gq, gk, eps, H, d, kind, pos, base)

    monkeypatch.setattr(st_oracle, "qkv_norm_rope", repeated)
    assert spatial_mismatch(CASES[0])
    assert temporal_mismatch(CASES[0])


def test_planted_unmasked_padding_is_caught(monkeypatch):
    tp = st_oracle.attn_temporal
    monkeypatch.setattr(st_oracle, "attn_temporal", lambda q, k, v, scale, tv=None: tp(q, k, v, scale, None))
    assert temporal_mismatch(CASES[0])


def test_planted_norm_on_v_is_caught(monkeypatch):
    orig = st_oracle.qkv_norm_rope

    def norm_v(x, w, gq, gk, eps, H, d, kind, pos, base):
        q, k, v = orig(x, w, gq, gk, eps, H, d, kind, pos, base)
        return q, k, st_oracle.rms_norm_heads(v, np.ones(d), eps)

    monkeypatch.setattr(st_oracle, "qkv_norm_rope", norm_v)
    assert spatial_mismatch(CASES[0])


def test_planted_reshape_instead_of_transpose_relayout_is_caught(monkeypatch):
    """[B,T,S,C] -> [B,S,T,C] done as a reshape (the bytes stay in [T,S] order)."""
    monkeypatch.setattr(st_oracle, "bt_to_bs", lambda x: x.reshape(x.shape[0], x.shape[2], x.shape[1], x.shape[3]))
    x, ws, wt, H, d, W = inputs(**CASES[0])
    T = x.shape[1]
    assert not close(oracle.block(x, ws, wt, H, d, W, EPS, BASE, T - 1), loop_block(x, ws, wt, H, d, W, T - 1))
