"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes one part of the oracle by a closed form, brute force on tiny
inputs written in a different formulation, a library routine, an invariant of
the mathematics, or a layout printed on the pages.  The last section plants
plausible mistakes in copies of oracle functions and checks that the pins
catch them.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

import oracle
import st_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- #
# Attention                                                                    #
# --------------------------------------------------------------------------- #
def brute_attention(q, k, v, scale, n_valid=None):
    """softmax(q k^T scale) v with scalar loops and no max subtraction."""
    Lq, d = q.shape
    Lk = k.shape[0]
    nv = Lk if n_valid is None else n_valid
    out = [[0.0] * v.shape[1] for _ in range(Lq)]
    for i in range(Lq):
        w = []
        for j in range(nv):
            s = 0.0
            for c in range(d):
                s += float(q[i, c]) * float(k[j, c])
            w.append(math.exp(s * scale))
        tot = sum(w)
        for j in range(nv):
            for c in range(v.shape[1]):
                out[i][c] += w[j] / tot * float(v[j, c])
    return np.array(out)


@pytest.mark.parametrize("L,d,seed", [(1, 3, 0), (4, 4, 1), (7, 5, 2), (5, 8, 3)])
def test_attention_matches_bruteforce(L, d, seed):
    r = rng(seed)
    q, k, v = r.standard_normal((3, L, d))
    scale = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(oracle.attention(q, k, v, scale), brute_attention(q, k, v, scale),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,nv", [(6, 3), (5, 1), (8, 7)])
def test_masked_attention_matches_bruteforce(L, nv):
    r = rng(10 + L)
    q, k, v = r.standard_normal((3, L, 4))
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.5, n_valid=nv),
                               brute_attention(q, k, v, 0.5, n_valid=nv), rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa_f64():
    torch = pytest.importorskip("torch")
    r = rng(5)
    q, k, v = r.standard_normal((3, 37, 9))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None]).numpy()[0]
    np.testing.assert_allclose(oracle.attention(q, k, v, 1.0 / math.sqrt(9)), ref, rtol=1e-12, atol=1e-13)


def test_softmax_rows_sum_to_one():
    r = rng(6)
    q, k = 3.0 * r.standard_normal((2, 50, 8))
    for nv in (None, 17):
        p = oracle.attention_probs(q, k, 0.35, n_valid=nv)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-14
        if nv is not None:
            assert np.all(p[:, nv:] == 0.0)


def test_single_key_returns_value():
    r = rng(7)
    q, k, v = r.standard_normal((3, 1, 6))
    np.testing.assert_array_equal(oracle.attention(q, k, v, 0.4), v)


def test_zero_query_gives_mean_of_values():
    r = rng(8)
    k, v = r.standard_normal((2, 11, 5))
    q = np.zeros((3, 5))
    np.testing.assert_allclose(oracle.attention(q, k, v, 1.0), np.tile(v.mean(axis=0), (3, 1)), rtol=1e-13)


def test_dominant_key_selects_its_value():
    r = rng(9)
    k = np.eye(6)[:4]                      # orthonormal keys
    v = r.standard_normal((4, 3))
    q = 200.0 * k[2:3]                     # scores 200 vs 0
    np.testing.assert_allclose(oracle.attention(q, k, v, 1.0), v[2:3], rtol=0, atol=1e-80)


def test_two_key_closed_form_uses_scale():
    d = 72
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((2, d)); k[0, 0] = 1.0     # score 1 * scale, and 0
    v = np.array([[1.0] + [0.0] * (d - 1), [0.0] * d])
    s = 1.0 / math.sqrt(d)
    want = math.exp(s) / (math.exp(s) + 1.0)
    assert abs(oracle.attention(q, k, v, s)[0, 0] - want) < 1e-15


def test_masked_keys_contribute_nothing():
    r = rng(11)
    q, k, v = r.standard_normal((3, 9, 4))
    k2, v2 = k.copy(), v.copy()
    k2[6:] = 1e3 * r.standard_normal((3, 4))
    v2[6:] = np.nan_to_num(np.full((3, 4), 1e300))
    np.testing.assert_array_equal(oracle.attention(q, k, v, 0.5, n_valid=6),
                                  oracle.attention(q, k2, v2, 0.5, n_valid=6))
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.5, n_valid=6),
                               oracle.attention(q, k[:6], v[:6], 0.5), rtol=1e-14)


def test_spatial_and_temporal_wrappers_are_per_sequence():
    r = rng(12)
    B, T, S, H, d = 1, 3, 5, 2, 4
    q, k, v = r.standard_normal((3, B, T, S, H, d))
    o = oracle.attn_spatial(q, k, v, 0.5)
    for t in range(T):
        for h in range(H):
            np.testing.assert_allclose(o[0, t, :, h], brute_attention(q[0, t, :, h], k[0, t, :, h],
                                                                      v[0, t, :, h], 0.5), rtol=1e-12)
    qt, kt, vt = (np.transpose(a, (0, 2, 1, 3, 4)) for a in (q, k, v))   # [B, S, T, H, d]
    ot = oracle.attn_temporal(qt, kt, vt, 0.5, t_valid=2)
    for s in range(S):
        for h in range(H):
            np.testing.assert_allclose(ot[0, s, :, h], brute_attention(qt[0, s, :, h], kt[0, s, :, h],
                                                                       vt[0, s, :, h], 0.5, n_valid=2),
                                       rtol=1e-12)


# --------------------------------------------------------------------------- #
# RMSNorm                                                                      #
# --------------------------------------------------------------------------- #
def test_rmsnorm_unit_mean_square_and_scale_invariance():
    r = rng(20)
    t = r.standard_normal((10, 3, 8))
    y = oracle.rms_norm_heads(t, np.ones(8), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_norm_heads(7.5 * t, np.ones(8), 0.0), y, rtol=1e-13)


def test_rmsnorm_zero_and_eps_closed_form():
    y = oracle.rms_norm_heads(np.zeros((2, 2, 4)), np.ones(4), 1e-6)
    assert np.all(y == 0.0)
    t = np.full((1, 1, 4), 1e-3)               # mean square 1e-6, so denominator sqrt(2e-6)
    np.testing.assert_allclose(oracle.rms_norm_heads(t, np.ones(4), 1e-6), 1e-3 / math.sqrt(2e-6), rtol=1e-14)


def test_rmsnorm_is_per_head_with_per_channel_gain():
    r = rng(21)
    t = r.standard_normal((4, 2, 6))
    g = np.arange(1, 7, dtype=float)
    base = oracle.rms_norm_heads(t, g, 1e-6)
    t2 = t.copy(); t2[:, 1] *= 100.0           # rescale head 1 only
    y2 = oracle.rms_norm_heads(t2, g, 1e-6)
    np.testing.assert_array_equal(y2[:, 0], base[:, 0])
    for j in range(6):                          # gain j multiplies channel j only
        np.testing.assert_allclose(base[..., j], g[j] * oracle.rms_norm_heads(t, np.ones(6), 1e-6)[..., j],
                                   rtol=1e-14)


# --------------------------------------------------------------------------- #
# RoPE                                                                         #
# --------------------------------------------------------------------------- #
def complex_rope(vec, p, base):
    """Reference in complex form: z_i = x_2i + i x_2i+1 multiplied by exp(i p base^(-2i/m))."""
    m = len(vec)
    out = []
    for i in range(m // 2):
        z = complex(vec[2 * i], vec[2 * i + 1]) * cmath.exp(1j * p * base ** (-2.0 * i / m))
        out += [z.real, z.imag]
    return np.array(out)


def test_rope_1d_matches_complex_form():
    r = rng(30)
    t = r.standard_normal((5, 2, 8))
    pos = np.array([0, 1, 3, 17, 50])
    y = oracle.rope(t, "1d", pos, 10000.0)
    for a in range(5):
        for h in range(2):
            np.testing.assert_allclose(y[a, h], complex_rope(t[a, h], pos[a], 10000.0), rtol=1e-13, atol=1e-15)


def test_rope_2d_axes_and_complex_form():
    r = rng(31)
    d = 12
    t = r.standard_normal((4, 1, d))
    pos = np.array([[0, 0], [0, 5], [3, 0], [2, 7]])
    y = oracle.rope(t, "2d", pos, 10000.0)
    np.testing.assert_array_equal(y[0], t[0])                       # (0, 0): identity
    np.testing.assert_array_equal(y[1, 0, :d // 2], t[1, 0, :d // 2])  # h = 0: first half untouched
    np.testing.assert_array_equal(y[2, 0, d // 2:], t[2, 0, d // 2:])  # w = 0: second half untouched
    for a in range(4):
        want = np.concatenate([complex_rope(t[a, 0, :d // 2], pos[a, 0], 10000.0),
                               complex_rope(t[a, 0, d // 2:], pos[a, 1], 10000.0)])
        np.testing.assert_allclose(y[a, 0], want, rtol=1e-13, atol=1e-15)


def test_rope_first_pair_rotates_by_position_radians():
    t = np.zeros((1, 1, 4)); t[0, 0, 0] = 1.0
    y = oracle.rope(t, "1d", np.array([2]), 10000.0)
    np.testing.assert_allclose(y[0, 0, :2], [math.cos(2.0), math.sin(2.0)], rtol=1e-15)
    t = np.zeros((1, 1, 4)); t[0, 0, 2] = 1.0                     # pair i = 1 of m = 4: base^(-1/2)
    y = oracle.rope(t, "1d", np.array([3]), 10000.0)
    np.testing.assert_allclose(y[0, 0, 2:], [math.cos(3 * 0.01), math.sin(3 * 0.01)], rtol=1e-14)


def test_rope_norm_composition_relative():
    r = rng(32)
    q, k = r.standard_normal((2, 1, 1, 16))
    rq = lambda x, p: oracle.rope(x, "1d", np.array([p]), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(rq(q, 9)), np.linalg.norm(q), rtol=1e-14)
    np.testing.assert_allclose(rq(rq(q, 4), 7), rq(q, 11), rtol=1e-12, atol=1e-14)
    a = float(np.sum(rq(q, 10) * rq(k, 3)))
    b = float(np.sum(rq(q, 27) * rq(k, 20)))
    np.testing.assert_allclose(a, b, rtol=1e-12)


# --------------------------------------------------------------------------- #
# Projection and the q/k/v split                                               #
# --------------------------------------------------------------------------- #
def test_qkv_split_order_and_v_bypass():
    r = rng(40)
    H, d, C, rows = 2, 4, 5, 3
    x = r.standard_normal((rows, C))
    w = r.standard_normal((3 * H * d, C))
    q, k, v = oracle.qkv_norm_rope(x, w, np.ones(d), np.ones(d), 1e-6, H, d, "none", None, 10000.0)
    for row in range(rows):
        for h in range(H):
            for j in range(d):
                c = h * d + j
                assert v[row, h, j] == pytest.approx(float(np.dot(x[row], w[2 * H * d + c])), rel=1e-13)
    # q and k are the normalised projections of their own thirds of w
    raw_q = np.array([[x[i] @ w[h * d:(h + 1) * d].T for h in range(H)] for i in range(rows)])
    raw_k = np.array([[x[i] @ w[H * d + h * d:H * d + (h + 1) * d].T for h in range(H)] for i in range(rows)])
    for raw, got in ((raw_q, q), (raw_k, k)):
        rms = np.sqrt(np.mean(raw ** 2, axis=-1, keepdims=True) + 1e-6)
        np.testing.assert_allclose(got, raw / rms, rtol=1e-13)


def test_norm_before_rope_on_q_and_k_only():
    r = rng(41)
    H, d, C, rows = 1, 8, 6, 4
    x = r.standard_normal((rows, C))
    w = r.standard_normal((3 * H * d, C))
    g = 1.0 + r.random(d)                       # non-uniform gain: norm/rope do not commute
    pos = np.array([1, 2, 3, 4])
    q, k, v = oracle.qkv_norm_rope(x, w, g, g, 1e-6, H, d, "1d", pos, 10000.0)
    raw = (x @ w.T).reshape(rows, 3, H, d)
    for i in range(rows):
        want = complex_rope(raw[i, 0, 0] * g / math.sqrt(np.mean(raw[i, 0, 0] ** 2) + 1e-6), pos[i], 10000.0)
        np.testing.assert_allclose(q[i, 0], want, rtol=1e-12)
    np.testing.assert_allclose(v[:, 0], raw[:, 2, 0], rtol=1e-13)


# --------------------------------------------------------------------------- #
# Relayouts                                                                    #
# --------------------------------------------------------------------------- #
def test_bt_to_bs_bruteforce_and_roundtrip():
    x = np.arange(2 * 4 * 6 * 3).reshape(2, 4, 6, 3)
    y = oracle.bt_to_bs(x)
    for b in range(2):
        for t in range(4):
            for s in range(6):
                for c in range(3):
                    assert y[b, s, t, c] == x[b, t, s, c]
    np.testing.assert_array_equal(oracle.bs_to_bt(y), x)


def test_blocked_bruteforce_and_roundtrip():
    B, T, S, C, nt, ns = 1, 4, 6, 3, 2, 3
    x = np.arange(B * T * S * C).reshape(B, T, S, C)
    xb = oracle.to_blocked(x, nt, ns)
    assert xb.shape == (B, nt, ns, T // nt, S // ns, C)
    for i in range(nt):
        for j in range(ns):
            for a in range(T // nt):
                for e in range(S // ns):
                    for c in range(C):
                        assert xb[0, i, j, a, e, c] == x[0, i * (T // nt) + a, j * (S // ns) + e, c]
    np.testing.assert_array_equal(oracle.from_blocked(xb), x)


def test_layouts_match_the_pages():
    with open(os.path.join(GOLDEN, "page_layouts.json")) as f:
        g = json.load(f)
    B, T, S, C, P = 1, 8, 12, 5, 1
    hp = g["hyperparameters"]
    N_T, N_S = hp["N_T"], hp["N_S"]
    env = {"B": B, "T": T, "S": S, "C": C, "P": P, "N_T": N_T, "N_S": N_S}
    shape = lambda names: tuple(int(eval(n.replace("/", "//"), {}, env)) for n in names)
    x = np.zeros((B, T, S, C))
    assert x.shape == shape(g["layer_layouts"]["spatial_input"])
    assert oracle.bt_to_bs(x).shape[0] == B and oracle.bt_to_bs(x).shape[2] == T
    assert oracle.to_blocked(x, N_T, N_S).shape == shape(g["sliced_layouts"]["x_blocked"])
    assert oracle.to_blocked(x, N_T, N_S).shape == shape(g["sliced_layouts"]["y_blocked"])
    assert oracle.from_blocked(oracle.to_blocked(x, N_T, N_S)).shape == shape(g["sliced_layouts"]["output"])


# --------------------------------------------------------------------------- #
# Layers, independence, the sliced schedule                                    #
# --------------------------------------------------------------------------- #
def small_block_inputs(seed, B=1, T=4, S=12, grid_w=4, C=16, H=2, d=8):
    r = rng(seed)
    x = r.standard_normal((B, T, S, C))
    mk = lambda: dict(w_qkv=0.3 * r.standard_normal((3 * H * d, C)), w_o=0.3 * r.standard_normal((C, H * d)),
                      g_q=1.0 + 0.1 * r.standard_normal(d), g_k=1.0 + 0.1 * r.standard_normal(d))
    return x, mk(), mk(), dict(H=H, d=d, grid_w=grid_w, eps=1e-6, base=10000.0)


def test_spatial_layer_independent_across_frames():
    x, ws, _, p = small_block_inputs(50)
    y = oracle.spatial_layer(x, ws, p["H"], p["d"], p["grid_w"], p["eps"], p["base"])
    x2 = x.copy(); x2[:, 1] += 5.0
    y2 = oracle.spatial_layer(x2, ws, p["H"], p["d"], p["grid_w"], p["eps"], p["base"])
    np.testing.assert_array_equal(y2[:, [0, 2, 3]], y[:, [0, 2, 3]])
    assert not np.allclose(y2[:, 1], y[:, 1])


def test_temporal_layer_independent_across_patches():
    x, _, wt, p = small_block_inputs(51)
    xs = oracle.bt_to_bs(x)
    y = oracle.temporal_layer(xs, wt, p["H"], p["d"], p["eps"], p["base"])
    x2 = xs.copy(); x2[:, 3] -= 2.0
    y2 = oracle.temporal_layer(x2, wt, p["H"], p["d"], p["eps"], p["base"])
    keep = [s for s in range(xs.shape[1]) if s != 3]
    np.testing.assert_array_equal(y2[:, keep], y[:, keep])


@pytest.mark.parametrize("n_t,n_s", [(1, 1), (2, 3), (4, 4), (4, 2)])
def test_sliced_equals_unsliced(n_t, n_s):
    x, ws, wt, p = small_block_inputs(60, T=4, S=12)
    a = oracle.block(x, ws, wt, p["H"], p["d"], p["grid_w"], p["eps"], p["base"])
    b = oracle.block_sliced(x, ws, wt, p["H"], p["d"], p["grid_w"], p["eps"], p["base"], n_t, n_s)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)


def test_padded_masked_sliced_equals_unpadded():
    x, ws, wt, p = small_block_inputs(61, T=3, S=8, grid_w=4)
    a = oracle.block(x, ws, wt, p["H"], p["d"], p["grid_w"], p["eps"], p["base"])
    xp = np.concatenate([x, np.zeros_like(x[:, :1])], axis=1)       # T = 4, zero frame at t = 3
    b = oracle.block_sliced(xp, ws, wt, p["H"], p["d"], p["grid_w"], p["eps"], p["base"], 2, 2, t_valid=3)
    np.testing.assert_allclose(b[:, :3], a, rtol=1e-12, atol=1e-14)
    # without the mask the zero frame's key changes the result
    c = oracle.block_sliced(xp, ws, wt, p["H"], p["d"], p["grid_w"], p["eps"], p["base"], 2, 2)
    assert not np.allclose(c[:, :3], a)


def test_zero_frame_through_spatial_layer_is_zero():
    x, ws, _, p = small_block_inputs(62)
    x[:, 2] = 0.0
    y = oracle.spatial_layer(x, ws, p["H"], p["d"], p["grid_w"], p["eps"], p["base"])
    assert np.all(y[:, 2] == 0.0)


def test_tiny_config_block_runs_on_synthetic_inputs():
    inp = st_synth.make_inputs(1)
    c = inp["cfg"]
    x = st_synth.to_f64(inp["x"])
    ws = dict(w_qkv=st_synth.to_f64(inp["w_qkv_s"]), w_o=st_synth.to_f64(inp["w_o_s"]), g_q=inp["g_q"], g_k=inp["g_k"])
    wt = dict(w_qkv=st_synth.to_f64(inp["w_qkv_t"]), w_o=st_synth.to_f64(inp["w_o_t"]), g_q=inp["g_q"], g_k=inp["g_k"])
    y = oracle.block(x, ws, wt, c["H"], c["d"], c["grid_w"], st_synth.EPS, st_synth.ROPE_BASE)
    ys = oracle.block_sliced(x, ws, wt, c["H"], c["d"], c["grid_w"], st_synth.EPS, st_synth.ROPE_BASE, 2, 2)
    assert y.shape == x.shape and np.all(np.isfinite(y))
    np.testing.assert_allclose(ys, y, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- #
# Attention over key chunks and the merge of partial results (R5)             #
# --------------------------------------------------------------------------- #
def brute_lse(q, k, scale, n_valid=None):
    """log sum_j exp(scale * q_i . k_j) with scalar loops and an exact sum."""
    nv = k.shape[0] if n_valid is None else n_valid
    out = []
    for i in range(q.shape[0]):
        terms = [math.exp(scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(q.shape[1])))
                 for j in range(nv)]
        out.append(math.log(math.fsum(terms)) if terms else -math.inf)
    return np.array(out)


@pytest.mark.parametrize("Lq,Lk,nv", [(3, 5, None), (4, 1, None), (2, 6, 4), (5, 7, 1)])
def test_chunk_attention_and_lse_match_bruteforce(Lq, Lk, nv):
    r = rng(80 + Lk)
    q, k, v = r.standard_normal((Lq, 6)), r.standard_normal((Lk, 6)), r.standard_normal((Lk, 6))
    o, lse = oracle.attention_lse(q, k, v, 0.4, nv)
    np.testing.assert_allclose(o, brute_attention(q, k, v, 0.4, nv), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, brute_lse(q, k, 0.4, nv), rtol=1e-13, atol=1e-13)


def test_lse_closed_forms():
    r = rng(81)
    q, k, v = r.standard_normal((3, 5)), r.standard_normal((1, 5)), r.standard_normal((1, 5))
    _, lse = oracle.attention_lse(q, k, v, 0.7)                       # one key: lse = scale q.k
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), rtol=1e-14)
    kk = r.standard_normal((9, 5))
    _, lse = oracle.attention_lse(np.zeros((2, 5)), kk, kk, 0.7)      # q = 0: every score 0 -> log L
    np.testing.assert_allclose(lse, np.log(9.0), rtol=1e-14)
    same = np.repeat(k, 6, axis=0)                                   # L equal keys: scale q.k + log L
    _, lse = oracle.attention_lse(q, same, same, 0.7)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]) + np.log(6.0), rtol=1e-13)


@pytest.mark.parametrize("cuts", [(3,), (1, 4), (2, 3, 7, 8)])
def test_chunked_then_merged_equals_unchunked(cuts):
    r = rng(82)
    L, d = 11, 7
    q, k, v = r.standard_normal((4, d)), r.standard_normal((L, d)), r.standard_normal((L, d))
    scale = 1.0 / math.sqrt(d)
    bounds = [0, *cuts, L]
    parts = [oracle.attention_lse(q, k[a:b], v[a:b], scale) for a, b in zip(bounds, bounds[1:])]
    o, lse = parts[0]
    for po, pl in parts[1:]:                                         # left to right
        o, lse = oracle.merge_partials(o, lse, po, pl)
    np.testing.assert_allclose(o, brute_attention(q, k, v, scale), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, brute_lse(q, k, scale), rtol=1e-13, atol=1e-13)
    o2, lse2 = parts[-1]
    for po, pl in reversed(parts[:-1]):                              # right to left, swapped operands
        o2, lse2 = oracle.merge_partials(po, pl, o2, lse2)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_merge_with_empty_chunk_is_identity():
    r = rng(83)
    q, k, v = r.standard_normal((3, 4)), r.standard_normal((5, 4)), r.standard_normal((5, 4))
    o, lse = oracle.attention_lse(q, k, v, 0.5)
    eo, el = oracle.attention_lse(q, k, v, 0.5, n_valid=0)
    assert np.all(eo == 0.0) and np.all(np.isneginf(el))
    mo, ml = oracle.merge_partials(o, lse, eo, el)
    assert np.array_equal(mo, o) and np.array_equal(ml, lse)
    mo, ml = oracle.merge_partials(eo, el, o, lse)
    assert np.array_equal(mo, o) and np.array_equal(ml, lse)
    zo, zl = oracle.merge_partials(eo, el, eo, el)
    assert np.all(zo == 0.0) and np.all(np.isneginf(zl))


def test_chunk_wrappers_are_per_sequence_with_head_major_lse():
    r = rng(84)
    q = r.standard_normal((2, 3, 2, 4))
    k, v = r.standard_normal((2, 5, 2, 4)), r.standard_normal((2, 5, 2, 4))
    o, lse = oracle.attn_chunk(q, k, v, 0.5, kv_valid=4)
    assert o.shape == (2, 3, 2, 4) and lse.shape == (2, 2, 3)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(o[b, :, h], brute_attention(q[b, :, h], k[b, :, h], v[b, :, h], 0.5, 4),
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], brute_lse(q[b, :, h], k[b, :, h], 0.5, 4), rtol=1e-13)
    o1, l1 = oracle.attn_chunk(q, k[:, :2], v[:, :2], 0.5)
    o2, l2 = oracle.attn_chunk(q, k[:, 2:], v[:, 2:], 0.5, kv_valid=2)
    mo, ml = oracle.merge_chunks(o1, l1, o2, l2)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, lse, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- #
# All-to-all between the patch-sharded and frame-sharded layouts              #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("B,T,S,C,P", [(1, 4, 6, 3, 2), (2, 6, 6, 2, 3), (1, 8, 4, 5, 4), (2, 3, 5, 2, 1)])
def test_a2a_redistributes_by_index(B, T, S, C, P):
    x = rng(90 + P).standard_normal((B, T, S, C))
    tp, sp = T // P, S // P
    out = oracle.a2a_s_to_t([x[:, :, r * sp:(r + 1) * sp] for r in range(P)])
    for q in range(P):                                 # rank q: frames q*T/P .. of every patch
        assert out[q].shape == (B, tp, S, C)
        for b in range(B):
            for t in range(tp):
                for s in range(S):
                    for c in range(C):
                        assert out[q][b, t, s, c] == x[b, q * tp + t, s, c]
    back = oracle.a2a_t_to_s(out)
    for r in range(P):
        assert np.array_equal(back[r], x[:, :, r * sp:(r + 1) * sp])


def test_all_to_all_is_a_block_transpose():
    send = [[(r, q) for q in range(3)] for r in range(3)]
    recv = oracle.all_to_all(send)
    assert all(recv[q][r] == (r, q) for r in range(3) for q in range(3))


# --------------------------------------------------------------------------- #
# V-Major change detection (R6)                                               #
# --------------------------------------------------------------------------- #
def test_v_change_by_loops_and_special_cases():
    r = rng(95)
    rows, H, d = 5, 3, 4
    vn, vc = r.standard_normal((rows, H, d)), r.standard_normal((rows, H, d))
    vc[1, 2] = vn[1, 2]                                      # unchanged vector
    vc[3, 0] = vn[3, 0] + np.array([0.5, -0.25, 0.0, 0.25])  # distance exactly 1.0
    dist, mask, idx, cache = oracle.v_change(vn, vc, 1.0)
    for i in range(rows):
        for h in range(H):
            want = math.fsum(abs(float(vn[i, h, j]) - float(vc[i, h, j])) for j in range(d))
            assert dist[i, h] == pytest.approx(want, rel=1e-15, abs=0)
            assert mask[i, h] == (want > 1.0)
            assert np.array_equal(cache[i, h], vn[i, h] if want > 1.0 else vc[i, h])
    assert dist[1, 2] == 0.0 and not mask[1, 2]
    assert dist[3, 0] == 1.0 and not mask[3, 0]               # strictly greater than the threshold
    assert list(idx) == [i * H + h for i in range(rows) for h in range(H) if mask[i, h]]
    _, m0, _, c0 = oracle.v_change(vn, vc, 0.0)                 # threshold 0: every changed vector
    assert m0.sum() == rows * H - 1 and np.array_equal(c0, vn)
    _, mi, ii, ci = oracle.v_change(vn, vc, math.inf)          # infinite threshold: nothing moves
    assert not mi.any() and ii.size == 0 and np.array_equal(ci, vc)


# --------------------------------------------------------------------------- #
# Planted mistakes: each must be caught by a pin above                         #
# --------------------------------------------------------------------------- #
def test_pins_catch_rope_sign_error():
    t = rng(70).standard_normal((1, 1, 8))

    def bad(tt, pos, base):          # rotation in the wrong direction
        m = tt.shape[-1]
        th = pos[0] * base ** (-2.0 * np.arange(m // 2) / m)
        a, b = tt[..., 0::2], tt[..., 1::2]
        o = np.empty_like(tt); o[..., 0::2] = a * np.cos(th) + b * np.sin(th); o[..., 1::2] = -a * np.sin(th) + b * np.cos(th)
        return o
    assert not np.allclose(bad(t, np.array([3]), 10000.0)[0, 0], complex_rope(t[0, 0], 3, 10000.0))


def test_pins_catch_missing_scale_and_transposed_projection():
    r = rng(71)
    q, k, v = r.standard_normal((3, 5, 4))
    assert not np.allclose(oracle.attention(q, k, v, 1.0), brute_attention(q, k, v, 0.5))
    x = r.standard_normal((3, 4)); w = r.standard_normal((4, 4))
    assert not np.allclose(x @ w, oracle.linear(x, w))           # x.W vs x.W^T differ


def test_pins_catch_norm_over_wrong_axis():
    t = rng(72).standard_normal((4, 2, 6))
    t[:, 1] *= 100.0
    over_c = t / np.sqrt(np.mean(t.reshape(4, -1) ** 2, axis=-1))[:, None, None]
    assert not np.allclose(over_c[:, 0], oracle.rms_norm_heads(t, np.ones(6), 0.0)[:, 0])


def test_pins_catch_wrong_merges():
    r = rng(73)
    q, k, v = r.standard_normal((3, 5)), r.standard_normal((8, 5)), r.standard_normal((8, 5))
    full = brute_attention(q, k, v, 0.5)
    (oa, la), (ob, lb) = oracle.attention_lse(q, k[:3], v[:3], 0.5), oracle.attention_lse(q, k[3:], v[3:], 0.5)
    assert not np.allclose((oa + ob) / 2, full)                                  # plain average
    assert not np.allclose(np.where((la > lb)[:, None], oa, ob), full)           # winner takes all
    wa, wb = np.exp(la)[:, None], np.exp(lb)[:, None]
    assert not np.allclose(wa * oa + wb * ob, full)                              # weights not normalised
    assert np.allclose((wa * oa + wb * ob) / (wa + wb), full)                    # the merge itself
