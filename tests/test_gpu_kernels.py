"""Kernel-level parity: each C-ABI entry point on the GPU against the fp64 oracle.

Inputs are seeded (st_synth), identical bytes on both sides.  Shapes span
several tiles with ragged tails (L not a multiple of 64 or 256, T = 51/52,
rows not a multiple of 128) plus the degenerate cases (L = 1, T = 1).
"""
import math

import numpy as np
import pytest

import oracle
import st_synth
from helpers import assert_close, empty, f64, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

t_ = torch()
if not t_.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import temporal_attention_amd as st  # noqa: E402

BF, F32 = st.ST_BF16, st.ST_F32


def sync():
    t_.cuda.synchronize()


# --------------------------------------------------------------------------- #
# Relayout: bit-exact                                                          #
# --------------------------------------------------------------------------- #
NP_T = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64, 16: np.dtype((np.void, 16))}


def run_relayout(src_np, dims, sstr, dstr, dst_elems, eb):
    """Upload src (flat array of element type), run st_relayout, return dst and expected."""
    src = t_.from_numpy(np.frombuffer(src_np.tobytes(), dtype=np.uint8).copy()).cuda()
    dst = t_.full((dst_elems * eb,), 0xA5, dtype=t_.uint8, device="cuda")
    st.st_relayout(src, sstr, dst, dstr, dims, len(dims), eb)
    sync()
    got = np.frombuffer(dst.cpu().numpy().tobytes(), dtype=NP_T[eb])
    exp = np.frombuffer(np.full(dst_elems * eb, 0xA5, np.uint8).tobytes(), dtype=NP_T[eb]).copy()
    idx = np.indices(dims).reshape(len(dims), -1)
    so = (np.asarray(sstr)[:, None] * idx).sum(0)
    do = (np.asarray(dstr)[:, None] * idx).sum(0)
    exp[do] = src_np[so]
    return got, exp


def contiguous_strides(shape):
    s = [1] * len(shape)
    for i in range(len(shape) - 2, -1, -1):
        s[i] = s[i + 1] * shape[i + 1]
    return s


@pytest.mark.parametrize("B,T,S,C,eb", [(1, 5, 37, 1152, 2), (2, 4, 6, 24, 4), (1, 51, 13, 72, 2), (1, 3, 7, 5, 2),
                                        (1, 2, 3, 8, 1), (1, 3, 4, 6, 8), (1, 2, 5, 3, 16)])
def test_relayout_bt_to_bs(B, T, S, C, eb):
    rng = np.random.default_rng(B * 1000 + T * 100 + S + C)
    n = B * T * S * C
    src = np.frombuffer(rng.integers(0, 256, n * eb, dtype=np.uint8).tobytes(), dtype=NP_T[eb])
    sstr = contiguous_strides([B, T, S, C])
    dstr = [S * T * C, C, T * C, 1]
    got, exp = run_relayout(src, [B, T, S, C], sstr, dstr, n, eb)
    assert got.tobytes() == exp.tobytes()
    if eb == 2:   # and it is exactly the oracle's index map
        want = oracle.bt_to_bs(src.reshape(B, T, S, C)).reshape(-1)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("T,S,C,nt,ns", [(8, 12, 16, 2, 3), (52, 40, 72, 4, 4), (4, 6, 1152, 4, 2)])
def test_relayout_blocked_matches_oracle(T, S, C, nt, ns):
    rng = np.random.default_rng(T + S + C)
    x = rng.integers(0, 65536, (1, T, S, C), dtype=np.uint16)
    tt, ss = T // nt, S // ns
    dims = [1, nt, tt, ns, ss, C]
    sx = [T * S * C, tt * S * C, S * C, ss * C, C, 1]
    bstr = contiguous_strides([1, nt, ns, tt, ss, C])
    db = [bstr[0], bstr[1], bstr[3], bstr[2], bstr[4], 1]
    got, _ = run_relayout(x.reshape(-1), dims, sx, db, x.size, 2)
    assert np.array_equal(got, oracle.to_blocked(x, nt, ns).reshape(-1))
    # and back
    back, _ = run_relayout(got, dims, db, sx, x.size, 2)
    assert np.array_equal(back, x.reshape(-1))


@pytest.mark.parametrize("shape,perm,eb", [((5, 7, 3), (2, 1, 0), 2), ((4, 9), (1, 0), 4), ((3, 4, 5, 6), (3, 0, 2, 1), 1),
                                           ((1 << 20,), (0,), 2), ((2, 1, 3), (1, 2, 0), 2)])
def test_relayout_general_permutations(shape, perm, eb):
    rng = np.random.default_rng(len(shape) * 7 + eb)
    n = int(np.prod(shape))
    src = np.frombuffer(rng.integers(0, 256, n * eb, dtype=np.uint8).tobytes(), dtype=NP_T[eb])
    out_shape = [shape[p] for p in perm]
    ostr = contiguous_strides(out_shape)
    dstr = [0] * len(shape)
    for j, p in enumerate(perm):
        dstr[p] = ostr[j]
    got, exp = run_relayout(src, list(shape), contiguous_strides(list(shape)), dstr, n, eb)
    assert got.tobytes() == exp.tobytes()
    assert np.array_equal(got.reshape(out_shape), np.transpose(src.reshape(shape), perm))


# Few long rows, cut into 2-8 KB pieces: a contiguous block whose row count is not a power of two,
# a pack-like permutation of long rows (the all-to-all pack of 8 ranks, scaled down), rows whose
# byte length is not a multiple of 16 (left whole), and a row length with no 2-8 KB divisor.
@pytest.mark.parametrize("shape,perm,eb", [((3 * 5 * 17 * 64 * 8,), (0,), 2), ((4, 3, 6, 2040), (1, 0, 2, 3), 2),
                                           ((2, 3, 4099), (1, 0, 2), 4), ((2, 5, 3 * 4097), (1, 0, 2), 2),
                                           ((3, 2062 * 8), (0, 1), 2)])   # no 2-8 KB divisor: halved once
def test_relayout_long_rows(shape, perm, eb):
    test_relayout_general_permutations(shape, perm, eb)


def test_relayout_empty_is_noop():
    src = t_.zeros(16, dtype=t_.uint8, device="cuda")
    dst = t_.full((16,), 7, dtype=t_.uint8, device="cuda")
    st.st_relayout(src, [4, 1], dst, [1, 4], [0, 4], 2, 1)
    sync()
    assert bool((dst == 7).all())


# --------------------------------------------------------------------------- #
# RoPE table                                                                   #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("d,kind,npos", [(72, st.ST_ROPE_2D, 120), (72, st.ST_ROPE_1D, 52), (128, st.ST_ROPE_2D, 256),
                                         (64, st.ST_ROPE_1D, 5)])
def test_rope_table(d, kind, npos):
    n = st.st_rope_table_floats(d, kind, npos)
    tab = t_.empty(n, dtype=t_.float32, device="cuda")
    st.st_rope_table(d, kind, 10000.0, npos, tab)
    sync()
    m = d // 2 if kind == st.ST_ROPE_2D else d
    i = np.arange(m // 2)
    theta = np.arange(npos)[:, None] * 10000.0 ** (-2.0 * i / m)
    want = np.stack([np.cos(theta), np.sin(theta)], -1).astype(np.float32).reshape(-1)
    got = tab.cpu().numpy()
    assert np.max(np.abs(got.astype(np.float64) - want)) <= 1.2e-7


# --------------------------------------------------------------------------- #
# QKV projection + RMSNorm + RoPE                                              #
# --------------------------------------------------------------------------- #
def rope_positions(rows, kind, period, offset, grid_w):
    i = np.arange(rows) % period + offset
    if kind == st.ST_ROPE_2D:
        return np.stack([i // grid_w, i % grid_w], 1)
    return i


QKV_CASES = [
    # rows, C, H, d, kind, period, offset, grid_w, dtype, q_scale, explicit positions
    (300, 1152, 16, 72, st.ST_ROPE_2D, 100, 0, 10, BF, 1.0, False),
    (130, 1152, 16, 72, st.ST_ROPE_1D, 51, 0, 0, BF, 1.0, False),
    (257, 1152, 16, 72, st.ST_ROPE_NONE, 1, 0, 0, BF, 1.0, False),
    (200, 384, 3, 128, st.ST_ROPE_2D, 65536, 40000, 256, BF, 1.0, False),
    (150, 128, 2, 64, st.ST_ROPE_2D, 64, 0, 8, BF, 1.0, False),
    (64, 128, 2, 64, st.ST_ROPE_2D, 64, 0, 8, F32, 1.0, False),
    (77, 96, 3, 36, st.ST_ROPE_1D, 10, 3, 0, F32, 1.0, False),
    (300, 1152, 16, 72, st.ST_ROPE_2D, 100, 0, 10, BF, 0.17, False),   # q stored scaled
    (77, 96, 3, 36, st.ST_ROPE_1D, 10, 3, 0, F32, 0.17, False),
    # positions from a caller array, in no periodic order
    (300, 1152, 16, 72, st.ST_ROPE_2D, 0, 0, 0, BF, 1.0, True),
    (130, 1152, 16, 72, st.ST_ROPE_1D, 0, 0, 0, BF, 1.0, True),
    (200, 384, 3, 128, st.ST_ROPE_2D, 0, 0, 0, BF, 1.0, True),
    (64, 128, 2, 64, st.ST_ROPE_2D, 0, 0, 0, F32, 1.0, True),
]


@pytest.mark.parametrize("rows,C,H,d,kind,period,offset,grid_w,dt,q_scale,explicit", QKV_CASES)
def test_qkv_norm_rope(rows, C, H, d, kind, period, offset, grid_w, dt, q_scale, explicit):
    sd = "bf16" if dt == BF else "f32"
    x = st_synth.randn((rows, C), 11 + rows, dtype=sd)
    w = st_synth.randn((3 * H * d, C), 12 + rows, std=0.02, dtype=sd)
    rng = np.random.default_rng(rows)
    g_q = (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    g_k = (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    pos_dev = None
    if explicit:   # random positions: 1D frames up to 500, 2D rows/columns up to 300
        hi = 500 if kind == st.ST_ROPE_1D else 300
        pos2 = rng.integers(0, hi, size=(rows, 2)).astype(np.int32)
        if kind == st.ST_ROPE_1D:
            pos2[:, 1] = 0
        pos = pos2[:, 0] if kind == st.ST_ROPE_1D else pos2
        pos_dev = t_.from_numpy(pos2).cuda()
        npos = hi
    else:
        pos = rope_positions(rows, kind, period, offset, grid_w)
        npos = int(pos.max()) + 1 if kind != st.ST_ROPE_NONE else 1
    tab = None
    if kind != st.ST_ROPE_NONE:
        tab = t_.empty(st.st_rope_table_floats(d, kind, npos), dtype=t_.float32, device="cuda")
        st.st_rope_table(d, kind, 10000.0, npos, tab)
    q, k, v = (empty((rows, H, d), dt == BF) for _ in range(3))
    st.st_qkv_norm_rope(to_dev(x), rows, C, to_dev(w), to_dev(g_q), to_dev(g_k), 1e-6, q_scale, kind, tab, npos,
                        pos_dev, period, offset, grid_w, H, d, dt, q, k, v)
    sync()
    rk = {st.ST_ROPE_NONE: "none", st.ST_ROPE_1D: "1d", st.ST_ROPE_2D: "2d"}[kind]
    oq, ok, ov = oracle.qkv_norm_rope(f64(x), f64(w), g_q.astype(np.float64) * q_scale, g_k, 1e-6, H, d, rk, pos,
                                      10000.0)
    for name, got, ref in (("q", q, oq), ("k", k, ok), ("v", v, ov)):
        assert_close(f64(got), ref, bf16=dt == BF, what=name)


def test_qkv_zero_rows_is_noop():
    q = empty((1, 16, 72))
    q.fill_(3.0)
    dummy = empty((8, 1152))
    w = empty((3 * 16 * 72, 1152))
    g = t_.ones(72, device="cuda")
    st.st_qkv_norm_rope(dummy, 0, 1152, w, g, g, 1e-6, 1.0, st.ST_ROPE_NONE, None, 0, None, 1, 0, 0, 16, 72, BF, q,
                        empty((1, 16, 72)), empty((1, 16, 72)))
    sync()
    assert bool((q.float() == 3.0).all())


def test_empty_calls_return_ok_and_write_nothing():
    """Zero sequences, zero-length sequences and zero rows: every call returns ST_OK (the binding
    raises otherwise) and leaves a sentinel-filled output untouched; V-Major reports 0 active."""
    H, d, C = 16, 72, 1152
    src = empty((64, H, d))
    w = empty((C, H * d))
    out = empty((64, C))
    out.fill_(5.0)
    ws = t_.empty(1 << 20, dtype=t_.uint8, device="cuda")
    for B, T, S in ((0, 3, 100), (1, 0, 100), (1, 3, 0)):
        st.st_attn_spatial(src, src, src, B, T, S, H, d, 0.1, BF, None, 0, out)
        st.st_attn_spatial(src, src, src, B, T, S, H, d, 0.1, BF, w, C, out, ws, ws.numel())
        st.st_attn_temporal(src, src, src, B, S, T, T, H, d, 0.1, BF, None, 0, out)
    st.st_out_proj(src, 0, H * d, w, C, BF, out)
    st.st_out_proj_relayout(src, 0, H * d, w, C, BF, 4, 5, out)
    lse = t_.full((64,), 7.0, device="cuda")
    st.st_attn_chunk(src, src, src, 1, 0, 50, 50, H, d, 0.1, BF, out, lse)
    st.st_attn_merge(src, lse, src, lse, 0, 50, H, d, BF, out, lse)
    mask = t_.full((64,), 9, dtype=t_.uint8, device="cuda")
    cnt = t_.full((1,), 123, dtype=t_.int64, device="cuda")
    st.st_v_change(src, empty((64, H, d)), 0, H, d, 1.0, BF, mask, None, cnt, 1)
    sync()
    assert bool((out.float() == 5.0).all())
    assert bool((lse == 7.0).all()) and bool((mask == 9).all())
    assert int(cnt.item()) == 0


# --------------------------------------------------------------------------- #
# Output projection                                                            #
# --------------------------------------------------------------------------- #
# The bf16 projection runs one workgroup per CU over its tiles once there are more tiles than
# CUs: 51,277 ragged rows (804 tiles, ~3 per workgroup), a single K step per tile (K = 64,
# 300 tiles), and 100 outputs (rows not 16-byte aligned: the 8-byte store path, 274 tiles).
@pytest.mark.parametrize("rows,K,N,dt", [(300, 1152, 1152, BF), (129, 384, 384, BF), (50, 1152, 100, BF),
                                         (64, 128, 128, F32), (51277, 1152, 1152, BF), (76800, 64, 288, BF),
                                         (70000, 1152, 100, BF)])
def test_out_proj(rows, K, N, dt):
    sd = "bf16" if dt == BF else "f32"
    a = st_synth.randn((rows, K), 21 + rows, dtype=sd)
    w = st_synth.randn((N, K), 22 + rows, std=0.02, dtype=sd)
    y = empty((rows, N), dt == BF)
    st.st_out_proj(to_dev(a), rows, K, to_dev(w), N, dt, y)
    sync()
    assert_close(f64(y), oracle.linear(f64(a), f64(w)), bf16=dt == BF, what="y")


# rows in [outer, n1, n2] order stored as [outer, n2, n1]: ragged GEMM tiles (rows not a
# multiple of 256), the 288-channel and the 256-channel tilings, fp32
@pytest.mark.parametrize("outer,n1,n2,K,N,dt", [(2, 5, 37, 1152, 1152, BF), (1, 51, 13, 384, 384, BF),
                                                (3, 7, 9, 1152, 100, BF), (1, 4, 6, 128, 128, F32),
                                                (1, 1, 70, 128, 64, BF), (1, 51, 1020, 1152, 1152, BF)])
def test_out_proj_relayout(outer, n1, n2, K, N, dt):
    sd = "bf16" if dt == BF else "f32"
    rows = outer * n1 * n2
    a = st_synth.randn((rows, K), 31 + rows, dtype=sd)
    w = st_synth.randn((N, K), 32 + rows, std=0.02, dtype=sd)
    ad, wd = to_dev(a), to_dev(w)
    y, y_ref = empty((rows, N), dt == BF), empty((rows, N), dt == BF)
    h = empty((rows, N), dt == BF)
    st.st_out_proj_relayout(ad, rows, K, wd, N, dt, n1, n2, y)
    st.st_out_proj(ad, rows, K, wd, N, dt, h)
    eb = 2 if dt == BF else 4
    st.st_relayout(h, [n1 * n2 * N, n2 * N, N, 1], y_ref, [n1 * n2 * N, N, n1 * N, 1], [outer, n1, n2, N], 4, eb)
    sync()
    assert t_.equal(y, y_ref)   # the fused store is bit-identical to projection + relayout
    ref = oracle.bt_to_bs(oracle.linear(f64(a), f64(w)).reshape(outer, n1, n2, N)).reshape(rows, N)
    assert_close(f64(y), ref, bf16=dt == BF, what="y")


# --------------------------------------------------------------------------- #
# Attention                                                                    #
# --------------------------------------------------------------------------- #
def qkv_tensors(shape, seed, dt, q_std=1.0):
    sd = "bf16" if dt == BF else "f32"
    return (st_synth.randn(shape, seed, std=q_std, dtype=sd), st_synth.randn(shape, seed + 1, dtype=sd),
            st_synth.randn(shape, seed + 2, dtype=sd))


SPATIAL_CASES = [
    # B, T, S, H, d, q_std, dtype
    (1, 2, 300, 2, 72, 1.0, BF),
    (2, 1, 1000, 1, 72, 3.0, BF),      # peaked softmax
    (1, 1, 1, 3, 72, 1.0, BF),         # L = 1
    (1, 3, 64, 2, 72, 1.0, BF),
    (1, 1, 3600, 1, 72, 1.0, BF),      # 720p frame: the last 512-query block holds 16 queries, 7 waves idle
    (1, 1, 700, 3, 128, 1.0, BF),
    (1, 2, 257, 2, 64, 2.0, BF),
    (1, 2, 64, 2, 64, 1.0, F32),
]


@pytest.mark.parametrize("B,T,S,H,d,q_std,dt", SPATIAL_CASES)
def test_attn_spatial(B, T, S, H, d, q_std, dt):
    q, k, v = qkv_tensors((B, T, S, H, d), 31 + S + d, dt, q_std)
    out = empty((B, T, S, H, d), dt == BF)
    scale = 1.0 / math.sqrt(d)
    st.st_attn_spatial(to_dev(q), to_dev(k), to_dev(v), B, T, S, H, d, scale, dt, None, 0, out)
    sync()
    ref = oracle.attn_spatial(f64(q), f64(k), f64(v), scale)
    assert_close(f64(out), ref, bf16=dt == BF, what="O")


TEMPORAL_CASES = [
    # B, S, T, t_valid, H, d, dtype
    (1, 37, 51, 51, 16, 72, BF),
    (1, 20, 52, 51, 16, 72, BF),
    (2, 10, 24, 24, 4, 72, BF),
    (1, 11, 30, 27, 5, 72, BF),        # one query tile, masked keys, a partial head group
    (1, 6, 32, 31, 4, 72, BF),         # one query tile, full
    (1, 7, 17, 12, 3, 64, BF),
    (1, 5, 64, 60, 3, 72, BF),
    (1, 3, 80, 70, 2, 72, BF),         # longer than the short kernel: long path
    (1, 9, 1, 1, 2, 72, BF),           # T = 1
    (1, 7, 33, 33, 2, 64, BF),
    (2, 5, 40, 37, 6, 64, BF),         # two head groups per (b, s), the second one partial
    (1, 4, 20, 20, 2, 128, BF),        # d = 128: long path
    (1, 64, 4, 4, 2, 64, F32),
    (1, 6, 10, 7, 2, 64, F32),
]


# Peaked softmax: q and k elements ~ N(0, 16), as after a per-head RMSNorm with gain 4, so scores
# q.k/sqrt(d) have standard deviation 16 and most queries are dominated by a few keys.  Near-ties
# between the top keys turn any extra rounding of the scores into output errors.
PEAKED_CASES = [(1, 2048, 2, 72), (2, 1500, 1, 72), (1, 1024, 2, 64), (1, 777, 2, 128)]


@pytest.mark.parametrize("prescaled", [False, True])
@pytest.mark.parametrize("T,S,H,d", PEAKED_CASES)
def test_attn_spatial_peaked_scores(T, S, H, d, prescaled):
    """prescaled: q stored times (1/sqrt(d)) log2(e) (rounded to bf16 once) and attended with
    scale ln 2, as inside the layer pair; the oracle sees the same stored q and scale."""
    shape = (1, T, S, H, d)
    q = st_synth.randn(shape, 900 + S, std=4.0)
    k = st_synth.randn(shape, 901 + S, std=4.0)
    v = st_synth.randn(shape, 902 + S)
    scale = 1.0 / math.sqrt(d)
    if prescaled:
        q = st_synth.f32_to_bf16_bits((f64(q) * (scale * math.log2(math.e))).astype(np.float32))
        scale = math.log(2.0)
    out = empty(shape)
    st.st_attn_spatial(to_dev(q), to_dev(k), to_dev(v), 1, T, S, H, d, scale, BF, None, 0, out)
    sync()
    ref = oracle.attn_spatial(f64(q), f64(k), f64(v), scale)
    ma, rl = assert_close(f64(out), ref, True, "O")
    print(f"peaked T={T} S={S} d={d} prescaled={prescaled}: max_abs={ma:.3e} rel_l2={rl:.3e}")


@pytest.mark.parametrize("B,S,T,tv,H,d,dt", TEMPORAL_CASES)
def test_attn_temporal(B, S, T, tv, H, d, dt):
    q, k, v = qkv_tensors((B, S, T, H, d), 41 + T + S, dt)
    out = empty((B, S, T, H, d), dt == BF)
    scale = 1.0 / math.sqrt(d)
    st.st_attn_temporal(to_dev(q), to_dev(k), to_dev(v), B, S, T, tv, H, d, scale, dt, None, 0, out)
    sync()
    ref = oracle.attn_temporal(f64(q), f64(k), f64(v), scale, tv)
    assert_close(f64(out), ref, bf16=dt == BF, what="O")


def test_attention_is_deterministic():
    q, k, v = qkv_tensors((1, 2, 500, 2, 72), 77, BF)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    outs = []
    for _ in range(3):
        o = empty((1, 2, 500, 2, 72))
        st.st_attn_spatial(dq, dk, dv, 1, 2, 500, 2, 72, 1 / math.sqrt(72), BF, None, 0, o)
        outs.append(to_host(o))
    sync()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("temporal,dt", [(False, BF), (True, BF), (False, F32), (True, F32)])
def test_attention_with_output_projection(temporal, dt):
    """w_o given: out = O . w_o^T, O staged in the caller's workspace; bit-identical to the
    attention call followed by st_out_proj, and within the bars of the oracle's linear(attention)."""
    bf = dt == BF
    B, A, L, H, d, C = (1, 40, 52, 16, 72, 1152) if bf else (1, 6, 10, 2, 64, 128)
    tv = L - 3 if temporal else L
    q, k, v = qkv_tensors((B, A, L, H, d), 77 + L, dt)
    w = st_synth.randn((C, H * d), 78, std=0.02, dtype="bf16" if bf else "f32")
    qd, kd, vd, wd = to_dev(q), to_dev(k), to_dev(v), to_dev(w)
    rows = B * A * L
    nb = st.st_attn_workspace(rows, H, d, dt)
    ws = t_.empty(nb, dtype=t_.uint8, device="cuda")
    out = empty((rows, C), bf)
    o, y2 = empty((B, A, L, H, d), bf), empty((rows, C), bf)
    scale = 1.0 / math.sqrt(d)
    if temporal:
        st.st_attn_temporal(qd, kd, vd, B, A, L, tv, H, d, scale, dt, wd, C, out, ws, nb)
        st.st_attn_temporal(qd, kd, vd, B, A, L, tv, H, d, scale, dt, None, 0, o)
    else:
        st.st_attn_spatial(qd, kd, vd, B, A, L, H, d, scale, dt, wd, C, out, ws, nb)
        st.st_attn_spatial(qd, kd, vd, B, A, L, H, d, scale, dt, None, 0, o)
    st.st_out_proj(o, rows, H * d, wd, C, dt, y2)
    sync()
    assert t_.equal(out, y2)
    att = oracle.attn_temporal(f64(q), f64(k), f64(v), scale, tv) if temporal else \
        oracle.attn_spatial(f64(q), f64(k), f64(v), scale)
    # the projection's input is the attention output as stored (bf16 or fp32)
    ref = oracle.linear(f64(o).reshape(rows, H * d), f64(w))
    assert_close(f64(out), ref, bf, "O w_o^T")
    assert_close(f64(o), att, bf, "O")
