"""C-ABI boundary tests that need no GPU.

The library must load, export every entry point include/st.h declares, and
reject every invalid argument on the host, before any HIP call, with its
documented status code.  Pointers here are fake aligned addresses: validation
never dereferences them, and every case below fails validation.
"""
import math
import os
import re

import numpy as np
import pytest

import temporal_attention_amd as st

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000          # fake 16-byte-aligned device addresses, far apart
P2, P3, P4, P5, P6, P7 = (P * k for k in range(2, 8))
BIG = 1 << 40        # far-apart region for outputs


def declared_functions():
    with open(os.path.join(ROOT, "include", "st.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(st_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(st.lib, n), n
    assert sorted(st.EXPORTS) == names


def test_status_strings():
    assert st.st_status_str(0) == "ok"
    assert "invalid" in st.st_status_str(1)
    assert st.st_status_str(99) == "unknown status"


def code(fn, *args):
    with pytest.raises(st.STError) as e:
        fn(*args, stream=0)
    return e.value.code


def test_rope_table_validation():
    assert st.st_rope_table_floats(72, st.ST_ROPE_2D, 120) == 120 * 18 * 2
    assert st.st_rope_table_floats(72, st.ST_ROPE_1D, 52) == 52 * 36 * 2
    assert code(st.st_rope_table, 72, 0, 10000.0, 10, P) == st.ST_EINVAL            # kind none
    assert code(st.st_rope_table, 70, st.ST_ROPE_2D, 10000.0, 10, P) == st.ST_EINVAL  # d % 4
    assert code(st.st_rope_table, 72, st.ST_ROPE_1D, -1.0, 10, P) == st.ST_EINVAL
    assert code(st.st_rope_table, 72, st.ST_ROPE_1D, 10000.0, 0, P) == st.ST_EINVAL
    assert code(st.st_rope_table, 72, st.ST_ROPE_1D, 10000.0, 10, None) == st.ST_EINVAL
    assert code(st.st_rope_table, 72, st.ST_ROPE_1D, 10000.0, 10, P + 4) == st.ST_EALIGN


def qkv_args(**kw):
    a = dict(x=P, rows=100, c_in=1152, w_qkv=P2, g_q=P3, g_k=P4, eps=1e-6, q_scale=1.0, rope_kind=st.ST_ROPE_2D,
             rope_table=P5, rope_npos=120, pos=None, pos_period=8160, pos_offset=0, grid_w=120, H=16, d=72,
             dtype=st.ST_BF16, q=BIG, k=2 * BIG, v=3 * BIG)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), st.ST_EINVAL),
    (dict(g_q=None), st.ST_EINVAL),
    (dict(dtype=7), st.ST_EINVAL),
    (dict(rows=-1), st.ST_EINVAL),
    (dict(eps=-1.0), st.ST_EINVAL),
    (dict(d=70), st.ST_EINVAL),                       # 2D RoPE needs d % 4 == 0
    (dict(d=96), st.ST_EUNSUPPORTED),                 # no bf16 kernel for d = 96
    (dict(d=256, dtype=st.ST_F32), st.ST_EUNSUPPORTED),
    (dict(c_in=1150), st.ST_EUNSUPPORTED),            # bf16 needs c_in % 64 == 0
    (dict(c_in=1160), st.ST_EUNSUPPORTED),
    (dict(c_in=1120), st.ST_EUNSUPPORTED),
    (dict(rope_kind=5), st.ST_EINVAL),
    (dict(rope_table=None), st.ST_EINVAL),
    (dict(rope_npos=60, rows=8160), st.ST_EINVAL),   # h up to 67 not in table
    (dict(rope_kind=st.ST_ROPE_1D, rope_npos=51, pos_period=52), st.ST_EINVAL),
    (dict(pos_period=0), st.ST_EINVAL),
    (dict(rope_table=P5 + 8), st.ST_EALIGN),
    (dict(x=P + 2), st.ST_EALIGN),
    (dict(q=P), st.ST_EINVAL),                        # q aliases x
    (dict(k=BIG + 64), st.ST_EINVAL),                 # k overlaps q
    (dict(q_scale=0.0), st.ST_EINVAL),
    (dict(q_scale=float("inf")), st.ST_EINVAL),
    (dict(pos=P6 + 4), st.ST_EALIGN),                 # positions need 8-byte alignment
    (dict(pos=BIG + 16), st.ST_EINVAL),               # positions overlap q
    # with positions the periodic rule is not checked: the call gets past it to the alignment check
    (dict(pos=P6, pos_period=0, rope_npos=1, x=P + 2), st.ST_EALIGN),
])
def test_qkv_validation(kw, want):
    assert code(st.st_qkv_norm_rope, *qkv_args(**kw)) == want


def test_layer_scales():
    qs, at = st.st_layer_scales(72, st.ST_BF16)
    assert abs(qs - math.log2(math.e) / math.sqrt(72)) < 1e-7 and abs(at - math.log(2)) < 1e-7
    # the softmax the layer computes is unchanged: q_scale * attn_scale = 1/sqrt(d)
    assert abs(qs * at - 1 / math.sqrt(72)) < 1e-7
    assert st.st_layer_scales(64, st.ST_F32) == (1.0, np.float32(1 / 8.0))
    with pytest.raises(st.STError):
        st.st_layer_scales(0, st.ST_BF16)


@pytest.mark.parametrize("args,want", [
    ((None, 10, 1152, P2, 1152, st.ST_BF16, BIG), st.ST_EINVAL),
    ((P, 10, 1152, P2, 1150, st.ST_BF16, BIG), st.ST_EUNSUPPORTED),
    ((P, 10, 1151, P2, 1152, st.ST_BF16, BIG), st.ST_EUNSUPPORTED),
    ((P, 10, 1160, P2, 1152, st.ST_BF16, BIG), st.ST_EUNSUPPORTED),
    ((P, 10, 1152, P2, 1152, 3, BIG), st.ST_EINVAL),
    ((P, 10, 1152, P2, 1152, st.ST_BF16, P + 16), st.ST_EINVAL),    # y overlaps a
    ((P, 10, 1152, P2, 1152, st.ST_BF16, BIG + 2), st.ST_EALIGN),
])
def test_out_proj_validation(args, want):
    assert code(st.st_out_proj, *args) == want


@pytest.mark.parametrize("args,want", [
    ((P, 12, 1152, P2, 1152, st.ST_BF16, 0, 4, BIG), st.ST_EINVAL),              # n1 < 1
    ((P, 12, 1152, P2, 1152, st.ST_BF16, 3, -1, BIG), st.ST_EINVAL),             # n2 < 1
    ((P, 10, 1152, P2, 1152, st.ST_BF16, 3, 4, BIG), st.ST_EINVAL),              # rows not a multiple of n1*n2
    ((P, -12, 1152, P2, 1152, st.ST_BF16, 3, 4, BIG), st.ST_EINVAL),
    ((None, 12, 1152, P2, 1152, st.ST_BF16, 3, 4, BIG), st.ST_EINVAL),
    ((P, 12, 1152, P2, 1150, st.ST_BF16, 3, 4, BIG), st.ST_EUNSUPPORTED),        # n_out % 4
    ((P, 12, 1160, P2, 1152, st.ST_BF16, 3, 4, BIG), st.ST_EUNSUPPORTED),        # bf16 k_in % 64
    ((P, 12, 1152, P2, 1152, 3, 3, 4, BIG), st.ST_EINVAL),                       # dtype
    ((P, 12, 1152, P2, 1152, st.ST_BF16, 3, 4, P + 16), st.ST_EINVAL),          # y overlaps a
    ((P, 12, 1152, P2, 1152, st.ST_BF16, 3, 4, BIG + 2), st.ST_EALIGN),
])
def test_out_proj_relayout_validation(args, want):
    assert code(st.st_out_proj_relayout, *args) == want


def attn_args(**kw):
    a = dict(q=P, k=P2, v=P3, B=1, T=51, S=8160, H=16, d=72, scale=0.1, dtype=st.ST_BF16, w_o=None, c_out=0,
             out=BIG, ws=None, ws_bytes=0)
    a.update(kw)
    return list(a.values())


ROWS = 51 * 8160


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), st.ST_EINVAL),
    (dict(scale=0.0), st.ST_EINVAL),                   # scale must be > 0
    (dict(scale=float("nan")), st.ST_EINVAL),
    (dict(B=-1), st.ST_EINVAL),
    (dict(d=80), st.ST_EUNSUPPORTED),
    (dict(out=P), st.ST_EINVAL),                       # out aliases q
    (dict(out=BIG + 8), st.ST_EALIGN),
    # with the output projection
    (dict(w_o=P4, c_out=0), st.ST_EINVAL),
    (dict(w_o=P4, c_out=1150), st.ST_EUNSUPPORTED),    # c_out % 4
    (dict(w_o=P4, c_out=1152, ws=None), st.ST_EWORKSPACE),
    (dict(w_o=P4, c_out=1152, ws=2 * BIG, ws_bytes=100), st.ST_EWORKSPACE),
    (dict(w_o=P4 + 8, c_out=1152, ws=2 * BIG, ws_bytes=1 << 40), st.ST_EALIGN),
    (dict(w_o=P4, c_out=1152, ws=BIG + 64, ws_bytes=1 << 40), st.ST_EINVAL),   # workspace overlaps out
    (dict(w_o=P4, c_out=1152, ws=P2, ws_bytes=1 << 40), st.ST_EINVAL),         # workspace overlaps k
])
def test_attn_spatial_validation(kw, want):
    assert code(st.st_attn_spatial, *attn_args(**kw)) == want


def test_attn_workspace():
    assert st.st_attn_workspace(ROWS, 16, 72, st.ST_BF16) == ROWS * 16 * 72 * 2
    assert st.st_attn_workspace(10, 2, 64, st.ST_F32) == 5120
    assert st.st_attn_workspace(-1, 2, 64, st.ST_F32) == 0


@pytest.mark.parametrize("t_valid,want", [(0, st.ST_EINVAL), (53, st.ST_EINVAL)])
def test_attn_temporal_validation(t_valid, want):
    assert code(st.st_attn_temporal, P, P2, P3, 1, 8160, 52, t_valid, 16, 72, 0.1, st.ST_BF16, None, 0, BIG, None,
                0) == want


def chunk_args(**kw):
    a = dict(q=P, k=P2, v=P3, outer=51, Lq=100, Lk=64, kv_valid=64, H=16, d=72, scale=0.1, dtype=st.ST_BF16, out=BIG,
             lse=2 * BIG)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), st.ST_EINVAL),
    (dict(lse=None), st.ST_EINVAL),
    (dict(kv_valid=-1), st.ST_EINVAL),
    (dict(kv_valid=65), st.ST_EINVAL),               # more valid keys than the chunk holds
    (dict(Lk=-1), st.ST_EINVAL),
    (dict(outer=-1), st.ST_EINVAL),
    (dict(scale=0.0), st.ST_EINVAL),
    (dict(dtype=5), st.ST_EINVAL),
    (dict(d=96), st.ST_EUNSUPPORTED),
    (dict(out=P2), st.ST_EINVAL),                    # out aliases k
    (dict(lse=P3 + 64), st.ST_EINVAL),               # lse overlaps v
    (dict(lse=BIG + 128), st.ST_EINVAL),             # lse overlaps out
    (dict(out=BIG + 4), st.ST_EALIGN),
    (dict(lse=2 * BIG + 2), st.ST_EALIGN),
])
def test_attn_chunk_validation(kw, want):
    assert code(st.st_attn_chunk, *chunk_args(**kw)) == want
    # the accumulating form validates the same way (acc_o, acc_lse in the roles of out, lse)
    assert code(st.st_attn_chunk_acc, *chunk_args(**kw)) == want


def merge_args(**kw):
    a = dict(o_a=P, lse_a=P2, o_b=P3, lse_b=P4, outer=51, L=100, H=16, d=72, dtype=st.ST_BF16, out=BIG, lse=2 * BIG)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(o_a=None), st.ST_EINVAL),
    (dict(lse_b=None), st.ST_EINVAL),
    (dict(H=0), st.ST_EINVAL),
    (dict(d=0), st.ST_EINVAL),
    (dict(dtype=9), st.ST_EINVAL),
    (dict(out=P + 32), st.ST_EINVAL),                # partial overlap with o_a (in place must be exact)
    (dict(lse=P2 + 4), st.ST_EINVAL),                # partial overlap with lse_a
    (dict(lse=BIG + 64), st.ST_EINVAL),              # lse inside out
    (dict(out=P2), st.ST_EINVAL),                    # out over lse_a
    (dict(out=BIG + 8), st.ST_EALIGN),
    (dict(lse=2 * BIG + 1), st.ST_EALIGN),
])
def test_attn_merge_validation(kw, want):
    assert code(st.st_attn_merge, *merge_args(**kw)) == want


def vchange_args(**kw):
    a = dict(v_new=P, v_cache=P2, rows=100, H=16, d=72, threshold=1.0, dtype=st.ST_BF16, mask=BIG, active_idx=2 * BIG,
             n_active=3 * BIG, update_cache=1)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(v_new=None), st.ST_EINVAL),
    (dict(mask=None), st.ST_EINVAL),
    (dict(n_active=None), st.ST_EINVAL),
    (dict(threshold=-1.0), st.ST_EINVAL),
    (dict(threshold=float("nan")), st.ST_EINVAL),
    (dict(H=0), st.ST_EINVAL),
    (dict(dtype=4), st.ST_EINVAL),
    (dict(d=70), st.ST_EUNSUPPORTED),                # rows must be whole 16-byte pieces
    (dict(d=264), st.ST_EUNSUPPORTED),               # more than 512 bytes per row
    (dict(v_cache=P + 64), st.ST_EINVAL),            # v_new and v_cache overlap
    (dict(mask=P2 + 16), st.ST_EINVAL),              # mask inside v_cache
    (dict(active_idx=BIG + 16), st.ST_EINVAL),       # idx overlaps mask
    (dict(v_new=P + 8), st.ST_EALIGN),
    (dict(n_active=3 * BIG + 4), st.ST_EALIGN),
    (dict(mask=BIG + 1), st.ST_EALIGN),
])
def test_v_change_validation(kw, want):
    assert code(st.st_v_change, *vchange_args(**kw)) == want


def test_relayout_validation():
    dims, s1, s2 = [2, 3, 4], [12, 4, 1], [12, 1, 3]
    assert code(st.st_relayout, None, s1, BIG, s2, dims, 3, 2) == st.ST_EINVAL
    assert code(st.st_relayout, P, s1, BIG, s2, dims, 0, 2) == st.ST_EINVAL           # ndim
    assert code(st.st_relayout, P, s1 * 3, BIG, s2 * 3, dims * 3, 7, 2) == st.ST_EINVAL
    assert code(st.st_relayout, P, s1, BIG, s2, dims, 3, 3) == st.ST_EINVAL           # elem_bytes
    assert code(st.st_relayout, P, s1, P, s2, dims, 3, 2) == st.ST_EINVAL             # src == dst
    assert code(st.st_relayout, P, s1, P + 8, s2, dims, 3, 2) == st.ST_EINVAL         # overlap
    assert code(st.st_relayout, P, s1, BIG, s2, [2, -3, 4], 3, 2) == st.ST_EINVAL
    assert code(st.st_relayout, P + 1, s1, BIG, s2, dims, 3, 2) == st.ST_EALIGN


def test_block_workspace_and_validation():
    ws = st.st_block_sliced_workspace(1, 52, 8160, 120, 1152, 16, 72, 4, 4, st.ST_BF16)
    N, slice_rows = 52 * 8160, max(13 * 8160, 2040 * 52)
    # one stream, bf16: the blocked intermediate plus q, k, v, o of the largest slice (and two small tables)
    assert N * 1152 * 2 + 4 * slice_rows * 1152 * 2 <= ws < N * 1152 * 2 + 4 * slice_rows * 1152 * 2 + (1 << 20)
    ws2 = st.st_block_sliced_2s_workspace(1, 52, 8160, 120, 1152, 16, 72, 4, 4, st.ST_BF16)
    assert ws2 >= ws + N * 1152 * 2 + 4 * slice_rows * 1152 * 2      # + blocked input, 2 x 2 slice buffers
    f32 = (1, 4, 64, 8, 128, 2, 64, 2, 2, st.ST_F32)    # fp32 always copies explicitly
    assert st.st_block_sliced_workspace(*f32) == st.st_block_sliced_2s_workspace(*f32)
    assert st.st_block_sliced_workspace(1, 51, 8160, 120, 1152, 16, 72, 4, 4, st.ST_BF16) == 0   # T % n_t
    w = st.layer_weights(P, P2, P3, P4)
    bad_w = st.layer_weights(P, None, P3, P4)
    base = dict(x=P5, B=1, T=52, t_valid=51, S=8160, grid_w=120, C_=1152, H=16, d=72, n_t=4, n_s=4, spatial=w,
                temporal=w, eps=1e-6, rope_base=10000.0, dtype=st.ST_BF16, y=BIG, ws=2 * BIG, ws_bytes=ws)

    def c(**kw):
        a = dict(base)
        a.update(kw)
        return code(st.st_block_sliced, *a.values())
    assert c(T=51) == st.ST_EINVAL                 # T % n_t
    a2 = list(base.values())
    with pytest.raises(st.STError) as e:           # the side stream must be a second, distinct stream
        st.st_block_sliced_2s(*a2, stream=0x1234, side_stream=0x1234)
    assert e.value.code == st.ST_EINVAL
    with pytest.raises(st.STError) as e:
        st.st_block_sliced_2s(*a2, stream=0x1234, side_stream=None)
    assert e.value.code == st.ST_EINVAL
    assert c(t_valid=0) == st.ST_EINVAL
    assert c(grid_w=121) == st.ST_EINVAL           # S % grid_w
    assert c(spatial=None) == st.ST_EINVAL
    assert c(temporal=bad_w) == st.ST_EINVAL
    assert c(ws_bytes=ws - 1) == st.ST_EWORKSPACE
    assert c(ws=None) == st.ST_EWORKSPACE
    assert c(d=80) == st.ST_EUNSUPPORTED
    assert c(y=P5) == st.ST_EINVAL                 # y aliases x
    assert c(x=P5 + 2) == st.ST_EALIGN


def test_block_noalloc_rejects_beyond_its_scratch_before_any_gpu_work():
    assert st.st_block_sliced_noalloc_max() == 256 << 20
    w = st.layer_weights(P, P2, P3, P4)
    # the 720p layer pair needs ~1 GB of workspace
    args = [P5, 1, 24, 24, 3600, 80, 1152, 16, 72, 1, 1, w, w, 1e-6, 10000.0, st.ST_BF16, BIG]
    assert code(st.st_block_sliced_noalloc, *args) == st.ST_EWORKSPACE
    args[9:11] = [4, 4]
    assert code(st.st_block_sliced_noalloc, *args) == st.ST_EWORKSPACE
    args[2] = 25                                                       # T % n_t
    assert code(st.st_block_sliced_noalloc, *args) == st.ST_EINVAL


def test_a2a_validation():
    args = dict(x=P, send=BIG, dir=st.ST_A2A_S2T, B=1, T=56, S=8160, C_=1152, P=8, elem_bytes=2)

    def c(fn, **kw):
        a = dict(args)
        a.update(kw)
        return code(fn, *a.values())
    for fn in (st.st_a2a_pack, st.st_a2a_unpack):
        assert c(fn, x=None) == st.ST_EINVAL
        assert c(fn, dir=2) == st.ST_EINVAL
        assert c(fn, T=51) == st.ST_EINVAL                      # T % P
        assert c(fn, S=8161) == st.ST_EINVAL                    # S % P
        assert c(fn, P=0) == st.ST_EINVAL
        assert c(fn, elem_bytes=3) == st.ST_EINVAL
        assert c(fn, x=P + 1) == st.ST_EALIGN
        assert c(fn, send=P + 64) == st.ST_EINVAL               # overlapping buffers


def test_weight_matrices_beyond_32_bit_offsets_are_unsupported():
    """The projection kernels address the weight matrix with 32-bit offsets: N*K >= 2^31 is refused
    on the host before any GPU work."""
    assert code(st.st_out_proj, P, 10, 65536, P2, 32768, st.ST_BF16, BIG) == st.ST_EUNSUPPORTED
    assert code(st.st_out_proj_relayout, P, 10, 65536, P2, 32768, st.ST_BF16, 2, 5, BIG) == st.ST_EUNSUPPORTED
    assert code(st.st_qkv_norm_rope, *qkv_args(c_in=1 << 20, H=128, d=64, rope_kind=st.ST_ROPE_NONE)) == \
        st.ST_EUNSUPPORTED
