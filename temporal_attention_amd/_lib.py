"""ctypes binding of libst.so: argument marshalling only.

Every function has the name and argument order of the C entry point in
include/st.h.  Pointer arguments accept a torch tensor (its data_ptr()), a
plain integer address, or None (NULL).  `stream` accepts a torch stream, an
integer hipStream_t, or None for torch's current stream (0 when no GPU is
visible).  A non-OK status raises STError carrying the code.

There is no fallback: if libst.so was not built, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libst.so")

ST_OK, ST_EINVAL, ST_EUNSUPPORTED, ST_EALIGN, ST_EWORKSPACE, ST_ELAUNCH = range(6)
ST_F32, ST_BF16 = 0, 1
ST_ROPE_NONE, ST_ROPE_1D, ST_ROPE_2D = 0, 1, 2
ST_A2A_S2T, ST_A2A_T2S = 0, 1

# Every entry point declared in include/st.h.
EXPORTS = (
    "st_status_str", "st_rope_table_floats", "st_rope_table", "st_qkv_norm_rope", "st_layer_scales", "st_out_proj",
    "st_out_proj_relayout", "st_attn_spatial", "st_attn_temporal", "st_attn_workspace", "st_attn_chunk",
    "st_attn_chunk_acc",
    "st_attn_merge", "st_relayout", "st_block_sliced", "st_block_sliced_2s", "st_block_sliced_workspace",
    "st_block_sliced_2s_workspace", "st_block_sliced_noalloc", "st_block_sliced_noalloc_max", "st_a2a_pack",
    "st_a2a_unpack",
    "st_v_change",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python temporal_attention_amd/build.py`")

# torch ships its own HIP runtime.  libst.so must bind to that same runtime
# (device memory and streams come from torch), so torch is loaded first.
import torch  # noqa: E402,F401

lib = C.CDLL(LIB_PATH)


def _hip_runtimes() -> list[str]:
    with open("/proc/self/maps") as f:
        return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are mapped ({_hip_runtimes()}); import torch before loading libst.so")

_p, _i, _i64, _f, _sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t


class st_layer_weights(C.Structure):
    _fields_ = [("w_qkv", _p), ("w_o", _p), ("g_q", _p), ("g_k", _p)]


_SIGS = {
    "st_status_str": (C.c_char_p, [_i]),
    "st_rope_table_floats": (_sz, [_i, _i, _i]),
    "st_rope_table": (_i, [_i, _i, _f, _i, _p, _p]),
    "st_qkv_norm_rope": (_i, [_p, _i64, _i, _p, _p, _p, _f, _f, _i, _p, _i, _p, _i64, _i64, _i, _i, _i, _i, _p, _p,
                              _p, _p]),
    "st_layer_scales": (_i, [_i, _i, C.POINTER(C.c_float), C.POINTER(C.c_float)]),
    "st_out_proj": (_i, [_p, _i64, _i, _p, _i, _i, _p, _p]),
    "st_out_proj_relayout": (_i, [_p, _i64, _i, _p, _i, _i, _i64, _i64, _p, _p]),
    "st_attn_spatial": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _i, _p, _p, _sz, _p]),
    "st_attn_temporal": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _i, _p, _p, _sz, _p]),
    "st_attn_workspace": (_sz, [_i64, _i, _i, _i]),
    "st_attn_chunk": (_i, [_p, _p, _p, _i64, _i, _i, _i, _i, _i, _f, _i, _p, _p, _p]),
    "st_attn_chunk_acc": (_i, [_p, _p, _p, _i64, _i, _i, _i, _i, _i, _f, _i, _p, _p, _p]),
    "st_attn_merge": (_i, [_p, _p, _p, _p, _i64, _i, _i, _i, _i, _p, _p, _p]),
    "st_v_change": (_i, [_p, _p, _i64, _i, _i, _f, _i, _p, _p, _p, _i, _p]),
    "st_relayout": (_i, [_p, C.POINTER(C.c_int64), _p, C.POINTER(C.c_int64), C.POINTER(C.c_int64), _i, _i, _p]),
    "st_block_sliced": (_i, [_p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, C.POINTER(st_layer_weights),
                             C.POINTER(st_layer_weights), _f, _f, _i, _p, _p, _sz, _p]),
    "st_block_sliced_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "st_block_sliced_2s_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "st_block_sliced_noalloc": (_i, [_p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, C.POINTER(st_layer_weights),
                                     C.POINTER(st_layer_weights), _f, _f, _i, _p, _p]),
    "st_block_sliced_noalloc_max": (_sz, []),
    "st_a2a_pack": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _p]),
    "st_a2a_unpack": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _p]),
    "st_block_sliced_2s": (_i, [_p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, C.POINTER(st_layer_weights),
                                C.POINTER(st_layer_weights), _f, _f, _i, _p, _p, _sz, _p, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype, _fn.argtypes = _res, _args


class STError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {lib.st_status_str(code).decode()} (status {code})")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, code: int) -> None:
    if code != ST_OK:
        raise STError(fn, code)


def st_status_str(status: int) -> str:
    return lib.st_status_str(status).decode()


def st_rope_table_floats(d: int, kind: int, n_pos: int) -> int:
    return lib.st_rope_table_floats(d, kind, n_pos)


def st_rope_table(d, kind, base, n_pos, table, stream=None):
    _check("st_rope_table", lib.st_rope_table(d, kind, base, n_pos, _ptr(table), _stream(stream)))


def st_qkv_norm_rope(x, rows, c_in, w_qkv, g_q, g_k, eps, q_scale, rope_kind, rope_table, rope_npos, pos, pos_period,
                     pos_offset, grid_w, H, d, dtype, q, k, v, stream=None):
    _check("st_qkv_norm_rope", lib.st_qkv_norm_rope(
        _ptr(x), rows, c_in, _ptr(w_qkv), _ptr(g_q), _ptr(g_k), eps, q_scale, rope_kind, _ptr(rope_table), rope_npos,
        _ptr(pos), pos_period, pos_offset, grid_w, H, d, dtype, _ptr(q), _ptr(k), _ptr(v), _stream(stream)))


def st_layer_scales(d, dtype):
    """(q_scale, attn_scale) of a layer of st_block_sliced for head dim d."""
    qs, at = C.c_float(), C.c_float()
    _check("st_layer_scales", lib.st_layer_scales(d, dtype, C.byref(qs), C.byref(at)))
    return qs.value, at.value


def st_out_proj(a, rows, k_in, w, n_out, dtype, y, stream=None):
    _check("st_out_proj", lib.st_out_proj(_ptr(a), rows, k_in, _ptr(w), n_out, dtype, _ptr(y), _stream(stream)))


def st_out_proj_relayout(a, rows, k_in, w, n_out, dtype, n1, n2, y, stream=None):
    _check("st_out_proj_relayout", lib.st_out_proj_relayout(_ptr(a), rows, k_in, _ptr(w), n_out, dtype, n1, n2,
                                                            _ptr(y), _stream(stream)))


def st_attn_spatial(q, k, v, B, T, S, H, d, scale, dtype, w_o, c_out, out, ws=None, ws_bytes=0, stream=None):
    _check("st_attn_spatial", lib.st_attn_spatial(_ptr(q), _ptr(k), _ptr(v), B, T, S, H, d, scale, dtype, _ptr(w_o),
                                                  c_out, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def st_attn_temporal(q, k, v, B, S, T, t_valid, H, d, scale, dtype, w_o, c_out, out, ws=None, ws_bytes=0,
                     stream=None):
    _check("st_attn_temporal", lib.st_attn_temporal(_ptr(q), _ptr(k), _ptr(v), B, S, T, t_valid, H, d, scale, dtype,
                                                    _ptr(w_o), c_out, _ptr(out), _ptr(ws), ws_bytes,
                                                    _stream(stream)))


def st_attn_workspace(rows, H, d, dtype) -> int:
    return lib.st_attn_workspace(rows, H, d, dtype)


def st_attn_chunk(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dtype, out, lse, stream=None):
    _check("st_attn_chunk", lib.st_attn_chunk(_ptr(q), _ptr(k), _ptr(v), outer, Lq, Lk, kv_valid, H, d, scale, dtype,
                                              _ptr(out), _ptr(lse), _stream(stream)))


def st_attn_chunk_acc(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dtype, acc_o, acc_lse, stream=None):
    _check("st_attn_chunk_acc", lib.st_attn_chunk_acc(_ptr(q), _ptr(k), _ptr(v), outer, Lq, Lk, kv_valid, H, d, scale,
                                                      dtype, _ptr(acc_o), _ptr(acc_lse), _stream(stream)))


def st_attn_merge(o_a, lse_a, o_b, lse_b, outer, L, H, d, dtype, out, lse, stream=None):
    _check("st_attn_merge", lib.st_attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), outer, L, H, d, dtype,
                                              _ptr(out), _ptr(lse), _stream(stream)))


def st_v_change(v_new, v_cache, rows, H, d, threshold, dtype, mask, active_idx, n_active, update_cache,
                stream=None):
    _check("st_v_change", lib.st_v_change(_ptr(v_new), _ptr(v_cache), rows, H, d, threshold, dtype, _ptr(mask),
                                          _ptr(active_idx), _ptr(n_active), int(bool(update_cache)),
                                          _stream(stream)))


def _i64arr(vals):
    return (C.c_int64 * len(vals))(*[int(x) for x in vals])


def st_relayout(src, src_strides, dst, dst_strides, dims, ndim, elem_bytes, stream=None):
    _check("st_relayout", lib.st_relayout(_ptr(src), _i64arr(src_strides), _ptr(dst), _i64arr(dst_strides),
                                          _i64arr(dims), ndim, elem_bytes, _stream(stream)))


def st_a2a_pack(x, send, dir, B, T, S, C_, P, elem_bytes, stream=None):
    _check("st_a2a_pack", lib.st_a2a_pack(_ptr(x), _ptr(send), dir, B, T, S, C_, P, elem_bytes, _stream(stream)))


def st_a2a_unpack(recv, y, dir, B, T, S, C_, P, elem_bytes, stream=None):
    _check("st_a2a_unpack", lib.st_a2a_unpack(_ptr(recv), _ptr(y), dir, B, T, S, C_, P, elem_bytes, _stream(stream)))


def layer_weights(w_qkv, w_o, g_q, g_k) -> st_layer_weights:
    return st_layer_weights(_ptr(w_qkv), _ptr(w_o), _ptr(g_q), _ptr(g_k))


def st_block_sliced_workspace(B, T, S, grid_w, C_, H, d, n_t, n_s, dtype) -> int:
    return lib.st_block_sliced_workspace(B, T, S, grid_w, C_, H, d, n_t, n_s, dtype)


def st_block_sliced_2s_workspace(B, T, S, grid_w, C_, H, d, n_t, n_s, dtype) -> int:
    return lib.st_block_sliced_2s_workspace(B, T, S, grid_w, C_, H, d, n_t, n_s, dtype)


def st_block_sliced(x, B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype, y,
                    ws, ws_bytes, stream=None):
    """spatial / temporal: st_layer_weights (see layer_weights) or None."""
    sp = C.byref(spatial) if spatial is not None else None
    tp = C.byref(temporal) if temporal is not None else None
    _check("st_block_sliced", lib.st_block_sliced(_ptr(x), B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s, sp, tp, eps,
                                                  rope_base, dtype, _ptr(y), _ptr(ws), ws_bytes, _stream(stream)))


def st_block_sliced_noalloc(x, B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype,
                            y, stream=None):
    """As st_block_sliced, with the workspace taken from the library's fixed device array."""
    sp = C.byref(spatial) if spatial is not None else None
    tp = C.byref(temporal) if temporal is not None else None
    _check("st_block_sliced_noalloc", lib.st_block_sliced_noalloc(_ptr(x), B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s,
                                                                  sp, tp, eps, rope_base, dtype, _ptr(y),
                                                                  _stream(stream)))


def st_block_sliced_noalloc_max() -> int:
    return lib.st_block_sliced_noalloc_max()


def st_block_sliced_2s(x, B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype, y,
                       ws, ws_bytes, stream=None, side_stream=None):
    """As st_block_sliced, with slice gathers/scatters on side_stream (a second, distinct stream)."""
    sp = C.byref(spatial) if spatial is not None else None
    tp = C.byref(temporal) if temporal is not None else None
    _check("st_block_sliced_2s", lib.st_block_sliced_2s(_ptr(x), B, T, t_valid, S, grid_w, C_, H, d, n_t, n_s, sp, tp,
                                                        eps, rope_base, dtype, _ptr(y), _ptr(ws), ws_bytes,
                                                        _stream(stream), _side(side_stream)))


def _side(s):
    if s is None or isinstance(s, int):
        return s
    return s.cuda_stream
