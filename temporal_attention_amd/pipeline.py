"""The unsliced spatial + temporal layer pair as an explicit sequence of C-ABI calls.

This is the same launch sequence st_block_sliced runs natively for
n_t = n_s = 1, exposed step by step so that callers can time or inspect each
kernel: torch provides the device buffers, every step is one libst.so call.

    qkv_spatial     st_qkv_norm_rope      x [B,T,S,C] -> q, k, v   (2D RoPE, (h, w) of s)
    attn_spatial    st_attn_spatial       q, k, v -> o             (over S per frame)
    proj_spatial    st_out_proj_relayout  o -> hs [B,S,T,C]        (relayout fused into the stores)
    qkv_temporal    st_qkv_norm_rope      hs -> q, k, v            (1D RoPE, t)
    attn_temporal   st_attn_temporal      q, k, v -> o             (over T per patch)
    proj_temporal   st_out_proj_relayout  o -> y [B,T,S,C]         (relayout fused into the stores)

With fused=False the two relayouts are separate st_relayout passes
(proj_* = st_out_proj into h, then relayout_fwd / relayout_bwd); the results
are bit-identical.

As in st_block_sliced, q is stored scaled by `q_scale` and the attention runs
with `scale` (st_layer_scales: in bf16, (1/sqrt(d)) * log2(e) and ln 2).
"""
from __future__ import annotations

import torch

from . import _lib as L


class LayerPair:
    def __init__(self, B, T, S, grid_w, C, H, d, t_valid=None, dtype=L.ST_BF16, eps=1e-6, rope_base=10000.0,
                 device="cuda"):
        self.B, self.T, self.S, self.grid_w, self.C, self.H, self.d = B, T, S, grid_w, C, H, d
        self.t_valid = T if t_valid is None else t_valid
        self.dtype, self.eps, self.base = dtype, eps, rope_base
        tdt = torch.bfloat16 if dtype == L.ST_BF16 else torch.float32
        self.N = B * T * S
        hd = H * d
        mk = lambda *shape: torch.empty(shape, dtype=tdt, device=device)  # noqa: E731
        self.q, self.k, self.v, self.o = (mk(self.N, H, d) for _ in range(4))
        self.h, self.hs, self.y = mk(self.N, C), mk(self.N, C), mk(self.N, C)
        self.npos2 = max(S // grid_w, grid_w)
        self.rope2 = torch.empty(L.st_rope_table_floats(d, L.ST_ROPE_2D, self.npos2), dtype=torch.float32,
                                 device=device)
        self.rope1 = torch.empty(L.st_rope_table_floats(d, L.ST_ROPE_1D, T), dtype=torch.float32, device=device)
        L.st_rope_table(d, L.ST_ROPE_2D, rope_base, self.npos2, self.rope2)
        L.st_rope_table(d, L.ST_ROPE_1D, rope_base, T, self.rope1)
        self.q_scale, self.scale = L.st_layer_scales(d, dtype)
        self.hd = hd
        self.x = None
        self.ws = self.wt = None

    def set_weights(self, spatial: dict, temporal: dict):
        """spatial / temporal: dicts of device tensors w_qkv, w_o, g_q, g_k."""
        self.ws, self.wt = spatial, temporal

    def steps(self, x, fused=True):
        """[(name, thunk)] for one pass over x ([B,T,S,C] device tensor)."""
        B, T, S, C, H, d, N, dt = self.B, self.T, self.S, self.C, self.H, self.d, self.N, self.dtype
        ws, wt = self.ws, self.wt
        eb = 2 if dt == L.ST_BF16 else 4
        fwd = ([B, T, S, C], [T * S * C, S * C, C, 1], [S * T * C, C, T * C, 1])
        bwd = ([B, S, T, C], [S * T * C, T * C, C, 1], [T * S * C, C, S * C, 1])
        if fused:
            return [
                ("qkv_spatial", lambda: L.st_qkv_norm_rope(
                    x, N, C, ws["w_qkv"], ws["g_q"], ws["g_k"], self.eps, self.q_scale, L.ST_ROPE_2D, self.rope2,
                    self.npos2, None, S, 0, self.grid_w, H, d, dt, self.q, self.k, self.v)),
                ("attn_spatial", lambda: L.st_attn_spatial(self.q, self.k, self.v, B, T, S, H, d, self.scale, dt,
                                                           None, 0, self.o)),
                ("proj_spatial", lambda: L.st_out_proj_relayout(self.o, N, self.hd, ws["w_o"], C, dt, T, S, self.hs)),
                ("qkv_temporal", lambda: L.st_qkv_norm_rope(
                    self.hs, N, C, wt["w_qkv"], wt["g_q"], wt["g_k"], self.eps, self.q_scale, L.ST_ROPE_1D, self.rope1,
                    T, None, T, 0, 0, H, d, dt, self.q, self.k, self.v)),
                ("attn_temporal", lambda: L.st_attn_temporal(self.q, self.k, self.v, B, S, T, self.t_valid, H, d,
                                                             self.scale, dt, None, 0, self.o)),
                ("proj_temporal", lambda: L.st_out_proj_relayout(self.o, N, self.hd, wt["w_o"], C, dt, S, T, self.y)),
            ]
        return [
            ("qkv_spatial", lambda: L.st_qkv_norm_rope(
                x, N, C, ws["w_qkv"], ws["g_q"], ws["g_k"], self.eps, self.q_scale, L.ST_ROPE_2D, self.rope2,
                self.npos2, None, S, 0, self.grid_w, H, d, dt, self.q, self.k, self.v)),
            ("attn_spatial", lambda: L.st_attn_spatial(self.q, self.k, self.v, B, T, S, H, d, self.scale, dt, None, 0,
                                                       self.o)),
            ("proj_spatial", lambda: L.st_out_proj(self.o, N, self.hd, ws["w_o"], C, dt, self.h)),
            ("relayout_fwd", lambda: L.st_relayout(self.h, fwd[1], self.hs, fwd[2], fwd[0], 4, eb)),
            ("qkv_temporal", lambda: L.st_qkv_norm_rope(
                self.hs, N, C, wt["w_qkv"], wt["g_q"], wt["g_k"], self.eps, self.q_scale, L.ST_ROPE_1D, self.rope1, T,
                None, T, 0, 0, H, d, dt, self.q, self.k, self.v)),
            ("attn_temporal", lambda: L.st_attn_temporal(self.q, self.k, self.v, B, S, T, self.t_valid, H, d,
                                                         self.scale, dt, None, 0, self.o)),
            ("proj_temporal", lambda: L.st_out_proj(self.o, N, self.hd, wt["w_o"], C, dt, self.h)),
            ("relayout_bwd", lambda: L.st_relayout(self.h, bwd[1], self.y, bwd[2], bwd[0], 4, eb)),
        ]

    def run(self, x, fused=True):
        for _, fn in self.steps(x, fused):
            fn()
        return self.y
