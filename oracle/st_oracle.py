"""fp64 CPU oracle of the ST-DiT attention block.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path and imports nothing from it;
the product path never calls it.

Every function is the plain definition of one step, in float64, on inputs that
were rounded to their storage precision before they arrive (bf16 or fp32 values
widened exactly).  There is no intermediate rounding, no blocking and no fusion.

Sources (page titles as printed on the pages):
  [SF]  ScaleFusion review (xllm-io paper-review blog), sections
        "Technical architecture" (layer table, distributed execution flow,
        spatial-temporal independence equations) and "Core innovations"
        (intra-layer scheduling, algorithm pseudocode).
  [CC]  "CoCoDiff: Optimizing Collective Communications for Distributed
        Diffusion Transformer Inference Under Ulysses Sequence Parallelism",
        section "V-First compute scheduling": Q and K get RMSNorm and RoPE after
        the linear projection; V gets neither.
  [PF]  PipeFusion technical summary, "Problem definition": attention cost is
        quadratic in sequence length; sequence parallelism (DeepSpeed-Ulysses,
        Ring-Attention) splits the sequence across devices.
  [VM]  CoCoDiff page, section "V-Major selective communication": per denoising
        step, each V vector is compared with the previous step's by L1
        distance; only vectors whose change exceeds a threshold are active
        (their Q, K, V are communicated), the rest come from the cache.
  [SW]  "Technical Summary: SwiftFusion", sections "Topology-Aware Communication
        Scheduling" (Ring Attention inside a machine) and "Torus Attention"
        (attention computed chunk by chunk as the chunks arrive).

Readings where the pages are silent (each is also listed in the design notes):
  R1  RMSNorm is per head over d, eps = 1e-6, gain vector of length d shared by
      all heads, separate for q and k.
  R2  w_qkv rows: q heads 0..H-1 (channel h*d + j), then k, then v; no biases.
      A layer is projection -> norm/RoPE -> attention -> output projection w_o.
  R3  RoPE rotates adjacent pairs (2i, 2i+1) by theta = p * base^(-2i/m) for an
      axis segment of length m.  1D: one segment (m = d, p = t).  2D axial:
      channels [0, d/2) by patch row h, [d/2, d) by patch column w, with
      s = h * W + w.  base = 10000, positions 0-based and global.
  R4  T is padded to a multiple of N_T with zero frames; keys at t >= t_valid
      are excluded from the temporal softmax (weight exactly 0).
  R5  Ring and Torus attention ([PF], [SW]) compute attention of the local
      queries against one key/value chunk at a time and combine the partial
      results; the pages do not print the combination.  The exact one is used:
      each chunk yields its normalised output and the log-sum-exp of its
      scaled scores (natural log; -inf for a chunk with no valid key), and two
      disjoint chunks combine with weights exp(lse_chunk - lse_union).
  R6  V-Major ([VM]): a "vector" is one (token, head) row of V (d values); its
      distance is sum_j |v_new_j - v_cache_j|; it is active when the distance
      is strictly greater than the caller's threshold (the page gives no
      value); active rows are the ones whose V replaces the cached V.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- #
# Projection, RMSNorm, RoPE                                                    #
# --------------------------------------------------------------------------- #
def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x . w^T with w stored [out, in] (R2).  x [rows, in] -> [rows, out]."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def rms_norm_heads(t: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the last axis ([CC] V-First; R1).

    t [..., d]:  t_j * g_j / sqrt(mean_j t_j^2 + eps)
    """
    ms = np.mean(t * t, axis=-1, keepdims=True)
    return t * np.asarray(g, np.float64) / np.sqrt(ms + eps)


def rope_segment(t: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate adjacent channel pairs of t [rows, ..., m] by theta_i = p * base^(-2i/m) (R3).

    pos: [rows] integer positions, broadcast over the middle axes.
    """
    m = t.shape[-1]
    i = np.arange(m // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / m)
    theta = np.asarray(pos, np.float64).reshape((-1,) + (1,) * (t.ndim - 1)) * inv_freq
    c, s = np.cos(theta), np.sin(theta)
    a, b = t[..., 0::2], t[..., 1::2]
    out = np.empty_like(t)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope(t: np.ndarray, kind: str, pos: np.ndarray, base: float) -> np.ndarray:
    """RoPE on t [rows, H, d].  kind "none" | "1d" (pos [rows]) | "2d" (pos [rows, 2] = (h, w))."""
    if kind == "none":
        return t.copy()
    if kind == "1d":
        return rope_segment(t, pos, base)
    if kind == "2d":
        d = t.shape[-1]
        out = np.empty_like(t)
        out[..., : d // 2] = rope_segment(t[..., : d // 2], pos[:, 0], base)
        out[..., d // 2:] = rope_segment(t[..., d // 2:], pos[:, 1], base)
        return out
    raise ValueError(kind)


def qkv_norm_rope(x, w_qkv, g_q, g_k, eps, H, d, rope_kind, pos, base):
    """Projection, then RMSNorm and RoPE on q and k only; v is the plain projection ([CC] V-First).

    x [rows, C]; returns q, k, v each [rows, H, d].
    """
    qkv = linear(x, w_qkv)
    rows = qkv.shape[0]
    q = qkv[:, 0 * H * d:1 * H * d].reshape(rows, H, d)
    k = qkv[:, 1 * H * d:2 * H * d].reshape(rows, H, d)
    v = qkv[:, 2 * H * d:3 * H * d].reshape(rows, H, d).copy()
    q = rope(rms_norm_heads(q, g_q, eps), rope_kind, pos, base)
    k = rope(rms_norm_heads(k, g_k, eps), rope_kind, pos, base)
    return q, k, v


def positions_2d(S: int, grid_w: int) -> np.ndarray:
    """(h, w) of each patch token s = h * W + w (R3)."""
    s = np.arange(S)
    return np.stack([s // grid_w, s % grid_w], axis=1)


# --------------------------------------------------------------------------- #
# Attention                                                                    #
# --------------------------------------------------------------------------- #
def attention_probs(q: np.ndarray, k: np.ndarray, scale: float, n_valid: int | None = None):
    """Softmax weights of one sequence: P = softmax(q k^T * scale) over the keys.

    q [Lq, d], k [Lk, d].  Keys j >= n_valid get weight exactly 0 (R4).
    """
    z = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    if n_valid is not None and n_valid < z.shape[1]:
        z[:, n_valid:] = -np.inf
    m = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - m)
    return p / np.sum(p, axis=1, keepdims=True)


def attention(q, k, v, scale: float, n_valid: int | None = None) -> np.ndarray:
    """O = softmax(q k^T * scale) v for one sequence; q, k, v [L, d]."""
    return attention_probs(q, k, scale, n_valid) @ np.asarray(v, np.float64)


def attention_lse(q, k, v, scale: float, n_valid: int | None = None):
    """Attention of q [Lq, d] over one key/value chunk k, v [Lk, d], and its log-sum-exp (R5).

    Returns (o [Lq, d], lse [Lq]): o = softmax(q k^T * scale) v over the chunk's valid keys
    (j < n_valid), lse_i = log sum_j exp(scale * q_i . k_j) over the same keys.  A chunk with
    no valid key gives o = 0 and lse = -inf.
    """
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    nv = k.shape[0] if n_valid is None else min(n_valid, k.shape[0])
    if nv == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    z = (q @ k[:nv].T) * scale
    m = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - m)
    l = np.sum(p, axis=1, keepdims=True)
    return (p / l) @ v[:nv], (m + np.log(l))[:, 0]


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets from the two partial results (R5).

    o_* [..., L, d] normalised partial outputs, lse_* [..., L].  The union's softmax mass is
    exp(lse_a) + exp(lse_b); each part's output is weighted by its share of it.
    """
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    ms = np.where(empty, 0.0, m)
    wa, wb = np.exp(lse_a - ms), np.exp(lse_b - ms)
    tot = wa + wb
    lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, tot)))
    den = np.where(empty, 1.0, tot)[..., None]
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / den
    return np.where(empty[..., None], 0.0, o), lse


def attn_chunk(q, k, v, scale: float, kv_valid: int | None = None):
    """Chunk attention over the middle axis: q [outer, Lq, H, d], k, v [outer, Lk, H, d].

    Returns o [outer, Lq, H, d] and lse [outer, H, Lq] (R5); keys j >= kv_valid excluded.
    """
    outer, Lq, H, d = q.shape
    o = np.empty((outer, Lq, H, d))
    lse = np.empty((outer, H, Lq))
    for b in range(outer):
        for h in range(H):
            o[b, :, h], lse[b, h] = attention_lse(q[b, :, h], k[b, :, h], v[b, :, h], scale, kv_valid)
    return o, lse


def merge_chunks(o_a, lse_a, o_b, lse_b):
    """merge_partials over [outer, L, H, d] outputs with [outer, H, L] log-sum-exps."""
    oa = np.moveaxis(np.asarray(o_a, np.float64), 2, 1)   # [outer, H, L, d]
    ob = np.moveaxis(np.asarray(o_b, np.float64), 2, 1)
    o, lse = merge_partials(oa, lse_a, ob, lse_b)
    return np.moveaxis(o, 1, 2), lse


def attn_spatial(q, k, v, scale: float) -> np.ndarray:
    """Spatial attention: q, k, v [B, T, S, H, d]; one sequence over S per (b, t, h) ([SF] layer table)."""
    B, T, S, H, d = q.shape
    out = np.empty((B, T, S, H, d))
    for b in range(B):
        for t in range(T):
            for h in range(H):
                out[b, t, :, h] = attention(q[b, t, :, h], k[b, t, :, h], v[b, t, :, h], scale)
    return out


def attn_temporal(q, k, v, scale: float, t_valid: int | None = None) -> np.ndarray:
    """Temporal attention: q, k, v [B, S, T, H, d]; one sequence over T per (b, s, h) ([SF] layer table).

    The (b, s, h) sequences are independent, so they are handled as one batch of
    small matrices; each is the same definition as attention().
    """
    B, S, T, H, d = q.shape
    qq = np.moveaxis(np.asarray(q, np.float64), 3, 2).reshape(B * S * H, T, d)
    kk = np.moveaxis(np.asarray(k, np.float64), 3, 2).reshape(B * S * H, T, d)
    vv = np.moveaxis(np.asarray(v, np.float64), 3, 2).reshape(B * S * H, T, d)
    z = np.matmul(qq, np.swapaxes(kk, 1, 2)) * scale
    if t_valid is not None and t_valid < T:
        z[:, :, t_valid:] = -np.inf
    m = np.max(z, axis=2, keepdims=True)
    p = np.exp(z - m)
    p /= np.sum(p, axis=2, keepdims=True)
    o = np.matmul(p, vv).reshape(B, S, H, T, d)
    return np.moveaxis(o, 2, 3)


# --------------------------------------------------------------------------- #
# Relayouts (pure index maps)                                                  #
# --------------------------------------------------------------------------- #
def bt_to_bs(x: np.ndarray) -> np.ndarray:
    """[B, T, S, C] -> [B, S, T, C]: the one-GPU form of the spatial<->temporal all-to-all ([SF] execution flow)."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def bs_to_bt(x: np.ndarray) -> np.ndarray:
    """[B, S, T, C] -> [B, T, S, C]."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def to_blocked(x: np.ndarray, n_t: int, n_s: int) -> np.ndarray:
    """[B, T, S, C] -> [B, N_T, N_S, T/N_T, S/N_S, C] ([SF] intra-layer scheduling, step 2, P = 1)."""
    B, T, S, C = x.shape
    y = x.reshape(B, n_t, T // n_t, n_s, S // n_s, C)
    return np.ascontiguousarray(np.transpose(y, (0, 1, 3, 2, 4, 5)))


def from_blocked(xb: np.ndarray) -> np.ndarray:
    """Inverse of to_blocked: [B, N_T, N_S, T/N_T, S/N_S, C] -> [B, T, S, C]."""
    B, n_t, n_s, tt, ss, C = xb.shape
    return np.ascontiguousarray(np.transpose(xb, (0, 1, 3, 2, 4, 5))).reshape(B, n_t * tt, n_s * ss, C)


# --------------------------------------------------------------------------- #
# Layers and the block                                                         #
# --------------------------------------------------------------------------- #
# --------------------------------------------------------------------------- #
# The all-to-all between the two shardings ([SF] layer table, execution flow)  #
# --------------------------------------------------------------------------- #
def shard(x: np.ndarray, P: int, axis: int) -> list:
    """x [B, T, S, C] split into P equal blocks along axis 1 (frames) or 2 (patches); block r is rank r's."""
    n = x.shape[axis] // P
    return [np.take(x, np.arange(r * n, (r + 1) * n), axis=axis) for r in range(P)]


def all_to_all(send: list) -> list:
    """send[r][q] is the block rank r sends to rank q; rank q receives recv[q][r] = send[r][q]."""
    P = len(send)
    return [[send[r][q] for r in range(P)] for q in range(P)]


def a2a_s_to_t(shards_s: list) -> list:
    """Patch-sharded [B, T, S/P, C] per rank -> frame-sharded [B, T/P, S, C] per rank (P = 1: identity).

    Rank r sends frame block q of its patches to rank q; rank q lays the received patch blocks
    side by side, in rank order, along S."""
    P = len(shards_s)
    recv = all_to_all([shard(xs, P, 1) for xs in shards_s])
    return [np.concatenate(recv[q], axis=2) for q in range(P)]


def a2a_t_to_s(shards_t: list) -> list:
    """Frame-sharded [B, T/P, S, C] per rank -> patch-sharded [B, T, S/P, C] per rank: the inverse exchange."""
    P = len(shards_t)
    recv = all_to_all([shard(xt, P, 2) for xt in shards_t])
    return [np.concatenate(recv[q], axis=1) for q in range(P)]


# --------------------------------------------------------------------------- #
# V-Major change detection ([VM], R6)                                          #
# --------------------------------------------------------------------------- #
def v_change(v_new, v_cache, threshold: float):
    """v_new, v_cache [rows, H, d] -> (dist [rows, H], active mask [rows, H], active flat
    indices r*H + h in increasing order, refreshed cache: v_new where active, else v_cache)."""
    a, b = np.asarray(v_new, np.float64), np.asarray(v_cache, np.float64)
    dist = np.sum(np.abs(a - b), axis=-1)
    mask = dist > threshold
    cache = np.where(mask[..., None], a, b)
    return dist, mask, np.flatnonzero(mask), cache


def spatial_layer(x, wts: dict, H: int, d: int, grid_w: int, eps: float, base: float):
    """Spatial layer on x [B, T, S, C]: attention over the S patches of each frame."""
    B, T, S, C = x.shape
    pos = np.tile(positions_2d(S, grid_w), (B * T, 1))
    q, k, v = qkv_norm_rope(x.reshape(B * T * S, C), wts["w_qkv"], wts["g_q"], wts["g_k"],
                            eps, H, d, "2d", pos, base)
    sh = (B, T, S, H, d)
    o = attn_spatial(q.reshape(sh), k.reshape(sh), v.reshape(sh), 1.0 / np.sqrt(d))
    return linear(o.reshape(B * T * S, H * d), wts["w_o"]).reshape(B, T, S, -1)


def temporal_layer(x, wts: dict, H: int, d: int, eps: float, base: float, t_valid: int | None = None):
    """Temporal layer on x [B, S, T, C]: attention over the T frames of each patch."""
    B, S, T, C = x.shape
    pos = np.tile(np.arange(T), B * S)
    q, k, v = qkv_norm_rope(x.reshape(B * S * T, C), wts["w_qkv"], wts["g_q"], wts["g_k"],
                            eps, H, d, "1d", pos, base)
    sh = (B, S, T, H, d)
    o = attn_temporal(q.reshape(sh), k.reshape(sh), v.reshape(sh), 1.0 / np.sqrt(d), t_valid)
    return linear(o.reshape(B * S * T, H * d), wts["w_o"]).reshape(B, S, T, -1)


def block(x, ws: dict, wt: dict, H, d, grid_w, eps, base, t_valid=None):
    """Unsliced layer pair on x [B, T, S, C] -> [B, T, S, C] ([SF] distributed execution flow at P = 1)."""
    h = spatial_layer(x, ws, H, d, grid_w, eps, base)
    y = temporal_layer(bt_to_bs(h), wt, H, d, eps, base, t_valid)
    return bs_to_bt(y)


def block_sliced(x, ws: dict, wt: dict, H, d, grid_w, eps, base, n_t: int, n_s: int, t_valid=None):
    """Layer pair under the slicing schedule at P = 1 ([SF] algorithm pseudocode, steps 1-3, 8, 10).

    The communication steps of the pseudocode have no work on one GPU; what is
    left is: rearrange the input into N_T x N_S blocks, run the spatial layer
    on one time slice at a time and the temporal layer on one space slice at a
    time (the spatial-temporal independence identities), rearrange back.
    """
    B, T, S, C = x.shape
    xb = to_blocked(x, n_t, n_s)                        # step 2
    hb = np.empty_like(xb, dtype=np.float64)            # spatial-layer output, blocked
    yb = np.empty_like(xb, dtype=np.float64)            # steps 1, 3: y in the blocked form
    tt, ss = T // n_t, S // n_s
    for i in range(n_t):                                # spatial layer, per time slice
        xs = np.transpose(xb[:, i], (0, 2, 1, 3, 4)).reshape(B, tt, S, C)
        hs = spatial_layer(xs, ws, H, d, grid_w, eps, base)
        hb[:, i] = np.transpose(hs.reshape(B, tt, n_s, ss, C), (0, 2, 1, 3, 4))
    for j in range(n_s):                                # temporal layer, per space slice
        xs = hb[:, :, j].reshape(B, T, ss, C)           # [B, N_T, T/N_T, S/N_S, C] -> [B, T, S/N_S, C]
        ys = temporal_layer(bt_to_bs(xs), wt, H, d, eps, base, t_valid)
        yb[:, :, j] = bs_to_bt(ys).reshape(B, n_t, tt, ss, C)
    return from_blocked(yb)                             # step 10
