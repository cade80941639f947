// C ABI of libst.so: argument validation (host only, before any HIP call),
// dispatch to the bf16 MFMA or fp32 kernels, and the layer-pair orchestration
// of st_block_sliced (ScaleFusion review, "Core innovations": intra-layer
// scheduling and algorithm pseudocode, at one GPU).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "st_internal.h"

using namespace st;

// Device scratch of st_block_sliced_noalloc: every GPU the library runs on
// holds one copy of this array until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in); it uses
// the per-device address that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = size_t(256) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

inline size_t esize(int dt) { return dt == ST_BF16 ? 2 : 4; }
inline bool dtype_ok(int dt) { return dt == ST_BF16 || dt == ST_F32; }

struct Range {
  uintptr_t lo, hi;
};
inline Range rng(const void *p, int64_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool head_dim_ok(int d, int dt, int rope_kind) {
  if (d < 2 || d > 128 || d % 2) return false;
  if (rope_kind == ST_ROPE_2D && d % 4) return false;
  if (dt == ST_BF16) return attn_bf16_supported(d);
  return true;
}

st_status check_rope(int kind, const float *table, int npos, const int32_t *pos, int64_t period, int64_t offset,
                     int grid_w, int d, int64_t rows) {
  if (kind == ST_ROPE_NONE) return ST_OK;
  if (kind != ST_ROPE_1D && kind != ST_ROPE_2D) return ST_EINVAL;
  if (!table || npos < 1) return ST_EINVAL;
  if (!aligned16(table)) return ST_EALIGN;
  if (kind == ST_ROPE_2D && d % 4) return ST_EINVAL;
  if (pos) return (uintptr_t)pos % 8 ? ST_EALIGN : ST_OK;   // positions are device data: range is the caller's
  if (period < 1 || offset < 0) return ST_EINVAL;
  const int64_t imax = std::min<int64_t>(period, std::max<int64_t>(rows, 1)) - 1 + offset;   // largest index used
  if (kind == ST_ROPE_1D) return imax < npos ? ST_OK : ST_EINVAL;
  if (grid_w < 1 || d % 4) return ST_EINVAL;
  if (imax / grid_w >= npos || std::min<int64_t>(grid_w - 1, imax) >= npos) return ST_EINVAL;
  return ST_OK;
}

// ---------------------------------------------------------------- dispatch
// xmap (bf16 only): row r of the projection reads row map_row(r, xmap) of x.
st_status do_qkv(const void *x, int64_t rows, int c_in, const void *w, const float *gq, const float *gk, float eps,
                 float q_scale, const RopeArgs &rope, int H, int d, int dt, void *q, void *k, void *v, hipStream_t s,
                 RowMap xmap = {}) {
  if (dt == ST_BF16) return launch_qkv_bf16(x, rows, c_in, w, gq, gk, eps, q_scale, rope, H, d, q, k, v, s, xmap);
  if (xmap.n1 != 0) return ST_EUNSUPPORTED;
  return launch_qkv_f32((const float *)x, rows, c_in, (const float *)w, gq, gk, eps, q_scale, rope, H, d, (float *)q,
                        (float *)k, (float *)v, s);
}

st_status do_linear(const void *a, int64_t rows, int k_in, const void *w, int n_out, int dt, void *y, hipStream_t s,
                    RowMap ymap = {}) {
  if (dt == ST_BF16) return launch_linear_bf16(a, rows, k_in, w, n_out, y, s, ymap);
  return launch_linear_f32((const float *)a, rows, k_in, (const float *)w, n_out, (float *)y, s, ymap);
}

st_status do_attn(const void *q, const void *k, const void *v, int64_t outer, int L, int nv, int H, int d, float scale,
                  int dt, void *out, bool short_ok, hipStream_t s) {
  if (dt == ST_F32)
    return launch_attn_f32((const float *)q, (const float *)k, (const float *)v, outer, L, nv, H, d, scale,
                           (float *)out, s);
  if (short_ok && attn_short_supported(L, d)) return launch_attn_short_bf16(q, k, v, outer, L, nv, H, d, scale, out, s);
  return launch_attn_bf16(q, k, v, outer, L, nv, H, d, scale, out, s);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct BlockPlan {
  size_t rope2, rope1, xb, hb, xs, xs2, q, k, v, o, ys, ys2, total;
  int npos2, npos1;
};

// explicit_copies: the sliced schedule moves slices with relayout passes (fp32, or
// the two-stream variant) and needs the blocked buffers and double-buffered
// slice buffers; the one-stream bf16 schedule needs only the blocked
// intermediate hb and the per-slice q, k, v, o.
BlockPlan plan_block(int B, int T, int S, int grid_w, int C, int H, int d, int n_t, int n_s, int dt,
                     bool explicit_copies) {
  BlockPlan p{};
  const size_t e = esize(dt);
  const int64_t N = (int64_t)B * T * S;
  const int64_t hd = (int64_t)H * d;
  p.npos2 = std::max(S / grid_w, grid_w);
  p.npos1 = T;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.rope2 = take((size_t)p.npos2 * (d / 4) * 2 * sizeof(float));
  p.rope1 = take((size_t)p.npos1 * (d / 2) * 2 * sizeof(float));
  const bool sliced = n_t > 1 || n_s > 1;
  int64_t rows;
  if (sliced) {
    rows = std::max<int64_t>((int64_t)B * (T / n_t) * S, (int64_t)B * (S / n_s) * T);
    if (explicit_copies) p.xb = take(N * C * e);
    p.hb = take(N * C * e);
    if (explicit_copies) {
      p.xs = take(rows * C * e);
      p.xs2 = take(rows * C * e);   // slice buffers are double-buffered (two-stream pipeline)
    }
  } else {
    p.xs = take(N * C * e);   // [B,S,T,C] input of the temporal layer (the spatial output, relayout fused)
    rows = N;
  }
  p.q = take(rows * hd * e);
  p.k = take(rows * hd * e);
  p.v = take(rows * hd * e);
  p.o = take(rows * hd * e);
  p.ys = sliced && explicit_copies ? take(rows * C * e) : 0;
  p.ys2 = sliced && explicit_copies ? take(rows * C * e) : 0;
  p.total = off;
  return p;
}

}  // namespace

// Scale of q and of the attention inside a layer.  bf16: the projection stores
// q times (1/sqrt(d)) * log2(e), rounded to bf16 once there, and the attention
// runs with scale ln 2, so its exponent base-2 argument is the score itself
// (softmax(q.k/sqrt(d)) unchanged).  fp32: plain q and scale 1/sqrt(d).
extern "C" st_status st_layer_scales(int d, int dtype, float *q_scale, float *attn_scale) {
  if (d < 1 || !dtype_ok(dtype) || !q_scale || !attn_scale) return ST_EINVAL;
  const double s = 1.0 / sqrt((double)d);
  if (dtype == ST_BF16) {
    *q_scale = (float)(s * 1.4426950408889634);
    *attn_scale = (float)0.69314718055994531;
  } else {
    *q_scale = 1.0f;
    *attn_scale = (float)s;
  }
  return ST_OK;
}

namespace {

// One layer: projection + norm/RoPE, attention, output projection.  The
// projection may read its rows through xmap and the output projection store
// them through ymap, which fuses a relayout on either side into the layer.
st_status run_layer(const void *x, int64_t outer, int L, int nv, int C, int H, int d, const st_layer_weights *w,
                    float eps, const RopeArgs &rope, int dt, void *q, void *k, void *v, void *o, void *y,
                    bool temporal, hipStream_t s, RowMap ymap = {}, RowMap xmap = {}) {
  const int64_t rows = outer * L;
  float q_scale, attn_scale;
  st_layer_scales(d, dt, &q_scale, &attn_scale);
  st_status r = do_qkv(x, rows, C, w->w_qkv, w->g_q, w->g_k, eps, q_scale, rope, H, d, dt, q, k, v, s, xmap);
  if (r != ST_OK) return r;
  r = do_attn(q, k, v, outer, L, nv, H, d, attn_scale, dt, o, temporal, s);
  if (r != ST_OK) return r;
  return do_linear(o, rows, H * d, w->w_o, C, dt, y, s, ymap);
}

// Events that order the two streams of the pipelined slicing schedule.  A
// wait covers the work recorded most recently before the wait is enqueued.
struct Events {
  hipEvent_t ev[8] = {};
  int n = 0;
  st_status make(int count) {
    for (n = 0; n < count; ++n)
      if (hipEventCreateWithFlags(&ev[n], hipEventDisableTiming) != hipSuccess) return ST_ELAUNCH;
    return ST_OK;
  }
  ~Events() {
    for (int i = 0; i < n; ++i) hipEventDestroy(ev[i]);   // released once the pending work completes
  }
};

// record on `from`, wait on `to` (no-op for one stream)
st_status order(hipStream_t from, hipStream_t to, hipEvent_t e) {
  if (from == to) return ST_OK;
  if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess) return ST_ELAUNCH;
  return ST_OK;
}

// One layer phase of the slicing schedule over n slices.  gather(i, dst) and
// scatter(i, src) run on `side`, layer(src, dst) on `main`; slice i's gather
// overlaps layer i-1 and its scatter overlaps layer i+1.  xs[2], ys[2] are the
// double-buffered slice inputs and outputs; ev holds 6 events: G[2], L[2], S[2].
template <class Gather, class Layer, class Scatter>
st_status slice_phase(int n, void *const xs[2], void *const ys[2], hipStream_t main, hipStream_t side, hipEvent_t *ev,
                      Gather gather, Layer layer, Scatter scatter) {
  hipEvent_t *G = ev, *Lv = ev + 2, *Sv = ev + 4;
  const bool two = main != side;
  st_status r = gather(0, xs[0]);
  if (r != ST_OK) return r;
  if (two && hipEventRecord(G[0], side) != hipSuccess) return ST_ELAUNCH;
  for (int i = 0; i < n; ++i) {
    const int b = i & 1, nb = b ^ 1;
    if (i + 1 < n) {   // prefetch slice i+1; its buffer was read by layer i-1
      if (two && i >= 1 && hipStreamWaitEvent(side, Lv[nb], 0) != hipSuccess) return ST_ELAUNCH;
      r = gather(i + 1, xs[nb]);
      if (r != ST_OK) return r;
      if (two && hipEventRecord(G[nb], side) != hipSuccess) return ST_ELAUNCH;
    }
    if (two) {
      if (hipStreamWaitEvent(main, G[b], 0) != hipSuccess) return ST_ELAUNCH;
      if (i >= 2 && hipStreamWaitEvent(main, Sv[b], 0) != hipSuccess) return ST_ELAUNCH;   // ys[b] read by scatter i-2
    }
    r = layer(xs[b], ys[b]);
    if (r != ST_OK) return r;
    if (two && (hipEventRecord(Lv[b], main) != hipSuccess || hipStreamWaitEvent(side, Lv[b], 0) != hipSuccess))
      return ST_ELAUNCH;
    r = scatter(i, ys[b]);
    if (r != ST_OK) return r;
    if (two && hipEventRecord(Sv[b], side) != hipSuccess) return ST_ELAUNCH;
  }
  return ST_OK;
}

// Validation of st_block_sliced's arguments other than the workspace (host only).
st_status check_block(const void *x, int B, int T, int t_valid, int S, int grid_w, int C, int H, int d, int n_t,
                      int n_s, const st_layer_weights *spatial, const st_layer_weights *temporal, float eps,
                      float rope_base, int dtype, void *y) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!x || !y || !spatial || !temporal) return ST_EINVAL;
  for (const st_layer_weights *w : {spatial, temporal})
    if (!w->w_qkv || !w->w_o || !w->g_q || !w->g_k) return ST_EINVAL;
  if (B < 1 || T < 1 || S < 1 || C < 1 || H < 1 || grid_w < 1 || n_t < 1 || n_s < 1) return ST_EINVAL;
  if (T % n_t || S % n_s || S % grid_w || t_valid < 1 || t_valid > T) return ST_EINVAL;
  if (d < 4 || d % 4) return ST_EINVAL;
  if (!(eps >= 0.f) || !isfinite(eps) || !(rope_base > 0.f) || !isfinite(rope_base)) return ST_EINVAL;
  if (!head_dim_ok(d, dtype, ST_ROPE_2D)) return ST_EUNSUPPORTED;
  if (dtype == ST_BF16 && (C % 64 || (H * d) % 64)) return ST_EUNSUPPORTED;
  if (C % 4) return ST_EUNSUPPORTED;
  if ((int64_t)B * T * S >= (1ll << 32) / 2) return ST_EUNSUPPORTED;
  if ((int64_t)3 * H * d * C >= (1ll << 31)) return ST_EUNSUPPORTED;   // 32-bit weight offsets
  for (const st_layer_weights *w : {spatial, temporal})
    for (const void *p : {w->w_qkv, w->w_o, (const void *)w->g_q, (const void *)w->g_k})
      if (!aligned16(p)) return ST_EALIGN;
  if (!aligned16(x) || !aligned16(y)) return ST_EALIGN;
  const int64_t bytes = (int64_t)B * T * S * C * (int64_t)esize(dtype);
  if (overlap(rng(x, bytes), rng(y, bytes))) return ST_EINVAL;
  return ST_OK;
}

st_status block_sliced(const void *x, int B, int T, int t_valid, int S, int grid_w, int C, int H, int d, int n_t,
                       int n_s, const st_layer_weights *spatial, const st_layer_weights *temporal, float eps,
                       float rope_base, int dtype, void *y, void *ws, size_t ws_bytes, hipStream_t s,
                       hipStream_t side) {
  const st_status c = check_block(x, B, T, t_valid, S, grid_w, C, H, d, n_t, n_s, spatial, temporal, eps, rope_base,
                                  dtype, y);
  if (c != ST_OK) return c;
  const BlockPlan P = plan_block(B, T, S, grid_w, C, H, d, n_t, n_s, dtype, side != s || dtype != ST_BF16);
  if (!ws || ws_bytes < P.total) return ST_EWORKSPACE;
  if (!aligned16(ws)) return ST_EALIGN;
  const size_t e = esize(dtype);
  const int64_t N = (int64_t)B * T * S;
  const Range rx = rng(x, N * C * e), ry = rng(y, N * C * e), rw = rng(ws, (int64_t)P.total);
  if (overlap(rx, ry) || overlap(ry, rw) || overlap(rx, rw)) return ST_EINVAL;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;

  char *W = static_cast<char *>(ws);
  float *rope2 = reinterpret_cast<float *>(W + P.rope2);
  float *rope1 = reinterpret_cast<float *>(W + P.rope1);
  void *q = W + P.q, *k = W + P.k, *v = W + P.v, *o = W + P.o;
  st_status r = launch_rope_table(d, ST_ROPE_2D, rope_base, P.npos2, rope2, s);
  if (r != ST_OK) return r;
  r = launch_rope_table(d, ST_ROPE_1D, rope_base, P.npos1, rope1, s);
  if (r != ST_OK) return r;
  const RopeArgs r2{ST_ROPE_2D, P.npos2, rope2, S, 0, grid_w};   // rows [.., S]: h = s / W, w = s % W
  const RopeArgs r1{ST_ROPE_1D, P.npos1, rope1, T, 0, 0};        // rows [.., T]: p = t
  const int eb = (int)e;
  const int64_t Cl = C;

  if (n_t == 1 && n_s == 1) {
    // Both relayouts ride on the output projections: the spatial layer's
    // rows (b, t, s) are stored as rows (b, s, t) of the temporal input, and
    // the temporal layer's rows (b, s, t) as rows (b, t, s) of y.
    void *hs = W + P.xs;
    r = run_layer(x, (int64_t)B * T, S, S, C, H, d, spatial, eps, r2, dtype, q, k, v, o, hs, false, s, row_swap(T, S));
    if (r != ST_OK) return r;
    return run_layer(hs, (int64_t)B * S, T, t_valid, C, H, d, temporal, eps, r1, dtype, q, k, v, o, y, true, s,
                     row_swap(S, T));
  }

  const int tt = T / n_t, ss_ = S / n_s;
  if (side == s && dtype == ST_BF16) {
    // Sliced schedule on one stream with every relayout fused into the layers'
    // row addressing: time slice i's projection reads its rows of x where they
    // lie and its output projection stores them into the blocked layout
    // hb[b][i][j][a][e] (a < T/N_T, e < S/N_S); space slice j's projection reads
    // its rows from hb and its output projection stores them at their place in
    // y.  Each slice runs the same kernels on the same rows as with explicit
    // gathers and scatters, so the results are bit-identical to those.
    const int64_t TS = (int64_t)T * S, blk = (int64_t)tt * ss_;
    void *hb = W + P.hb;
    for (int i = 0; i < n_t; ++i) {
      RowMap xm;   // slice row (b, a*S + s) -> x row b*T*S + i*tt*S + a*S + s
      xm.n1 = 1;
      xm.n3 = (int64_t)tt * S;
      xm.s0 = TS;
      xm.s3 = 1;
      xm.base = (int64_t)i * tt * S;
      RowMap ym;   // slice row (b, a, j, e), s = j*ss + e -> hb row ((b*N_T + i)*N_S + j)*tt*ss + a*ss + e
      ym.n1 = tt;
      ym.n2 = n_s;
      ym.n3 = ss_;
      ym.s0 = TS;
      ym.s1 = ss_;
      ym.s2 = blk;
      ym.s3 = 1;
      ym.base = (int64_t)i * n_s * blk;
      r = run_layer(x, (int64_t)B * tt, S, S, C, H, d, spatial, eps, r2, dtype, q, k, v, o, hb, false, s, ym, xm);
      if (r != ST_OK) return r;
    }
    for (int j = 0; j < n_s; ++j) {
      RowMap xm;   // slice row (b, e, i, a), t = i*tt + a -> hb row ((b*N_T + i)*N_S + j)*tt*ss + a*ss + e
      xm.n1 = ss_;
      xm.n2 = n_t;
      xm.n3 = tt;
      xm.s0 = TS;
      xm.s1 = 1;
      xm.s2 = (int64_t)n_s * blk;
      xm.s3 = ss_;
      xm.base = (int64_t)j * blk;
      RowMap ym;   // slice row (b, e, t) -> y row (b*T + t)*S + j*ss + e
      ym.n1 = ss_;
      ym.n2 = T;
      ym.s0 = TS;
      ym.s1 = 1;
      ym.s2 = S;
      ym.base = (int64_t)j * ss_;
      r = run_layer(hb, (int64_t)B * ss_, T, t_valid, C, H, d, temporal, eps, r1, dtype, q, k, v, o, y, true, s, ym,
                    xm);
      if (r != ST_OK) return r;
    }
    return ST_OK;
  }

  // Sliced schedule with explicit relayouts.  Blocked layout xb[b][i][j][a][e][c]
  // with a < T/N_T, e < S/N_S.  Relayouts run on `side`, layers on `s`; with
  // one stream this is the plain order of the pseudocode.
  Events E;
  if (side != s) {
    r = E.make(8);
    if (r != ST_OK) return r;
    r = order(s, side, E.ev[6]);   // the side stream starts after the caller's earlier work
    if (r != ST_OK) return r;
  }
  const int64_t bstr[6] = {(int64_t)n_t * n_s * tt * ss_ * Cl, (int64_t)n_s * tt * ss_ * Cl, (int64_t)tt * ss_ * Cl,
                           ss_ * Cl, Cl, 1};   // strides of [B, N_T, N_S, tt, ss, C]
  void *xb = W + P.xb, *hb = W + P.hb;
  void *const xs[2] = {W + P.xs, W + P.xs2}, *const ys[2] = {W + P.ys, W + P.ys2};
  {  // step 2: x [B,T,S,C] viewed as [B, N_T, tt, N_S, ss, C] -> blocked
    const int64_t dims[6] = {B, n_t, tt, n_s, ss_, C};
    const int64_t sx[6] = {(int64_t)T * S * Cl, (int64_t)tt * S * Cl, S * Cl, ss_ * Cl, Cl, 1};
    const int64_t db[6] = {bstr[0], bstr[1], bstr[3], bstr[2], bstr[4], 1};
    r = launch_relayout(x, sx, xb, db, dims, 6, eb, side);
    if (r != ST_OK) return r;
  }
  {  // spatial layer, one time slice at a time: gather [B, tt, S, C], compute, scatter back
    const int64_t dims[5] = {B, tt, n_s, ss_, C};
    const int64_t sb[5] = {bstr[0], bstr[3], bstr[2], bstr[4], 1};
    const int64_t sc[5] = {(int64_t)tt * S * Cl, S * Cl, ss_ * Cl, Cl, 1};
    r = slice_phase(
        n_t, xs, ys, s, side, E.ev,
        [&](int i, void *dst) {
          return launch_relayout(static_cast<char *>(xb) + (int64_t)i * bstr[1] * eb, sb, dst, sc, dims, 5, eb, side);
        },
        [&](void *src, void *dst) {
          return run_layer(src, (int64_t)B * tt, S, S, C, H, d, spatial, eps, r2, dtype, q, k, v, o, dst, false, s);
        },
        [&](int i, void *src) {
          return launch_relayout(src, sc, static_cast<char *>(hb) + (int64_t)i * bstr[1] * eb, sb, dims, 5, eb, side);
        });
    if (r != ST_OK) return r;
  }
  void *yb = xb;   // temporal results go back into xb (its input was fully consumed by the spatial gathers)
  {  // temporal layer, one space slice at a time: gather [B, ss, T, C], compute, scatter back
    const int64_t dims[5] = {B, n_t, tt, ss_, C};
    const int64_t sb[5] = {bstr[0], bstr[1], bstr[3], bstr[4], 1};
    const int64_t sc[5] = {(int64_t)ss_ * T * Cl, (int64_t)tt * Cl, Cl, (int64_t)T * Cl, 1};
    r = slice_phase(
        n_s, xs, ys, s, side, E.ev,
        [&](int j, void *dst) {
          return launch_relayout(static_cast<const char *>(hb) + (int64_t)j * bstr[2] * eb, sb, dst, sc, dims, 5, eb,
                                 side);
        },
        [&](void *src, void *dst) {
          return run_layer(src, (int64_t)B * ss_, T, t_valid, C, H, d, temporal, eps, r1, dtype, q, k, v, o, dst, true,
                           s);
        },
        [&](int j, void *src) {
          return launch_relayout(src, sc, static_cast<char *>(yb) + (int64_t)j * bstr[2] * eb, sb, dims, 5, eb, side);
        });
    if (r != ST_OK) return r;
  }
  {  // step 10: blocked -> [B, T, S, C]
    const int64_t dims[6] = {B, n_t, tt, n_s, ss_, C};
    const int64_t sx[6] = {(int64_t)T * S * Cl, (int64_t)tt * S * Cl, S * Cl, ss_ * Cl, Cl, 1};
    const int64_t db[6] = {bstr[0], bstr[1], bstr[3], bstr[2], bstr[4], 1};
    r = launch_relayout(yb, db, y, sx, dims, 6, eb, side);
    if (r != ST_OK) return r;
  }
  return order(side, s, E.ev[7]);   // the caller's stream sees the finished output
}

}  // namespace

extern "C" {

const char *st_status_str(int status) {
  switch (status) {
    case ST_OK: return "ok";
    case ST_EINVAL: return "invalid argument";
    case ST_EUNSUPPORTED: return "unsupported";
    case ST_EALIGN: return "misaligned pointer";
    case ST_EWORKSPACE: return "workspace too small";
    case ST_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t st_rope_table_floats(int d, int kind, int n_pos) {
  if (n_pos < 1 || d < 2) return 0;
  if (kind == ST_ROPE_1D) return (size_t)n_pos * (d / 2) * 2;
  if (kind == ST_ROPE_2D) return (size_t)n_pos * (d / 4) * 2;
  return 0;
}

st_status st_rope_table(int d, int kind, float base, int n_pos, float *table, void *stream) {
  if (kind != ST_ROPE_1D && kind != ST_ROPE_2D) return ST_EINVAL;
  if (d < 2 || d > 4096 || d % 2 || (kind == ST_ROPE_2D && d % 4)) return ST_EINVAL;
  if (n_pos < 1 || !(base > 0.f) || !isfinite(base) || !table) return ST_EINVAL;
  if (!aligned16(table)) return ST_EALIGN;
  if ((int64_t)n_pos * d >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return launch_rope_table(d, kind, (double)base, n_pos, table, (hipStream_t)stream);
}

st_status st_qkv_norm_rope(const void *x, int64_t rows, int c_in, const void *w_qkv, const float *g_q,
                           const float *g_k, float eps, float q_scale, int rope_kind, const float *rope_table,
                           int rope_npos, const int32_t *pos, int64_t pos_period, int64_t pos_offset, int grid_w, int H,
                           int d, int dtype, void *q, void *k, void *v, void *stream) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!x || !w_qkv || !g_q || !g_k || !q || !k || !v) return ST_EINVAL;
  if (rows < 0 || c_in < 1 || H < 1 || !(eps >= 0.f) || !isfinite(eps)) return ST_EINVAL;
  if (!(q_scale > 0.f) || !isfinite(q_scale)) return ST_EINVAL;
  if (rope_kind != ST_ROPE_NONE && rope_kind != ST_ROPE_1D && rope_kind != ST_ROPE_2D) return ST_EINVAL;
  if (d < 2 || d % 2 || (rope_kind == ST_ROPE_2D && d % 4)) return ST_EINVAL;
  if (!head_dim_ok(d, dtype, rope_kind)) return ST_EUNSUPPORTED;
  if (dtype == ST_BF16 && c_in % 64) return ST_EUNSUPPORTED;
  const st_status rs = check_rope(rope_kind, rope_table, rope_npos, pos, pos_period, pos_offset, grid_w, d, rows);
  if (rs != ST_OK) return rs;
  // the projection kernels index the weight matrix with 32-bit offsets
  if ((int64_t)H * d * 3 * c_in >= (1ll << 31) || rows >= (1ll << 40)) return ST_EUNSUPPORTED;
  for (const void *p : {x, w_qkv, (const void *)g_q, (const void *)g_k, (const void *)q, (const void *)k,
                        (const void *)v})
    if (!aligned16(p)) return ST_EALIGN;
  const size_t e = esize(dtype);
  const Range rx = rng(x, rows * c_in * e), rw = rng(w_qkv, (int64_t)3 * H * d * c_in * e);
  const Range rq = rng(q, rows * H * d * e), rk = rng(k, rows * H * d * e), rv = rng(v, rows * H * d * e);
  for (Range out : {rq, rk, rv})
    if (overlap(out, rx) || overlap(out, rw)) return ST_EINVAL;
  if (overlap(rq, rk) || overlap(rq, rv) || overlap(rk, rv)) return ST_EINVAL;
  const int32_t *p = rope_kind == ST_ROPE_NONE ? nullptr : pos;
  if (p)
    for (Range out : {rq, rk, rv})
      if (overlap(out, rng(p, rows * 8))) return ST_EINVAL;
  RopeArgs ra{rope_kind, rope_npos, rope_table, pos_period, pos_offset, grid_w, p};
  if (rows == 0) return ST_OK;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return do_qkv(x, rows, c_in, w_qkv, g_q, g_k, eps, q_scale, ra, H, d, dtype, q, k, v, (hipStream_t)stream);
}

st_status st_out_proj(const void *a, int64_t rows, int k_in, const void *w, int n_out, int dtype, void *y,
                      void *stream) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!a || !w || !y || rows < 0 || k_in < 1 || n_out < 1) return ST_EINVAL;
  if (n_out % 4 || (dtype == ST_BF16 && k_in % 64)) return ST_EUNSUPPORTED;
  if (rows >= (1ll << 40) || (int64_t)k_in * n_out >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y)) return ST_EALIGN;
  const size_t e = esize(dtype);
  const Range ry = rng(y, rows * n_out * e);
  if (overlap(ry, rng(a, rows * k_in * e)) || overlap(ry, rng(w, (int64_t)n_out * k_in * e))) return ST_EINVAL;
  if (rows == 0) return ST_OK;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return do_linear(a, rows, k_in, w, n_out, dtype, y, (hipStream_t)stream);
}

st_status st_out_proj_relayout(const void *a, int64_t rows, int k_in, const void *w, int n_out, int dtype,
                               int64_t n1, int64_t n2, void *y, void *stream) {
  if (n1 < 1 || n2 < 1 || n1 >= (1ll << 31) || n2 >= (1ll << 31) || rows < 0 || rows % (n1 * n2)) return ST_EINVAL;
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!a || !w || !y || k_in < 1 || n_out < 1) return ST_EINVAL;
  if (n_out % 4 || (dtype == ST_BF16 && k_in % 64)) return ST_EUNSUPPORTED;
  if (rows >= (1ll << 40) || (int64_t)k_in * n_out >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y)) return ST_EALIGN;
  const size_t e = esize(dtype);
  const Range ry = rng(y, rows * n_out * e);
  if (overlap(ry, rng(a, rows * k_in * e)) || overlap(ry, rng(w, (int64_t)n_out * k_in * e))) return ST_EINVAL;
  if (rows == 0) return ST_OK;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return do_linear(a, rows, k_in, w, n_out, dtype, y, (hipStream_t)stream, row_swap(n1, n2));
}

size_t st_attn_workspace(int64_t rows, int H, int d, int dtype) {
  if (rows < 0 || H < 1 || d < 1 || !dtype_ok(dtype) || rows >= (1ll << 40)) return 0;
  return align256((size_t)rows * H * d * esize(dtype));
}

// w_o != NULL: the attention output is staged in ws and out = O . w_o^T.
static st_status attn_common(const void *q, const void *k, const void *v, int64_t outer, int L, int nv, int H, int d,
                             float scale, int dtype, const void *w_o, int c_out, void *out, void *ws, size_t ws_bytes,
                             bool temporal, void *stream) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!q || !k || !v || !out || H < 1 || d < 2 || d % 2) return ST_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ST_EINVAL;
  if (w_o && c_out < 1) return ST_EINVAL;
  if (!head_dim_ok(d, dtype, ST_ROPE_NONE)) return ST_EUNSUPPORTED;
  if (outer >= (1ll << 40) || L >= (1 << 30)) return ST_EUNSUPPORTED;
  if (w_o && (c_out % 4 || (dtype == ST_BF16 && (H * d) % 64) || (int64_t)H * d * c_out >= (1ll << 31)))
    return ST_EUNSUPPORTED;
  for (const void *p : {q, k, v, (const void *)out})
    if (!aligned16(p)) return ST_EALIGN;
  const int64_t rows = outer * L;
  const int64_t e = (int64_t)esize(dtype), bytes = rows * H * d * e;
  const Range rq = rng(q, bytes), rk = rng(k, bytes), rv = rng(v, bytes);
  const Range ro = rng(out, w_o ? rows * c_out * e : bytes);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv)) return ST_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0) return ST_OK;
  if (!w_o) {
    if (const st_status dc = device_ok(); dc != ST_OK) return dc;
    return do_attn(q, k, v, outer, L, nv, H, d, scale, dtype, out, temporal, s);
  }
  if (!ws || ws_bytes < st_attn_workspace(rows, H, d, dtype)) return ST_EWORKSPACE;
  if (!aligned16(w_o) || !aligned16(ws)) return ST_EALIGN;
  const Range rw = rng(w_o, (int64_t)c_out * H * d * e), rs = rng(ws, bytes);
  if (overlap(ro, rw) || overlap(ro, rs)) return ST_EINVAL;
  for (const Range &in : {rq, rk, rv, rw})
    if (overlap(rs, in)) return ST_EINVAL;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  const st_status r = do_attn(q, k, v, outer, L, nv, H, d, scale, dtype, ws, temporal, s);
  if (r != ST_OK) return r;
  return do_linear(ws, rows, H * d, w_o, c_out, dtype, out, s);
}

st_status st_attn_spatial(const void *q, const void *k, const void *v, int B, int T, int S, int H, int d, float scale,
                          int dtype, const void *w_o, int c_out, void *out, void *ws, size_t ws_bytes, void *stream) {
  if (B < 0 || T < 0 || S < 0) return ST_EINVAL;
  return attn_common(q, k, v, (int64_t)B * T, S, S, H, d, scale, dtype, w_o, c_out, out, ws, ws_bytes, false, stream);
}

st_status st_attn_temporal(const void *q, const void *k, const void *v, int B, int S, int T, int t_valid, int H, int d,
                           float scale, int dtype, const void *w_o, int c_out, void *out, void *ws, size_t ws_bytes,
                           void *stream) {
  if (B < 0 || S < 0 || T < 0) return ST_EINVAL;
  if (T > 0 && (t_valid < 1 || t_valid > T)) return ST_EINVAL;
  return attn_common(q, k, v, (int64_t)B * S, T, t_valid, H, d, scale, dtype, w_o, c_out, out, ws, ws_bytes, true,
                     stream);
}

static st_status chunk_check(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk, int kv_valid,
                             int H, int d, float scale, int dtype, void *out, float *lse) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!q || !k || !v || !out || !lse || H < 1 || outer < 0 || Lq < 0 || Lk < 0) return ST_EINVAL;
  if (kv_valid < 0 || kv_valid > Lk || d < 2 || d % 2) return ST_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ST_EINVAL;
  if (!head_dim_ok(d, dtype, ST_ROPE_NONE)) return ST_EUNSUPPORTED;
  if (outer >= (1ll << 40) || Lq >= (1 << 30) || Lk >= (1 << 30)) return ST_EUNSUPPORTED;
  for (const void *p : {q, k, v, (const void *)out})
    if (!aligned16(p)) return ST_EALIGN;
  if ((uintptr_t)lse % 4) return ST_EALIGN;
  const int64_t e = (int64_t)esize(dtype);
  const Range ro = rng(out, outer * Lq * H * d * e), rl = rng(lse, outer * H * Lq * 4);
  const Range rq = rng(q, outer * Lq * H * d * e), rk = rng(k, outer * Lk * H * d * e), rv = rng(v, outer * Lk * H * d * e);
  for (const Range &in : {rq, rk, rv})
    if (overlap(ro, in) || overlap(rl, in)) return ST_EINVAL;
  if (overlap(ro, rl)) return ST_EINVAL;
  return ST_OK;
}

st_status st_attn_chunk(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk, int kv_valid,
                        int H, int d, float scale, int dtype, void *out, float *lse, void *stream) {
  const st_status c = chunk_check(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dtype, out, lse);
  if (c != ST_OK) return c;
  if (outer == 0 || Lq == 0) return ST_OK;
  hipStream_t s = (hipStream_t)stream;
  const int e = (int)esize(dtype);
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  if (kv_valid == 0) return launch_attn_empty(out, lse, outer, Lq, H, d, e, s);
  if (dtype == ST_F32)
    return launch_attn_chunk_f32((const float *)q, (const float *)k, (const float *)v, outer, Lq, Lk, kv_valid, H, d,
                                 scale, (float *)out, lse, s);
  return launch_attn_chunk_bf16(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, out, lse, s);
}

st_status st_attn_chunk_acc(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk, int kv_valid,
                            int H, int d, float scale, int dtype, void *acc_o, float *acc_lse, void *stream) {
  const st_status c = chunk_check(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, dtype, acc_o, acc_lse);
  if (c != ST_OK) return c;
  if (outer == 0 || Lq == 0 || kv_valid == 0) return ST_OK;   // an empty chunk leaves the accumulator as it is
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == ST_F32)
    return launch_attn_chunk_f32((const float *)q, (const float *)k, (const float *)v, outer, Lq, Lk, kv_valid, H, d,
                                 scale, (float *)acc_o, acc_lse, s, true);
  return launch_attn_chunk_bf16(q, k, v, outer, Lq, Lk, kv_valid, H, d, scale, acc_o, acc_lse, s, true);
}

st_status st_attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t outer, int L,
                        int H, int d, int dtype, void *out, float *lse, void *stream) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!o_a || !lse_a || !o_b || !lse_b || !out || !lse || outer < 0 || L < 0 || H < 1 || d < 1) return ST_EINVAL;
  if (outer >= (1ll << 40) || L >= (1 << 30) || d > 4096) return ST_EUNSUPPORTED;
  for (const void *p : {o_a, o_b, (const void *)out})
    if (!aligned16(p)) return ST_EALIGN;
  for (const float *p : {lse_a, lse_b, (const float *)lse})
    if ((uintptr_t)p % 4) return ST_EALIGN;
  const int64_t ob = outer * L * H * d * (int64_t)esize(dtype), lb = outer * H * L * 4;
  const Range ro = rng(out, ob), rl = rng(lse, lb);
  const Range ra = rng(o_a, ob), rb = rng(o_b, ob), rla = rng(lse_a, lb), rlb = rng(lse_b, lb);
  // in place on either input is fine (each row is read before it is written); partial overlap is not
  if ((overlap(ro, ra) && out != o_a) || (overlap(ro, rb) && out != o_b)) return ST_EINVAL;
  if ((overlap(rl, rla) && lse != lse_a) || (overlap(rl, rlb) && lse != lse_b)) return ST_EINVAL;
  for (const Range &x : {rl, rla, rlb})
    if (overlap(ro, x) || overlap(ra, x) || overlap(rb, x)) return ST_EINVAL;
  if (outer == 0 || L == 0) return ST_OK;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return launch_attn_merge(o_a, lse_a, o_b, lse_b, outer, L, H, d, (int)esize(dtype), out, lse, (hipStream_t)stream);
}

st_status st_v_change(const void *v_new, void *v_cache, int64_t rows, int H, int d, float threshold, int dtype,
                      uint8_t *mask, int32_t *active_idx, int64_t *n_active, int update_cache, void *stream) {
  if (!dtype_ok(dtype)) return ST_EINVAL;
  if (!v_new || !v_cache || !mask || !n_active || rows < 0 || H < 1 || d < 1) return ST_EINVAL;
  if (isnan(threshold) || threshold < 0.f) return ST_EINVAL;
  const int64_t e = (int64_t)esize(dtype);
  if ((d * e) % 16 || d * e > 512) return ST_EUNSUPPORTED;
  const int64_t nvec = rows * H;
  if (rows >= (1ll << 40) || nvec >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (!aligned16(v_new) || !aligned16(v_cache)) return ST_EALIGN;
  if ((uintptr_t)n_active % 8 || (uintptr_t)active_idx % 4 || !aligned16(mask)) return ST_EALIGN;
  const Range rn = rng(v_new, nvec * d * e), rc = rng(v_cache, nvec * d * e), rm = rng(mask, nvec),
              ri = rng(active_idx, active_idx ? nvec * 4 : 0), rk = rng(n_active, 8);
  if (overlap(rn, rc)) return ST_EINVAL;
  for (const Range &o : {rm, ri, rk})
    if (overlap(o, rn) || overlap(o, rc)) return ST_EINVAL;
  if (overlap(rm, ri) || overlap(rm, rk) || overlap(ri, rk)) return ST_EINVAL;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return launch_v_change(v_new, v_cache, nvec, d, (int)e, threshold, mask, active_idx, n_active, update_cache,
                         (hipStream_t)stream);
}

st_status st_relayout(const void *src, const int64_t *src_strides, void *dst, const int64_t *dst_strides,
                      const int64_t *dims, int ndim, int elem_bytes, void *stream) {
  if (!src || !dst || !src_strides || !dst_strides || !dims) return ST_EINVAL;
  if (ndim < 1 || ndim > 6) return ST_EINVAL;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16) return ST_EINVAL;
  if (src == dst) return ST_EINVAL;
  int64_t smin = 0, smax = 0, dmin = 0, dmax = 0;
  bool empty = false;
  for (int i = 0; i < ndim; ++i) {
    if (dims[i] < 0) return ST_EINVAL;
    if (dims[i] == 0) empty = true;
    const int64_t ext = dims[i] > 0 ? dims[i] - 1 : 0;
    (src_strides[i] >= 0 ? smax : smin) += src_strides[i] * ext;
    (dst_strides[i] >= 0 ? dmax : dmin) += dst_strides[i] * ext;
  }
  if ((uintptr_t)src % elem_bytes || (uintptr_t)dst % elem_bytes) return ST_EALIGN;
  if (empty) return ST_OK;
  const Range rs{(uintptr_t)src + smin * elem_bytes, (uintptr_t)src + (smax + 1) * elem_bytes};
  const Range rd{(uintptr_t)dst + dmin * elem_bytes, (uintptr_t)dst + (dmax + 1) * elem_bytes};
  if (overlap(rs, rd)) return ST_EINVAL;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return launch_relayout(src, src_strides, dst, dst_strides, dims, ndim, elem_bytes, (hipStream_t)stream);
}

size_t st_block_sliced_workspace(int B, int T, int S, int grid_w, int C, int H, int d, int n_t, int n_s, int dtype) {
  if (B < 1 || T < 1 || S < 1 || grid_w < 1 || C < 1 || H < 1 || d < 4 || n_t < 1 || n_s < 1 || !dtype_ok(dtype))
    return 0;
  if (T % n_t || S % n_s || S % grid_w) return 0;
  return plan_block(B, T, S, grid_w, C, H, d, n_t, n_s, dtype, dtype != ST_BF16).total;
}

size_t st_block_sliced_2s_workspace(int B, int T, int S, int grid_w, int C, int H, int d, int n_t, int n_s,
                                    int dtype) {
  if (B < 1 || T < 1 || S < 1 || grid_w < 1 || C < 1 || H < 1 || d < 4 || n_t < 1 || n_s < 1 || !dtype_ok(dtype))
    return 0;
  if (T % n_t || S % n_s || S % grid_w) return 0;
  return plan_block(B, T, S, grid_w, C, H, d, n_t, n_s, dtype, true).total;
}

st_status st_block_sliced(const void *x, int B, int T, int t_valid, int S, int grid_w, int C, int H, int d, int n_t,
                          int n_s, const st_layer_weights *spatial, const st_layer_weights *temporal, float eps,
                          float rope_base, int dtype, void *y, void *ws, size_t ws_bytes, void *stream) {
  return block_sliced(x, B, T, t_valid, S, grid_w, C, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype, y, ws,
                      ws_bytes, (hipStream_t)stream, (hipStream_t)stream);
}

// Per-device address of the scratch array, looked up once per device, with
// that device current, on the first call there.
static std::mutex scratch_mu;
static void *scratch_dev[64];

static st_status scratch_for_current_device(void **p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ST_ELAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ST_ELAUNCH;
    scratch_dev[dev] = ptr;
  }
  *p = scratch_dev[dev];
  return ST_OK;
}

size_t st_block_sliced_noalloc_max(void) { return kScratchBytes; }

st_status st_block_sliced_noalloc(const void *x, int B, int T, int t_valid, int S, int grid_w, int C, int H, int d,
                                  int n_t, int n_s, const st_layer_weights *spatial, const st_layer_weights *temporal,
                                  float eps, float rope_base, int dtype, void *y, void *stream) {
  const st_status c = check_block(x, B, T, t_valid, S, grid_w, C, H, d, n_t, n_s, spatial, temporal, eps, rope_base,
                                  dtype, y);
  if (c != ST_OK) return c;
  const size_t need = st_block_sliced_workspace(B, T, S, grid_w, C, H, d, n_t, n_s, dtype);
  if (need == 0 || need > kScratchBytes) return ST_EWORKSPACE;
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  void *ws = nullptr;
  const st_status r = scratch_for_current_device(&ws);
  if (r != ST_OK) return r;
  return block_sliced(x, B, T, t_valid, S, grid_w, C, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype, y, ws,
                      kScratchBytes, (hipStream_t)stream, (hipStream_t)stream);
}

st_status st_block_sliced_2s(const void *x, int B, int T, int t_valid, int S, int grid_w, int C, int H, int d, int n_t,
                             int n_s, const st_layer_weights *spatial, const st_layer_weights *temporal, float eps,
                             float rope_base, int dtype, void *y, void *ws, size_t ws_bytes, void *stream,
                             void *side_stream) {
  if (!side_stream || side_stream == stream) return ST_EINVAL;
  return block_sliced(x, B, T, t_valid, S, grid_w, C, H, d, n_t, n_s, spatial, temporal, eps, rope_base, dtype, y, ws,
                      ws_bytes, (hipStream_t)stream, (hipStream_t)side_stream);
}

}  // extern "C"
