// fp32 kernels of the attention block, for fp32 storage (small correctness
// workloads).  Same operations as the bf16 MFMA path -- projection, per-head
// RMSNorm and RoPE on q and k (CoCoDiff page, "V-First compute scheduling"),
// attention over the middle axis of [outer, L, H, d] -- written as plain
// per-thread fp32 loops: one thread per output element of a projection, one
// per (row, head) for the normalisation, one per query for attention.
#include <math.h>

#include "st_internal.h"

namespace st {
namespace {

// y[r, n] = sum_k a[r, k] * w[n, k]; output row r of column n goes to
// dst_for(n) with its own row stride (q/k/v split) or to y.
__global__ void linear_f32_kernel(const float *a, int64_t rows, int K, const float *w, int N, float *y, RowMap ym) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * N) return;
  const int64_t r = i / N;
  const int n = (int)(i % N);
  const float *ar = a + r * K, *wr = w + (int64_t)n * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(ar[k], wr[k], acc);
  y[map_row(r, ym) * N + n] = acc;
}

__global__ void qkv_f32_kernel(const float *x, int64_t rows, int K, const float *w, int H, int d, float *q,
                               float *k, float *v) {
  const int N = 3 * H * d;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * N) return;
  const int64_t r = i / N;
  const int n = (int)(i % N);
  const float *xr = x + r * K, *wr = w + (int64_t)n * K;
  float acc = 0.f;
  for (int kk = 0; kk < K; ++kk) acc = fmaf(xr[kk], wr[kk], acc);
  const int which = n / (H * d), c = n % (H * d);
  float *dst = which == 0 ? q : (which == 1 ? k : v);
  dst[r * H * d + c] = acc;
}

// In place on q and k: RMSNorm over d, then RoPE.  One thread per (row, head, tensor).
__global__ void norm_rope_f32_kernel(int64_t rows, int H, int d, float *q, float *k, const float *g_q,
                                     const float *g_k, float eps, float q_scale, RopeArgs rope) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * H * 2) return;
  const int which = (int)(i % 2);
  const int64_t rh = i / 2;
  const int64_t r = rh / H;
  float *t = (which == 0 ? q : k) + rh * d;
  const float *g = which == 0 ? g_q : g_k;
  float ss = 0.f;
  for (int j = 0; j < d; ++j) ss = fmaf(t[j], t[j], ss);
  const float inv = rsqrtf(ss / (float)d + eps);
  const float qs = which == 0 ? q_scale : 1.0f;
  for (int j = 0; j < d; ++j) t[j] = t[j] * inv * (g[j] * qs);
  if (rope.kind == ST_ROPE_NONE) return;
  int p0, p1 = 0;
  if (rope.pos) {   // caller's positions, clamped into the table
    p0 = min(max(rope.pos[2 * r], 0), rope.npos - 1);
    p1 = min(max(rope.pos[2 * r + 1], 0), rope.npos - 1);
  } else {
    const int64_t pi = r % rope.period + rope.offset;
    if (rope.kind == ST_ROPE_1D) {
      p0 = (int)pi;
    } else {
      p0 = (int)(pi / rope.grid_w);
      p1 = (int)(pi % rope.grid_w);
    }
  }
  const int npairs = rope.kind == ST_ROPE_2D ? d / 4 : d / 2;
  for (int j = 0; j < d; j += 2) {
    int pos = p0, pair = j / 2;
    if (rope.kind == ST_ROPE_2D && j >= d / 2) {
      pos = p1;
      pair = (j - d / 2) / 2;
    }
    const float c = rope.table[((int64_t)pos * npairs + pair) * 2];
    const float s = rope.table[((int64_t)pos * npairs + pair) * 2 + 1];
    const float a = t[j], b = t[j + 1];
    t[j] = a * c - b * s;
    t[j + 1] = a * s + b * c;
  }
}

// One thread per (outer, head, query): two passes over the keys.
// One thread per (sequence, head, query); L queries over Lk keys, the first nv
// of them valid (nv >= 1).  lse (optional, [outer, H, L]) gets m + log(l).
// With acc, o and lse hold a partial result over other keys and receive its
// merge with this one (weights exp(lse_part - lse_union)).
__global__ void attn_f32_kernel(const float *q, const float *k, const float *v, int64_t outer, int L, int Lk, int nv,
                                int H, int d, float scale, float *o, float *lse, int acc_mode) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= outer * H * L) return;
  const int qi = (int)(i % L);
  const int64_t oh = i / L;
  const int h = (int)(oh % H);
  const int64_t ou = oh / H;
  const int64_t rs = (int64_t)H * d;
  const int64_t base = ou * L * rs + (int64_t)h * d;
  const int64_t kbase = ou * Lk * rs + (int64_t)h * d;
  const float *qr = q + base + qi * rs;
  float m = -INFINITY;
  for (int j = 0; j < nv; ++j) {
    const float *kr = k + kbase + j * rs;
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(qr[c], kr[c], s);
    m = fmaxf(m, s * scale);
  }
  float acc[128];
  for (int c = 0; c < d; ++c) acc[c] = 0.f;
  float l = 0.f;
  for (int j = 0; j < nv; ++j) {
    const float *kr = k + kbase + j * rs;
    const float *vr = v + kbase + j * rs;
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(qr[c], kr[c], s);
    const float p = expf(s * scale - m);
    l += p;
    for (int c = 0; c < d; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
  }
  float *orow = o + base + qi * rs;
  const float lp = m + logf(l);
  if (acc_mode) {
    const float la = lse[oh * L + qi];
    const float mm = fmaxf(la, lp);
    const float wa = expf(la - mm), wp = expf(lp - mm), tot = wa + wp;
    const float fa = wa / tot, fp = wp / tot;
    for (int c = 0; c < d; ++c) orow[c] = (fa > 0.f ? fa * orow[c] : 0.f) + fp * (acc[c] / l);
    lse[oh * L + qi] = mm + logf(tot);
    return;
  }
  for (int c = 0; c < d; ++c) orow[c] = acc[c] / l;
  if (lse) lse[oh * L + qi] = lp;
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

st_status launch_qkv_f32(const float *x, int64_t rows, int c_in, const float *w, const float *g_q,
                         const float *g_k, float eps, float q_scale, const RopeArgs &rope, int H, int d, float *q,
                         float *k, float *v, hipStream_t s) {
  if (rows == 0) return ST_OK;
  const int64_t n = rows * 3 * H * d;
  if (blocks_for(n) >= (1u << 31) || blocks_for(rows * H * 2) >= (1u << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL(qkv_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, s, x, rows, c_in, w, H, d, q, k, v);
  hipLaunchKernelGGL(norm_rope_f32_kernel, dim3(blocks_for(rows * H * 2)), dim3(256), 0, s, rows, H, d, q, k, g_q,
                     g_k, eps, q_scale, rope);
  return launch_status();
}

st_status launch_linear_f32(const float *a, int64_t rows, int k_in, const float *w, int n_out, float *y,
                            hipStream_t s, RowMap ym) {
  if (rows == 0) return ST_OK;
  const int64_t n = rows * n_out;
  if (blocks_for(n) >= (1u << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL(linear_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, s, a, rows, k_in, w, n_out, y, ym);
  return launch_status();
}

st_status launch_attn_f32(const float *q, const float *k, const float *v, int64_t outer, int L, int n_valid, int H,
                          int d, float scale, float *out, hipStream_t s) {
  const int64_t n = outer * H * L;
  if (n == 0) return ST_OK;
  if (blocks_for(n) >= (1u << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, s, q, k, v, outer, L, L, min(n_valid, L), H,
                     d, scale, out, (float *)nullptr, 0);
  return launch_status();
}

st_status launch_attn_chunk_f32(const float *q, const float *k, const float *v, int64_t outer, int Lq, int Lk,
                                int n_valid, int H, int d, float scale, float *out, float *lse, hipStream_t s,
                                bool accumulate) {
  const int64_t n = outer * H * Lq;
  if (n == 0) return ST_OK;
  if (blocks_for(n) >= (1u << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(blocks_for(n)), dim3(256), 0, s, q, k, v, outer, Lq, Lk,
                     min(n_valid, Lk), H, d, scale, out, lse, accumulate ? 1 : 0);
  return launch_status();
}

}  // namespace st
