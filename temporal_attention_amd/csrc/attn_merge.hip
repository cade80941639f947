// Merge of attention results computed over disjoint key chunks: the step that
// Ring attention (PipeFusion summary, sequence parallelism; SwiftFusion,
// "Topology-Aware Communication Scheduling") and Torus attention (SwiftFusion,
// "Torus Attention") repeat as key/value chunks arrive.  A chunk result is the
// output normalised over the chunk's keys plus the natural log-sum-exp of its
// scaled scores; the union's output weights each part by exp(lse_part -
// lse_union).
//
// Rows (one per (sequence, query, head)) that start 16-byte aligned take the
// blocked kernel: a workgroup takes 32 consecutive queries with all their
// heads (one contiguous run of rows), computes their weights once, reading
// and writing each head's log-sum-exps as one run of 32 floats, then streams
// the rows 16 bytes per thread.  With more than 256 heads such rows take the
// contiguous-pass kernel (a wavefront pass covers floor(64 / pieces)
// consecutive rows); other rows take a group of LPR lanes per row.  In all of
// them every element is read and written by one thread, reads first, so the
// merge may run in place on either input.
// HBM-bound: per row, two rows and two log-sum-exps in, one of each out.
#include <math.h>

#include <algorithm>

#include "st_internal.h"

namespace st {
namespace {

template <typename T> struct Elem;
template <> struct Elem<u16> {
  __device__ static float load(u16 x) { return __uint_as_float((uint32_t)x << 16); }
  __device__ static u16 store(float x) { return (u16)(pack_bf16x2(x, 0.f) & 0xFFFFu); }
};
template <> struct Elem<float> {
  __device__ static float load(float x) { return x; }
  __device__ static float store(float x) { return x; }
};

template <typename T, int LPR>
__global__ void __launch_bounds__(256) attn_merge_kernel(const T *oa, const float *la, const T *ob, const float *lb,
                                                         int64_t rows, int L, int H, int d, T *o, float *lse) {
  constexpr int RPW = 64 / LPR;                 // rows per wavefront pass
  constexpr int VW = 16 / sizeof(T);            // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int j = lane % LPR;
  const bool vec = d % VW == 0;                 // rows start 16-byte aligned
  for (int64_t r0 = wave * RPW; r0 < rows; r0 += nwaves * RPW) {
    const int64_t r = r0 + lane / LPR;          // row in [outer, L, H] order
    if (r >= rows) continue;
    const int h = (int)(r % H);
    const int64_t ql = r / H;                   // outer * L + query
    const int qi = (int)(ql % L);
    const int64_t li = (ql / L * H + h) * (int64_t)L + qi;
    const float a = la[li], b = lb[li];
    const float m = fmaxf(a, b);
    const bool empty = m == -INFINITY;          // neither part has a valid key
    const float wa = empty ? 0.f : expf(a - m), wb = empty ? 0.f : expf(b - m);
    const float tot = wa + wb;
    const float fa = empty ? 0.f : wa / tot, fb = empty ? 0.f : wb / tot;
    const T *ra = oa + r * d, *rb = ob + r * d;
    T *ro = o + r * d;
    if (vec) {
      for (int c = j * VW; c < d; c += LPR * VW) {
        const uint4 x = *reinterpret_cast<const uint4 *>(ra + c), y = *reinterpret_cast<const uint4 *>(rb + c);
        const T *xe = reinterpret_cast<const T *>(&x), *ye = reinterpret_cast<const T *>(&y);
        T z[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e)
          z[e] = Elem<T>::store(fmaf(fa, Elem<T>::load(xe[e]), fb * Elem<T>::load(ye[e])));
        *reinterpret_cast<uint4 *>(ro + c) = *reinterpret_cast<const uint4 *>(z);
      }
    } else {
      for (int c = j; c < d; c += LPR) ro[c] = Elem<T>::store(fmaf(fa, Elem<T>::load(ra[c]), fb * Elem<T>::load(rb[c])));
    }
    if (j == 0) lse[li] = empty ? -INFINITY : m + logf(tot);
  }
}

// Rows of 16-byte-aligned rows with P <= 64 pieces: a wavefront pass takes
// floor(64 / P) consecutive rows as one contiguous run (lane l holds piece l),
// U passes of loads in flight; every lane of a row reads the same two
// log-sum-exps.  I is the index type (32-bit when every row index fits).
template <typename T, typename I, int U>
__global__ void __launch_bounds__(256) attn_merge_flat_kernel(const T *oa, const float *la, const T *ob,
                                                              const float *lb, I rows, I L, I H, int P, T *o,
                                                              float *lse) {
  constexpr int VW = 16 / sizeof(T);            // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int rpw = 64 / P;                       // rows per wavefront pass
  const int rl = lane / P, j = lane - rl * P;   // row within the pass, piece within the row
  const bool used = rl < rpw;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t step = (int64_t)rpw * U;
  for (int64_t r00 = wave * step; r00 < (int64_t)rows; r00 += nwaves * step) {   // uniform per wavefront
    uint4 x[U], y[U];
    float fa[U], fb[U], ln[U];
    I li[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r00 + u * rpw + rl;     // row in [outer, L, H] order
      x[u] = y[u] = make_uint4(0, 0, 0, 0);
      fa[u] = fb[u] = ln[u] = 0.f;
      li[u] = 0;
      if (used && r < (int64_t)rows) {
        const int64_t off = ((r00 + u * rpw) * P + lane) * VW;
        x[u] = *reinterpret_cast<const uint4 *>(oa + off);
        y[u] = *reinterpret_cast<const uint4 *>(ob + off);
        const I ri = (I)r, h = ri % H, ql = ri / H;   // ql = outer * L + query
        li[u] = (ql / L * H + h) * L + ql % L;
        const float a = la[li[u]], b = lb[li[u]];
        const float m = fmaxf(a, b);
        const bool empty = m == -INFINITY;      // neither part has a valid key
        const float wa = empty ? 0.f : expf(a - m), wb = empty ? 0.f : expf(b - m);
        const float tot = wa + wb;
        fa[u] = empty ? 0.f : wa / tot;
        fb[u] = empty ? 0.f : wb / tot;
        ln[u] = empty ? -INFINITY : m + logf(tot);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r00 + u * rpw + rl;
      if (!used || r >= (int64_t)rows) continue;
      const T *xe = reinterpret_cast<const T *>(&x[u]), *ye = reinterpret_cast<const T *>(&y[u]);
      T z[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) z[e] = Elem<T>::store(fmaf(fa[u], Elem<T>::load(xe[e]), fb[u] * Elem<T>::load(ye[e])));
      *reinterpret_cast<uint4 *>(o + ((r00 + u * rpw) * P + lane) * VW) = *reinterpret_cast<const uint4 *>(z);
      if (j == 0) lse[li[u]] = ln[u];
    }
  }
}

// Blocks of 32 consecutive query rows (ql = outer * L + query) with all H
// heads: rows r = ql * H + h, contiguous in o.  The 32 * H merge weights are
// computed first, one thread per (h, query), so a block reads and writes each
// head's log-sum-exps as one run of 32 floats; then every thread streams
// 16-byte pieces of the block's rows, U pieces loaded before any is stored (a
// piece is read and written by the same thread, so this holds in place too).
template <typename T, int U>
__global__ void __launch_bounds__(256) attn_merge_blk_kernel(const T *oa, const float *la, const T *ob,
                                                             const float *lb, int64_t nql, int L, int H, int P, T *o,
                                                             float *lse) {
  constexpr int VW = 16 / sizeof(T);            // elements per 16-byte piece
  extern __shared__ float wgt[];                // [2][32 * H]: fa, fb per row of the block
  const int64_t ql0 = (int64_t)blockIdx.x * 32;
  const int nq = (int)min<int64_t>(32, nql - ql0);
  for (int t = threadIdx.x; t < 32 * H; t += blockDim.x) {
    const int h = t >> 5, qo = t & 31;
    if (qo >= nq) continue;
    const int64_t ql = ql0 + qo;
    const int64_t li = (ql / L * H + h) * L + ql % L;
    const float a = la[li], b = lb[li];
    const float m = fmaxf(a, b);
    const bool empty = m == -INFINITY;          // neither part has a valid key
    const float wa = empty ? 0.f : expf(a - m), wb = empty ? 0.f : expf(b - m);
    const float tot = wa + wb;
    wgt[qo * H + h] = empty ? 0.f : wa / tot;
    wgt[32 * H + qo * H + h] = empty ? 0.f : wb / tot;
    lse[li] = empty ? -INFINITY : m + logf(tot);
  }
  __syncthreads();
  const int nv = nq * H * P;                    // pieces of the block's rows
  const int64_t v0 = ql0 * H * P;
  const float invp = 1.0f / (float)P;
  for (int vb = 0; vb < nv; vb += U * (int)blockDim.x) {
    uint4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = vb + u * (int)blockDim.x + (int)threadIdx.x;
      if (v < nv) {
        x[u] = *reinterpret_cast<const uint4 *>(oa + (v0 + v) * VW);
        y[u] = *reinterpret_cast<const uint4 *>(ob + (v0 + v) * VW);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = vb + u * (int)blockDim.x + (int)threadIdx.x;
      if (v >= nv) continue;
      int rr = (int)(((float)v + 0.5f) * invp);   // row within the block (v < 2^22: exact)
      const float fa = wgt[rr], fb = wgt[32 * H + rr];
      const T *xe = reinterpret_cast<const T *>(&x[u]), *ye = reinterpret_cast<const T *>(&y[u]);
      T z[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) z[e] = Elem<T>::store(fmaf(fa, Elem<T>::load(xe[e]), fb * Elem<T>::load(ye[e])));
      *reinterpret_cast<uint4 *>(o + (v0 + v) * VW) = *reinterpret_cast<const uint4 *>(z);
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) attn_empty_kernel(T *o, float *lse, int64_t n_o, int64_t n_lse) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_o) o[i] = Elem<T>::store(0.f);
  if (i < n_lse) lse[i] = -INFINITY;
}

}  // namespace

template <typename T, int LPR>
void merge_launch(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t rows, int L, int H,
                  int d, void *o, float *lse, hipStream_t s) {
  const int64_t waves = (rows + 64 / LPR - 1) / (64 / LPR);
  const uint32_t blocks = (uint32_t)std::min<int64_t>((waves + 3) / 4, 256 * 128);
  hipLaunchKernelGGL((attn_merge_kernel<T, LPR>), dim3(blocks), dim3(256), 0, s, static_cast<const T *>(o_a), lse_a,
                     static_cast<const T *>(o_b), lse_b, rows, L, H, d, static_cast<T *>(o), lse);
}

template <typename T>
void merge_flat_launch(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t rows, int L,
                       int H, int P, void *o, float *lse, hipStream_t s) {
  constexpr int U = 4;                                  // passes whose loads are issued together
  const int64_t step = (int64_t)(64 / P) * U;           // rows per wavefront iteration
  const int64_t waves = (rows + step - 1) / step;
  const uint32_t blocks = (uint32_t)std::min<int64_t>((waves + 3) / 4, 256 * 64);
  const T *a = static_cast<const T *>(o_a), *b = static_cast<const T *>(o_b);
  if (rows < (1ll << 31))
    hipLaunchKernelGGL((attn_merge_flat_kernel<T, int32_t, U>), dim3(blocks), dim3(256), 0, s, a, lse_a, b, lse_b,
                       (int32_t)rows, (int32_t)L, (int32_t)H, P, static_cast<T *>(o), lse);
  else
    hipLaunchKernelGGL((attn_merge_flat_kernel<T, int64_t, U>), dim3(blocks), dim3(256), 0, s, a, lse_a, b, lse_b,
                       rows, (int64_t)L, (int64_t)H, P, static_cast<T *>(o), lse);
}

st_status launch_attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t outer,
                            int L, int H, int d, int elem_bytes, void *o, float *lse, hipStream_t s) {
  const int64_t rows = outer * L * H;
  if (rows == 0) return ST_OK;
  const int pieces = d * elem_bytes / 16;
  if ((d * elem_bytes) % 16 == 0 && H <= 256) {   // blocks of 32 queries x H heads
    const int64_t nql = outer * L;
    const int64_t blocks = (nql + 31) / 32;
    const size_t shm = (size_t)2 * 32 * H * sizeof(float);
    if (blocks < (1ll << 31)) {
      if (elem_bytes == 2)
        hipLaunchKernelGGL((attn_merge_blk_kernel<u16, 4>), dim3((uint32_t)blocks), dim3(256), shm, s,
                           static_cast<const u16 *>(o_a), lse_a, static_cast<const u16 *>(o_b), lse_b, nql, L, H,
                           pieces, static_cast<u16 *>(o), lse);
      else
        hipLaunchKernelGGL((attn_merge_blk_kernel<float, 4>), dim3((uint32_t)blocks), dim3(256), shm, s,
                           static_cast<const float *>(o_a), lse_a, static_cast<const float *>(o_b), lse_b, nql, L, H,
                           pieces, static_cast<float *>(o), lse);
      return launch_status();
    }
  }
  if ((d * elem_bytes) % 16 == 0 && pieces <= 64) {
    if (elem_bytes == 2) merge_flat_launch<u16>(o_a, lse_a, o_b, lse_b, rows, L, H, pieces, o, lse, s);
    else merge_flat_launch<float>(o_a, lse_a, o_b, lse_b, rows, L, H, pieces, o, lse, s);
    return launch_status();
  }
  // lanes per row: enough for the row's 16-byte vectors (or elements), a power of two
  const int units = (d * elem_bytes) % 16 == 0 ? d * elem_bytes / 16 : d;
  const int lpr = units <= 8 ? 8 : units <= 16 ? 16 : units <= 32 ? 32 : 64;
  if (elem_bytes == 2) {
    if (lpr == 8) merge_launch<u16, 8>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else if (lpr == 16) merge_launch<u16, 16>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else if (lpr == 32) merge_launch<u16, 32>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else merge_launch<u16, 64>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
  } else {
    if (lpr == 8) merge_launch<float, 8>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else if (lpr == 16) merge_launch<float, 16>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else if (lpr == 32) merge_launch<float, 32>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
    else merge_launch<float, 64>(o_a, lse_a, o_b, lse_b, rows, L, H, d, o, lse, s);
  }
  return launch_status();
}

st_status launch_attn_empty(void *o, float *lse, int64_t outer, int L, int H, int d, int elem_bytes, hipStream_t s) {
  const int64_t n_o = outer * L * H * d, n_lse = outer * H * L;
  if (n_o == 0) return ST_OK;
  const int64_t blocks = (n_o + 255) / 256;
  if (blocks >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(attn_empty_kernel<u16>, dim3((uint32_t)blocks), dim3(256), 0, s, static_cast<u16 *>(o), lse,
                       n_o, n_lse);
  else
    hipLaunchKernelGGL(attn_empty_kernel<float>, dim3((uint32_t)blocks), dim3(256), 0, s, static_cast<float *>(o),
                       lse, n_o, n_lse);
  return launch_status();
}

}  // namespace st
