// Merge of attention results computed over disjoint key chunks: the step that
// Ring attention (PipeFusion summary, sequence parallelism; SwiftFusion,
// "Topology-Aware Communication Scheduling") and Torus attention (SwiftFusion,
// "Torus Attention") repeat as key/value chunks arrive.  A chunk result is the
// output normalised over the chunk's keys plus the natural log-sum-exp of its
// scaled scores; the union's output weights each part by exp(lse_part -
// lse_union).
//
// One thread per (sequence, query, head) row: it reads both parts' log-sum-exps
// and rows, then writes its own row and log-sum-exp, so the merge may run in
// place on either input.  HBM-bound: 3 rows of d elements per row merged.
#include <math.h>

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

template <typename T>
__global__ void __launch_bounds__(256) attn_merge_kernel(const T *oa, const float *la, const T *ob, const float *lb,
                                                         int64_t rows, int L, int H, int d, T *o, float *lse) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // row in [outer, L, H] order
  if (r >= rows) return;
  const int h = (int)(r % H);
  const int64_t ql = r / H;                  // outer * L + query
  const int qi = (int)(ql % L);
  const int64_t seq = ql / L;
  const int64_t li = (seq * H + h) * (int64_t)L + qi;
  const float a = la[li], b = lb[li];
  const float m = fmaxf(a, b);
  const T *ra = oa + r * d, *rb = ob + r * d;
  T *ro = o + r * d;
  if (m == -INFINITY) {   // neither part has a valid key
    for (int c = 0; c < d; ++c) ro[c] = Elem<T>::store(0.f);
    lse[li] = -INFINITY;
    return;
  }
  const float wa = expf(a - m), wb = expf(b - m);
  const float tot = wa + wb;
  const float fa = wa / tot, fb = wb / tot;
  constexpr int VW = 16 / sizeof(T);   // elements per 16-byte vector
  if (d % VW == 0) {                   // rows start 16-byte aligned (d * sizeof(T) a multiple of 16)
    for (int c = 0; c < d; c += VW) {
      const uint4 x = *reinterpret_cast<const uint4 *>(ra + c), y = *reinterpret_cast<const uint4 *>(rb + c);
      const T *xe = reinterpret_cast<const T *>(&x), *ye = reinterpret_cast<const T *>(&y);
      T z[VW];
#pragma unroll
      for (int j = 0; j < VW; ++j) z[j] = Elem<T>::store(fmaf(fa, Elem<T>::load(xe[j]), fb * Elem<T>::load(ye[j])));
      *reinterpret_cast<uint4 *>(ro + c) = *reinterpret_cast<const uint4 *>(z);
    }
  } else {
    for (int c = 0; c < d; ++c) ro[c] = Elem<T>::store(fmaf(fa, Elem<T>::load(ra[c]), fb * Elem<T>::load(rb[c])));
  }
  lse[li] = m + logf(tot);
}

template <typename T>
__global__ void __launch_bounds__(256) attn_empty_kernel(T *o, float *lse, int64_t n_o, int64_t n_lse) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_o) o[i] = Elem<T>::store(0.f);
  if (i < n_lse) lse[i] = -INFINITY;
}

}  // namespace

st_status launch_attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t outer,
                            int L, int H, int d, int elem_bytes, void *o, float *lse, hipStream_t s) {
  const int64_t rows = outer * L * H;
  if (rows == 0) return ST_OK;
  const int64_t blocks = (rows + 255) / 256;
  if (blocks >= (1ll << 31)) return ST_EUNSUPPORTED;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(attn_merge_kernel<u16>, dim3((uint32_t)blocks), dim3(256), 0, s,
                       static_cast<const u16 *>(o_a), lse_a, static_cast<const u16 *>(o_b), lse_b, rows, L, H, d,
                       static_cast<u16 *>(o), lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<float>, dim3((uint32_t)blocks), dim3(256), 0, s,
                       static_cast<const float *>(o_a), lse_a, static_cast<const float *>(o_b), lse_b, rows, L, H,
                       d, static_cast<float *>(o), lse);
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
