// V-Major change detection (CoCoDiff page, "V-Major selective communication"):
// in each denoising step a V vector is compared with the cached one from the
// previous step by L1 distance, and only vectors that changed by more than a
// threshold are active -- their Q, K, V are the ones sent; the others are read
// from the cache.  A vector is one (token, head) row of V.
//
// Rows are contiguous, so a wavefront pass takes floor(64 / P) consecutive
// rows of P 16-byte pieces as one contiguous run (lane l holds piece l): each
// lane sums |v_new - v_cache| over its piece in fp32, the P lanes of a row
// reduce with shuffles, and the row's first lane writes the mask byte.  A
// second kernel compacts the mask into the index list, 1024 vectors per
// wavefront with one atomic add each, so the list is in increasing order
// within each 1024-vector chunk and in unspecified order across chunks; the
// count is exact.  Optionally the active rows' new V is written into the cache.
// HBM-bound: two reads of V per row, plus the outputs.
#include <algorithm>

#include "st_internal.h"

namespace st {
namespace {

template <typename T> __device__ __forceinline__ float widen(T x);
template <> __device__ __forceinline__ float widen<u16>(u16 x) { return __uint_as_float((uint32_t)x << 16); }
template <> __device__ __forceinline__ float widen<float>(float x) { return x; }

template <typename T, int U>
__global__ void __launch_bounds__(256) v_change_kernel(const T *vn, T *vc, int64_t nvec, int P, float thr,
                                                       uint8_t *mask, int update) {
  constexpr int VW = 16 / sizeof(T);          // elements per 16-byte piece
  const int lane = threadIdx.x & 63;
  const int vpw = 64 / P;                     // vectors per wavefront pass
  const int vl = lane / P, j = lane - vl * P; // vector within the pass, piece within the vector
  const bool used = vl < vpw;
  const int lead = vl * P;                    // first lane of this lane's vector
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t step = (int64_t)vpw * U;      // vectors per wavefront iteration
  for (int64_t v00 = wave * step; v00 < nvec; v00 += nwaves * step) {   // uniform per wavefront
    // Pass u covers vectors v00 + u*vpw ...: its pieces are one contiguous run
    // of vpw*P*16 bytes in each array.
    uint4 xn[U], xc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v00 + u * vpw + vl;
      xn[u] = xc[u] = make_uint4(0, 0, 0, 0);
      if (used && v < nvec) {
        const int64_t off = ((v00 + u * vpw) * P + lane) * VW;
        xn[u] = *reinterpret_cast<const uint4 *>(vn + off);
        xc[u] = *reinterpret_cast<const uint4 *>(vc + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v00 + u * vpw + vl;
      const bool valid = used && v < nvec;
      float part = 0.f;
      const T *x = reinterpret_cast<const T *>(&xn[u]), *y = reinterpret_cast<const T *>(&xc[u]);
#pragma unroll
      for (int e = 0; e < VW; ++e) part += fabsf(widen<T>(x[e]) - widen<T>(y[e]));
      // Segmented sum over the P lanes of a vector: after the step with
      // offset o, lane j holds the sum of pieces j .. j+2o-1 of its vector,
      // so the vector's first lane ends with the whole distance.
      for (int o = 1; o < P; o <<= 1) {
        const float up = __shfl_down(part, o);
        if (j + o < P) part += up;
      }
      const bool act = __shfl(valid && part > thr ? 1 : 0, lead) != 0;
      if (update && act && valid) *reinterpret_cast<uint4 *>(vc + ((v00 + u * vpw) * P + lane) * VW) = xn[u];
      if (valid && j == 0) mask[v] = act ? 1 : 0;
    }
  }
}

// Compaction of the mask: each lane takes 16 mask bytes (a wavefront 1024
// vectors), a wavefront prefix sum orders its active vectors, and one atomic
// add per wavefront chunk reserves their place in the list.
__global__ void __launch_bounds__(256) v_compact_kernel(const uint8_t *mask, int64_t nvec, int32_t *idx,
                                                        unsigned long long *count) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t c0 = wave * 1024; c0 < nvec; c0 += nwaves * 1024) {   // uniform per wavefront
    const int64_t v0 = c0 + lane * 16;
    uint32_t bits = 0;                        // bit e: vector v0 + e is active
    if (v0 + 16 <= nvec) {
      const uint4 m = *reinterpret_cast<const uint4 *>(mask + v0);
      const uint32_t w[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) bits |= ((w[q] >> (8 * e)) & 1u) << (4 * q + e);
    } else {
      for (int e = 0; v0 + e < nvec; ++e) bits |= (uint32_t)(mask[v0 + e] & 1) << e;
    }
    const int n = __builtin_popcount(bits);
    int incl = n;                             // inclusive prefix sum over the wavefront
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (total == 0) continue;
    unsigned long long base = 0;
    if (lane == 0) base = atomicAdd(count, (unsigned long long)total);
    base = __shfl(base, 0);
    if (idx) {
      int64_t at = (int64_t)base + incl - n;
      for (uint32_t b = bits; b; b &= b - 1) idx[at++] = (int32_t)(v0 + __builtin_ctz(b));
    }
  }
}

__global__ void zero_count_kernel(unsigned long long *count) { *count = 0; }

template <typename T>
void v_launch(const void *vn, void *vc, int64_t nvec, int P, float thr, uint8_t *mask, int update, hipStream_t s) {
  constexpr int U = 4;                                  // passes whose loads are issued together
  const int64_t step = (int64_t)(64 / P) * U;           // vectors per wavefront iteration
  const int64_t waves = (nvec + step - 1) / step;
  const uint32_t blocks = (uint32_t)std::min<int64_t>((waves + 3) / 4, 256 * 64);
  hipLaunchKernelGGL((v_change_kernel<T, U>), dim3(blocks), dim3(256), 0, s, static_cast<const T *>(vn),
                     static_cast<T *>(vc), nvec, P, thr, mask, update);
}

}  // namespace

st_status launch_v_change(const void *v_new, void *v_cache, int64_t nvec, int d, int elem_bytes, float threshold,
                          uint8_t *mask, int32_t *idx, int64_t *n_active, int update, hipStream_t s) {
  unsigned long long *count = reinterpret_cast<unsigned long long *>(n_active);
  hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(1), 0, s, count);
  if (nvec == 0) return launch_status();
  const int pieces = d * elem_bytes / 16;   // 1..32 (checked by the caller)
  if (elem_bytes == 2) v_launch<u16>(v_new, v_cache, nvec, pieces, threshold, mask, update, s);
  else v_launch<float>(v_new, v_cache, nvec, pieces, threshold, mask, update, s);
  const int64_t waves = (nvec + 1023) / 1024;
  const uint32_t blocks = (uint32_t)std::min<int64_t>((waves + 3) / 4, 256 * 64);
  hipLaunchKernelGGL(v_compact_kernel, dim3(blocks), dim3(256), 0, s, mask, nvec, idx, count);
  return launch_status();
}

}  // namespace st
