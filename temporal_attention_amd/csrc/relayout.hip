// Strided N-D copy: the one-GPU form of the spatial <-> temporal redistribution
// and of the blocked rearranges / slice gathers of the slicing schedule
// (ScaleFusion review, "Technical architecture" execution flow; "Core
// innovations" algorithm pseudocode).  Pure data movement, bit-exact.
//
// Design: the host drops size-1 dimensions, orders the others by destination
// stride (largest first) and merges dimensions that are contiguous inside
// their neighbour on both sides.  One lane moves one vector -- 16 bytes when
// every row start allows it -- and lanes are numbered in destination order, so
// the workgroups the dispatcher hands out at any moment write one contiguous
// stretch of the destination while their reads gather rows from wherever
// they lie.  The grid covers every vector once (no grid-stride loop) and both
// directions bypass the caches (nontemporal): every byte is touched once.
// Measured on a 0.96 GB [T,S,C] -> [S,T,C] permutation this moves 6.1 TB/s,
// against 6.5 TB/s for a plain copy of the same bytes by the same scheme and
// 5.1-5.2 TB/s for the earlier form (a wavefront per pair of source rows, a
// grid-stride loop in source order).  Divisions by the dimension sizes use
// precomputed multiply-shift constants (division by invariant integers).
#include <algorithm>
#include <numeric>
#include <vector>

#include "st_internal.h"

namespace st {
namespace {

constexpr int kMaxDims = 6;

// Unsigned 32-bit division by an invariant divisor: q = (t + ((n - t) >> s1)) >> s2,
// t = mulhi(m, n), with m, s1, s2 chosen on the host for the divisor.
struct FastDiv {
  uint32_t d, m, s1, s2;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  f.m = (uint32_t)((((unsigned __int128)1 << 32) * (((unsigned __int128)1 << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  uint32_t t = __umulhi(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

struct Params {
  const char *src;
  char *dst;
  int nd;                      // number of row dims described below
  FastDiv dim[kMaxDims];
  int64_t ss[kMaxDims];        // source strides in bytes
  int64_t ds[kMaxDims];        // destination strides in bytes
  uint32_t nvec;               // vectors in all
  uint32_t row_vecs;           // vectors per row
  FastDiv rv;                  // divider by row_vecs
};

__device__ __forceinline__ void row_offsets(const Params &p, uint32_t row, int64_t &so, int64_t &dso) {
  so = 0;
  dso = 0;
  for (int k = p.nd - 1; k >= 0; --k) {
    const uint32_t q = fdiv(row, p.dim[k]);
    const uint32_t i = row - q * p.dim[k].d;
    so += (int64_t)i * p.ss[k];
    dso += (int64_t)i * p.ds[k];
    row = q;
  }
}

template <int VB> struct Vec;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <> struct Vec<16> { typedef u32x4 T; };
template <> struct Vec<8> { typedef u32x2 T; };
template <> struct Vec<4> { typedef uint32_t T; };
template <> struct Vec<2> { typedef uint16_t T; };
template <> struct Vec<1> { typedef uint8_t T; };

// One lane per VB-byte vector; vector i is column i % row_vecs of row i / row_vecs.
template <int VB>
__global__ void __launch_bounds__(256) relayout_kernel(Params p) {
  typedef typename Vec<VB>::T V;
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.nvec) return;
  const uint32_t row = fdiv(i, p.rv);
  const uint32_t c = i - row * p.row_vecs;
  int64_t so, dso;
  row_offsets(p, row, so, dso);
  const V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(p.src + so) + c);
  __builtin_nontemporal_store(v, reinterpret_cast<V *>(p.dst + dso) + c);
}

template <int VB>
st_status launch_vb(const Params &p, hipStream_t s) {
  hipLaunchKernelGGL(relayout_kernel<VB>, dim3((p.nvec + 255) / 256), dim3(256), 0, s, p);
  return launch_status();
}

// Merge dim k into dim k+1 when k+1 is contiguous inside k on both sides.
void merge_dims(std::vector<int64_t> &D, std::vector<int64_t> &SS, std::vector<int64_t> &DS) {
  for (int k = (int)D.size() - 2; k >= 0; --k) {
    if (SS[k] == SS[k + 1] * D[k + 1] && DS[k] == DS[k + 1] * D[k + 1]) {
      D[k + 1] *= D[k];
      D.erase(D.begin() + k);
      SS.erase(SS.begin() + k);
      DS.erase(DS.begin() + k);
    }
  }
}

}  // namespace

st_status launch_relayout(const void *src, const int64_t *src_str, void *dst, const int64_t *dst_str,
                          const int64_t *dims, int ndim, int elem_bytes, hipStream_t s) {
  std::vector<int64_t> D, SS, DS;
  for (int k = 0; k < ndim; ++k) {
    if (dims[k] == 0) return ST_OK;
    if (dims[k] == 1) continue;
    D.push_back(dims[k]);
    SS.push_back(src_str[k]);
    DS.push_back(dst_str[k]);
  }
  if (D.empty()) {  // a single element
    D.push_back(1);
    SS.push_back(1);
    DS.push_back(1);
  }
  // Destination order: dimensions by |destination stride|, largest first (stable).
  std::vector<int> ord(D.size());
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return std::llabs(DS[a]) > std::llabs(DS[b]); });
  {
    std::vector<int64_t> D2, S2, T2;
    for (int k : ord) {
      D2.push_back(D[k]);
      S2.push_back(SS[k]);
      T2.push_back(DS[k]);
    }
    D.swap(D2);
    SS.swap(S2);
    DS.swap(T2);
  }
  merge_dims(D, SS, DS);
  const int64_t eb = elem_bytes;
  // Rows: the innermost dimension when it is contiguous on both sides, else single elements.
  const bool inner_contig = SS.back() == 1 && DS.back() == 1;
  if (!inner_contig) {
    D.push_back(1);
    SS.push_back(1);
    DS.push_back(1);
  }
  const int nd = (int)D.size();
  if (nd - 1 > kMaxDims) return ST_EUNSUPPORTED;
  const int64_t row_bytes = D[nd - 1] * eb;
  int64_t g = row_bytes | (int64_t)(uintptr_t)src | (int64_t)(uintptr_t)dst;
  for (int k = 0; k < nd - 1; ++k) g |= SS[k] * eb | DS[k] * eb;
  int vb = 16;
  while (vb > 1 && (g % vb) != 0) vb >>= 1;
  int64_t nrows = 1;
  for (int k = 0; k < nd - 1; ++k) nrows *= D[k];
  const int64_t row_vecs = row_bytes / vb;
  if (nrows * row_vecs >= (1ll << 32)) return ST_EUNSUPPORTED;
  Params p{};
  p.src = static_cast<const char *>(src);
  p.dst = static_cast<char *>(dst);
  p.nd = nd - 1;
  for (int k = 0; k < nd - 1; ++k) {
    p.dim[k] = make_fastdiv((uint32_t)D[k]);
    p.ss[k] = SS[k] * eb;
    p.ds[k] = DS[k] * eb;
  }
  p.nvec = (uint32_t)(nrows * row_vecs);
  p.row_vecs = (uint32_t)row_vecs;
  p.rv = make_fastdiv((uint32_t)row_vecs);
  switch (vb) {
    case 16: return launch_vb<16>(p, s);
    case 8: return launch_vb<8>(p, s);
    case 4: return launch_vb<4>(p, s);
    case 2: return launch_vb<2>(p, s);
    default: return launch_vb<1>(p, s);
  }
}

}  // namespace st
