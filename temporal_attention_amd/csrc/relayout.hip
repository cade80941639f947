// Strided N-D copy: the one-GPU form of the spatial <-> temporal redistribution
// and of the blocked rearranges / slice gathers of the slicing schedule
// (ScaleFusion review, "Technical architecture" execution flow; "Core
// innovations" algorithm pseudocode).  Pure data movement, bit-exact.
//
// Design: the host merges dimensions that are contiguous in both source and
// destination and drops size-1 dimensions.  When the innermost dimension is
// contiguous on both sides the copy moves whole rows (for the [B,T,S,C] <->
// [B,S,T,C] permutation a row is one C-vector, 2304 bytes in bf16) with the
// widest vector width that every row start allows, one wavefront per pair of
// rows so the rows' offsets are computed once and the lanes stream the rows.  Short
// rows use a lane-per-vector kernel; a non-contiguous innermost dimension
// falls back to a lane-per-element kernel.  Divisions by the dimension sizes
// use precomputed multiply-shift constants (division by invariant integers).
#include <algorithm>
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
  int nd;                      // number of (outer, or all) dims described below
  FastDiv dim[kMaxDims];
  int64_t ss[kMaxDims];        // source strides in bytes
  int64_t ds[kMaxDims];        // destination strides in bytes
  uint32_t nrows;              // product of dim[0..nd)
  uint32_t row_vecs;           // vectors per row (row kernels)
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

// One wavefront per kRows rows; lanes stride each row in VB-byte vectors.  A
// wave loads all its rows' vectors before storing any, so each wave keeps
// kRows * 3 KB in flight, and both directions bypass the caches
// (nontemporal): every byte is touched exactly once.
constexpr int kRows = 2;
template <int VB>
__global__ void __launch_bounds__(256) relayout_rows_kernel(Params p) {
  typedef typename Vec<VB>::T V;
  constexpr int kU = 3;   // vectors per lane per row pass
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  const uint32_t nwaves = gridDim.x * (blockDim.x >> 6);
  for (uint32_t row0 = wave * kRows; row0 < p.nrows; row0 += nwaves * kRows) {
    for (uint32_t c0 = 0; c0 < p.row_vecs; c0 += 64 * kU) {
      V buf[kRows][kU];
      int64_t dso[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        int64_t so;
        row_offsets(p, row0 + r, so, dso[r]);
        const V *s = reinterpret_cast<const V *>(p.src + so);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t c = c0 + u * 64 + lane;
          if (row0 + r < p.nrows && c < p.row_vecs) buf[r][u] = __builtin_nontemporal_load(s + c);
        }
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        V *d = reinterpret_cast<V *>(p.dst + dso[r]);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t c = c0 + u * 64 + lane;
          if (row0 + r < p.nrows && c < p.row_vecs) __builtin_nontemporal_store(buf[r][u], d + c);
        }
      }
    }
  }
}

// One lane per vector; for rows shorter than a wavefront.
template <int VB>
__global__ void __launch_bounds__(256) relayout_items_kernel(Params p, uint32_t nitems) {
  typedef typename Vec<VB>::T V;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < nitems; i += stride) {
    const uint32_t row = fdiv(i, p.rv);
    const uint32_t c = i - row * p.row_vecs;
    int64_t so, dso;
    row_offsets(p, row, so, dso);
    const V *s = reinterpret_cast<const V *>(p.src + so);
    V *d = reinterpret_cast<V *>(p.dst + dso);
    d[c] = s[c];
  }
}

template <int VB>
st_status launch_rows(const Params &p, hipStream_t s) {
  if (p.row_vecs >= 32) {
    const uint32_t waves = (p.nrows + kRows - 1) / kRows;
    uint32_t blocks = (waves + 3) / 4;
    blocks = std::min<uint32_t>(blocks, 256u * 64u);
    hipLaunchKernelGGL(relayout_rows_kernel<VB>, dim3(blocks), dim3(256), 0, s, p);
  } else {
    const uint64_t nitems = (uint64_t)p.nrows * p.row_vecs;
    uint32_t blocks = (uint32_t)std::min<uint64_t>((nitems + 255) / 256, 256u * 256u);
    hipLaunchKernelGGL(relayout_items_kernel<VB>, dim3(blocks), dim3(256), 0, s, p, (uint32_t)nitems);
  }
  return launch_status();
}

}  // namespace

st_status launch_relayout(const void *src, const int64_t *src_str, void *dst, const int64_t *dst_str,
                          const int64_t *dims, int ndim, int elem_bytes, hipStream_t s) {
  // Drop size-1 dims, then merge dim k into dim k+1 when k+1 is contiguous
  // inside k on both sides.
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
  for (int k = (int)D.size() - 2; k >= 0; --k) {
    if (SS[k] == SS[k + 1] * D[k + 1] && DS[k] == DS[k + 1] * D[k + 1]) {
      D[k + 1] *= D[k];
      D.erase(D.begin() + k);
      SS.erase(SS.begin() + k);
      DS.erase(DS.begin() + k);
    }
  }
  const int64_t eb = elem_bytes;
  const bool inner_contig = SS.back() == 1 && DS.back() == 1;
  if (inner_contig && (int)D.size() < kMaxDims) {
    // Few long rows (e.g. one contiguous block): cut every row into equal
    // pieces of 2-8 KB so that enough wavefronts share the copy.  A piece is a
    // whole number of 16-byte units when the row is, so cutting never narrows
    // the vector width; failing an exact 2-8 KB divisor, rows are halved while
    // the halves stay whole units of at least 2 KB.
    int64_t outer = 1;
    for (size_t k = 0; k + 1 < D.size(); ++k) outer *= D[k];
    const int64_t inner = D.back(), row_bytes = inner * eb;
    const int64_t grain = row_bytes % 16 == 0 ? 16 : eb;   // bytes; a multiple of eb
    const int64_t units = row_bytes / grain;
    int64_t f = 1;
    if (outer < 65536 && row_bytes > 8192) {
      for (int64_t pu = (2048 + grain - 1) / grain; pu * grain <= 8192; ++pu)
        if (units % pu == 0) {
          f = units / pu;
          break;
        }
      if (f == 1)
        while (outer * f < 65536 && (units / f) % 2 == 0 && (units / f / 2) * grain >= 2048) f *= 2;
    }
    if (f > 1) {  // [..., inner] -> [..., f (stride inner/f), inner/f (stride 1)]
      const int64_t part = inner / f;
      D.back() = part;
      D.insert(D.end() - 1, f);
      SS.insert(SS.end() - 1, part);
      DS.insert(DS.end() - 1, part);
    }
  }
  const int nd = (int)D.size();
  Params p{};
  p.src = static_cast<const char *>(src);
  p.dst = static_cast<char *>(dst);

  if (inner_contig) {
    const int64_t row_bytes = D[nd - 1] * eb;
    int64_t g = row_bytes | (int64_t)(uintptr_t)src | (int64_t)(uintptr_t)dst;
    for (int k = 0; k < nd - 1; ++k) g |= SS[k] * eb | DS[k] * eb;
    int vb = 16;
    while (vb > 1 && (g % vb) != 0) vb >>= 1;
    int64_t nrows = 1;
    for (int k = 0; k < nd - 1; ++k) nrows *= D[k];
    const int64_t row_vecs = row_bytes / vb;
    if (nrows >= (1ll << 32) || row_vecs >= (1ll << 32) || nrows * row_vecs >= (1ll << 32))
      return ST_EUNSUPPORTED;
    p.nd = nd - 1;
    for (int k = 0; k < nd - 1; ++k) {
      p.dim[k] = make_fastdiv((uint32_t)D[k]);
      p.ss[k] = SS[k] * eb;
      p.ds[k] = DS[k] * eb;
    }
    p.nrows = (uint32_t)nrows;
    p.row_vecs = (uint32_t)row_vecs;
    p.rv = make_fastdiv((uint32_t)row_vecs);
    switch (vb) {
      case 16: return launch_rows<16>(p, s);
      case 8: return launch_rows<8>(p, s);
      case 4: return launch_rows<4>(p, s);
      case 2: return launch_rows<2>(p, s);
      default: return launch_rows<1>(p, s);
    }
  }
  // Non-contiguous innermost dim: one element per lane (rows of one element).
  int64_t nitems = 1;
  for (int k = 0; k < nd; ++k) nitems *= D[k];
  if (nitems >= (1ll << 32)) return ST_EUNSUPPORTED;
  p.nd = nd;
  for (int k = 0; k < nd; ++k) {
    p.dim[k] = make_fastdiv((uint32_t)D[k]);
    p.ss[k] = SS[k] * eb;
    p.ds[k] = DS[k] * eb;
  }
  p.nrows = (uint32_t)nitems;
  p.row_vecs = 1;
  p.rv = make_fastdiv(1);
  switch (elem_bytes) {
    case 16: return launch_rows<16>(p, s);
    case 8: return launch_rows<8>(p, s);
    case 4: return launch_rows<4>(p, s);
    case 2: return launch_rows<2>(p, s);
    default: return launch_rows<1>(p, s);
  }
}

}  // namespace st
