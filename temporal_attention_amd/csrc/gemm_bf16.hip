// bf16 MFMA projections of the attention block.
//
//   QKV:  q|k|v = x . w_qkv^T, then per-head RMSNorm and RoPE on q and k,
//         v plain (CoCoDiff page, "V-First compute scheduling").
//   Wo:   y = o . w_o^T.
//
// Both are C^T = W . X^T computed with v_mfma_f32_16x16x32_bf16: the A operand
// is a 16-row block of W (output channels), the B operand a 16-row block of X
// (tokens).  Both operands are K-contiguous in memory, so global loads, LDS
// stores and LDS operand reads are all 16-byte vectors.  In the accumulator a
// lane holds 4 consecutive output channels of one token, which makes the
// normalisation epilogue lane-local: RoPE pairs (2i, 2i+1) sit in one lane,
// and the per-head sum of squares needs only a 4-lane reduction (the lanes
// l, l^16, l^32, l^48 that share a token).  A wave's channel range holds
// whole heads, so the epilogue runs on the fp32 accumulator and stores bf16
// once: the norm and RoPE cost no extra HBM traffic.
//
// Tiling: 4 waves as 2 (channels) x 2 (tokens); a wave owns 16*CT channels x
// 64 tokens (CT*4 accumulator tiles).  K advances 32 per step through a
// double-buffered LDS stage fed by register prefetch, one barrier per step.
// The grid is remapped so the channel tiles of one token block run on the same
// XCD and share its L2 copy of the activations.
#include "st_internal.h"

namespace st {
namespace {

constexpr int kBK = 32;          // K per pipeline step
constexpr int kLdsK = kBK + 8;   // padded LDS row (80 B): conflict-free 16 B reads
constexpr int kWM = 64;          // tokens per wave
constexpr int kBM = 2 * kWM;     // tokens per workgroup

struct GemmArgs {
  const u16 *x;      // [M, K]
  const u16 *w;      // [N, K]
  int64_t M;
  int K, N;
  // plain output
  u16 *y;            // [M, N]
  // qkv output
  u16 *q, *k, *v;    // [M, H, D]
  int H;
  const float *g_q, *g_k;
  float eps;
  RopeArgs rope;
};

template <int CT>
struct Tile {
  static constexpr int WN = 16 * CT;   // channels per wave
  static constexpr int BN = 2 * WN;    // channels per workgroup
  static constexpr int A_CHUNKS = BN * kBK / 8;
  static constexpr int B_CHUNKS = kBM * kBK / 8;
  static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
  static constexpr int B_PER_T = (B_CHUNKS + 255) / 256;
  static constexpr int LDS_A = BN * kLdsK;   // u16 elements per stage
  static constexpr int LDS_B = kBM * kLdsK;
};

template <int CT>
__device__ __forceinline__ void load_stage(const GemmArgs &a, int64_t m0, int n0, int k0, uint4 (&ra)[Tile<CT>::A_PER_T],
                                           uint4 (&rb)[Tile<CT>::B_PER_T]) {
  typedef Tile<CT> TL;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TL::A_PER_T; ++i) {
    const int c = t + 256 * i;
    const int row = c >> 2, kc = (c & 3) * 8;
    const int n = n0 + row, kk = k0 + kc;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (c < TL::A_CHUNKS && n < a.N && kk < a.K) val = *reinterpret_cast<const uint4 *>(a.w + (int64_t)n * a.K + kk);
    ra[i] = val;
  }
#pragma unroll
  for (int i = 0; i < TL::B_PER_T; ++i) {
    const int c = t + 256 * i;
    const int row = c >> 2, kc = (c & 3) * 8;
    const int64_t m = m0 + row;
    const int kk = k0 + kc;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (c < TL::B_CHUNKS && m < a.M && kk < a.K) val = *reinterpret_cast<const uint4 *>(a.x + m * a.K + kk);
    rb[i] = val;
  }
}

template <int CT>
__device__ __forceinline__ void store_stage(u16 *As, u16 *Bs, const uint4 (&ra)[Tile<CT>::A_PER_T],
                                            const uint4 (&rb)[Tile<CT>::B_PER_T]) {
  typedef Tile<CT> TL;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TL::A_PER_T; ++i) {
    const int c = t + 256 * i;
    if (c < TL::A_CHUNKS) *reinterpret_cast<uint4 *>(As + (c >> 2) * kLdsK + (c & 3) * 8) = ra[i];
  }
#pragma unroll
  for (int i = 0; i < TL::B_PER_T; ++i) {
    const int c = t + 256 * i;
    if (c < TL::B_CHUNKS) *reinterpret_cast<uint4 *>(Bs + (c >> 2) * kLdsK + (c & 3) * 8) = rb[i];
  }
}

template <int CT, int D>
__device__ __forceinline__ void epilogue_qkv(const GemmArgs &a, f32x4 (&acc)[CT][4], int64_t m0, int nw0, int wm,
                                             int l16, int g4);

// MODE 0: plain output y.  MODE 1: q/k/v with RMSNorm + RoPE on q, k (head dim D).
template <int CT, int MODE, int D>
__global__ void __launch_bounds__(256, 2) gemm_bf16_kernel(GemmArgs a, uint32_t n_tiles_n, uint32_t nblocks) {
  typedef Tile<CT> TL;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * (TL::LDS_A + TL::LDS_B)];

  const uint32_t tile = xcd_remap(blockIdx.x, nblocks);
  const int64_t m0 = (int64_t)(tile / n_tiles_n) * kBM;
  const int n0 = (int)(tile % n_tiles_n) * TL::BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;

  f32x4 acc[CT][4];
#pragma unroll
  for (int i = 0; i < CT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[TL::A_PER_T], rb[TL::B_PER_T];
  const int nk = (a.K + kBK - 1) / kBK;
  load_stage<CT>(a, m0, n0, 0, ra, rb);
  store_stage<CT>(lds, lds + TL::LDS_A, ra, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage<CT>(a, m0, n0, (kt + 1) * kBK, ra, rb);
    const u16 *As = lds + buf * (TL::LDS_A + TL::LDS_B);
    const u16 *Bs = As + TL::LDS_A;
    bf16x8 bf[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      bf[tt] = *reinterpret_cast<const bf16x8 *>(Bs + (wm * kWM + tt * 16 + l16) * kLdsK + g4 * 8);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const bf16x8 af = *reinterpret_cast<const bf16x8 *>(As + (wn * TL::WN + ct * 16 + l16) * kLdsK + g4 * 8);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[tt], acc[ct][tt], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      u16 *An = lds + (buf ^ 1) * (TL::LDS_A + TL::LDS_B);
      store_stage<CT>(An, An + TL::LDS_A, ra, rb);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  const int nw0 = n0 + wn * TL::WN;   // first channel of this wave
  if constexpr (MODE == 0) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int64_t r = m0 + wm * kWM + tt * 16 + l16;
      if (r >= a.M) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = nw0 + ct * 16 + g4 * 4;
        if (n >= a.N) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[ct][tt][0], acc[ct][tt][1]);
        o.y = pack_bf16x2(acc[ct][tt][2], acc[ct][tt][3]);
        *reinterpret_cast<uint2 *>(a.y + r * a.N + n) = o;
      }
    }
  } else {
    epilogue_qkv<CT, D>(a, acc, m0, nw0, wm, l16, g4);
  }
}

// MODE 1 epilogue: the wave's channels are HPW whole heads.
template <int CT, int D>
__device__ __forceinline__ void epilogue_qkv(const GemmArgs &a, f32x4 (&acc)[CT][4], int64_t m0, int nw0, int wm,
                                             int l16, int g4) {
  typedef Tile<CT> TL;
  constexpr int HPW = TL::WN / D;
  static_assert(TL::WN % D == 0, "wave channel range must hold whole heads");
  const int H = a.H;
  const int hd = H * D;
  const int gh0 = nw0 / D;   // global head index (over 3H) of the wave's first head
  const int npairs = a.rope.kind == ST_ROPE_2D ? D / 4 : D / 2;

#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int64_t r = m0 + wm * kWM + tt * 16 + l16;
    // per-head sum of squares over this lane's channels, then over the 4 lanes of the token
    float ss[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) ss[hh] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int cl = ct * 16 + g4 * 4;
      const int hh = cl / D;
      float s4 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) s4 += acc[ct][tt][j] * acc[ct][tt][j];
#pragma unroll
      for (int h2 = 0; h2 < HPW; ++h2) ss[h2] += (hh == h2) ? s4 : 0.f;
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      ss[hh] += __shfl_xor(ss[hh], 16);
      ss[hh] += __shfl_xor(ss[hh], 32);
    }
    if (r >= a.M) continue;
    // position of this token
    int p0 = 0, p1 = 0;
    if (a.rope.kind != ST_ROPE_NONE) {
      const int64_t i = r % a.rope.period + a.rope.offset;
      if (a.rope.kind == ST_ROPE_1D) {
        p0 = (int)i;
      } else {
        p0 = (int)(i / a.rope.grid_w);
        p1 = (int)(i % a.rope.grid_w);
      }
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int cl = ct * 16 + g4 * 4;
      const int hh = cl / D;
      const int gh = gh0 + hh;
      if (gh >= 3 * H) continue;
      const int which = gh / H;              // 0 q, 1 k, 2 v
      const int jd = cl - hh * D;            // dim within the head (multiple of 4)
      float o[4] = {acc[ct][tt][0], acc[ct][tt][1], acc[ct][tt][2], acc[ct][tt][3]};
      if (which < 2) {
        float sh = 0.f;
#pragma unroll
        for (int h2 = 0; h2 < HPW; ++h2) sh = (hh == h2) ? ss[h2] : sh;
        const float inv = rsqrtf(sh * (1.0f / D) + a.eps);
        const float4 g = *reinterpret_cast<const float4 *>((which == 0 ? a.g_q : a.g_k) + jd);
        o[0] *= inv * g.x;
        o[1] *= inv * g.y;
        o[2] *= inv * g.z;
        o[3] *= inv * g.w;
        if (a.rope.kind != ST_ROPE_NONE) {
          int pos, pair;
          if (a.rope.kind == ST_ROPE_1D) {
            pos = p0;
            pair = jd >> 1;
          } else {
            const bool second = jd >= D / 2;
            pos = second ? p1 : p0;
            pair = (jd - (second ? D / 2 : 0)) >> 1;
          }
          const float4 cs = *reinterpret_cast<const float4 *>(a.rope.table + ((int64_t)pos * npairs + pair) * 2);
          const float x0 = o[0], x1 = o[1], x2 = o[2], x3 = o[3];
          o[0] = x0 * cs.x - x1 * cs.y;
          o[1] = x0 * cs.y + x1 * cs.x;
          o[2] = x2 * cs.z - x3 * cs.w;
          o[3] = x2 * cs.w + x3 * cs.z;
        }
      }
      u16 *dst = which == 0 ? a.q : (which == 1 ? a.k : a.v);
      uint2 ov;
      ov.x = pack_bf16x2(o[0], o[1]);
      ov.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2 *>(dst + r * hd + (gh - which * H) * D + jd) = ov;
    }
  }
}

template <int CT, int MODE, int D>
st_status launch_gemm(const GemmArgs &a, hipStream_t s) {
  typedef Tile<CT> TL;
  if (a.M == 0) return ST_OK;
  const int64_t mt = (a.M + kBM - 1) / kBM;
  const uint32_t nt = (a.N + TL::BN - 1) / TL::BN;
  const int64_t nb = mt * nt;
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((gemm_bf16_kernel<CT, MODE, D>), dim3((uint32_t)nb), dim3(256), 0, s, a, nt, (uint32_t)nb);
  return launch_status();
}

}  // namespace

st_status launch_qkv_bf16(const void *x, int64_t rows, int c_in, const void *w, const float *g_q, const float *g_k,
                          float eps, const RopeArgs &rope, int H, int d, void *q, void *k, void *v, hipStream_t s) {
  GemmArgs a{};
  a.x = static_cast<const u16 *>(x);
  a.w = static_cast<const u16 *>(w);
  a.M = rows;
  a.K = c_in;
  a.N = 3 * H * d;
  a.q = static_cast<u16 *>(q);
  a.k = static_cast<u16 *>(k);
  a.v = static_cast<u16 *>(v);
  a.H = H;
  a.g_q = g_q;
  a.g_k = g_k;
  a.eps = eps;
  a.rope = rope;
  switch (d) {
    case 72: return launch_gemm<9, 1, 72>(a, s);    // wave = 2 heads x 72
    case 64: return launch_gemm<8, 1, 64>(a, s);    // wave = 2 heads x 64
    case 128: return launch_gemm<8, 1, 128>(a, s);  // wave = 1 head x 128
    default: return ST_EUNSUPPORTED;
  }
}

st_status launch_linear_bf16(const void *a_, int64_t rows, int k_in, const void *w, int n_out, void *y,
                             hipStream_t s) {
  GemmArgs a{};
  a.x = static_cast<const u16 *>(a_);
  a.w = static_cast<const u16 *>(w);
  a.M = rows;
  a.K = k_in;
  a.N = n_out;
  a.y = static_cast<u16 *>(y);
  if (n_out % 288 == 0) return launch_gemm<9, 0, 0>(a, s);
  return launch_gemm<8, 0, 0>(a, s);
}

}  // namespace st
