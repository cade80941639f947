// bf16 attention over the middle axis L of [outer, L, H, d] tensors:
//   O = softmax(Q K^T * scale) V per (outer, head), keys j >= n_valid masked.
// Spatial attention is outer = B*T, L = S (ScaleFusion review, "Technical
// architecture": the spatial layer attends over the S patches of a frame);
// temporal attention is outer = B*S, L = T (the temporal layer attends over
// the T frames of a patch).
//
// Both kernels compute the transposed score tile S^T = K . Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K, B = 16 dims x 32
// queries of Q^T).  In the 32x32 accumulator a lane then holds 16 keys of ONE
// query, so the row max and the exponentials are lane-local apart from one
// exchange between the two half-waves, and the same registers, converted to
// bf16, are directly the B operand of O^T = V^T . P^T: the k-slot order of a
// 16-key MFMA step only has to match between A and B, so V^T is read from LDS
// in the key order the score accumulator already has.  The output
// accumulator O^T again holds one query per lane, so the softmax rescale is a
// per-lane multiply.
//
// d = 72 is padded to 80 for Q.K (five 16-wide steps) and to 96 for P.V
// (three 32-row tiles); the spare row 72 of V^T is filled with ones, so row
// 72 of O^T accumulates the softmax denominator in the same MFMAs.
//
// Long sequences (attn_long_kernel): a workgroup of 4 waves owns 32*NT
// queries per wave; K and V^T tiles of 64 keys are staged through a
// double-buffered LDS stage (V transposed on the way in), and the online
// softmax only rescales the accumulator when a query's running maximum grows
// by more than 8 (in log2 units), so exponentials stay <= 2^8 in between.
// Short sequences (attn_short_kernel, L <= 64): one wave per (outer, head)
// loads its whole Q and K straight into operand registers and V^T through a
// private LDS slice; a workgroup covers all heads of one outer index, which
// is one contiguous [L, H, d] block of each tensor.
#include <math.h>

#include "st_internal.h"

namespace st {
namespace {

struct AttnArgs {
  const u16 *q, *k, *v;
  u16 *o;
  int64_t outer;
  int L, n_valid, H;
  float c;   // scale * log2(e)
};

template <int D>
struct Dims {
  static constexpr int DQK = (D + 15) / 16 * 16;          // Q.K contraction, padded
  static constexpr bool ONES = (D % 32) != 0;              // spare V^T row carries ones
  static constexpr int DV = ONES ? (D / 32 + 1) * 32 : D;  // P.V output rows, padded
  static constexpr int KS = DQK / 16;
  static constexpr int DT = DV / 32;
  static constexpr int CH = D / 8;                         // 16-byte chunks per row
  // location of the ones row inside O^T: tile, register, lane half
  static constexpr int ONES_DT = D / 32;
  static constexpr int ONES_R = ((D % 32) / 8) * 4 + (D % 4);
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// Transpose 4 keys x 8 dims (4 x uint4) into 8 dims x 4 keys (8 x uint2).
__device__ __forceinline__ void transpose4x8(const uint4 (&kv)[4], uint2 (&out)[8]) {
  const uint32_t w[4][4] = {{kv[0].x, kv[0].y, kv[0].z, kv[0].w},
                            {kv[1].x, kv[1].y, kv[1].z, kv[1].w},
                            {kv[2].x, kv[2].y, kv[2].z, kv[2].w},
                            {kv[3].x, kv[3].y, kv[3].z, kv[3].w}};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = make_uint2(lo_pair(w[0][j], w[1][j]), lo_pair(w[2][j], w[3][j]));
    out[2 * j + 1] = make_uint2(hi_pair(w[0][j], w[1][j]), hi_pair(w[2][j], w[3][j]));
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint2 a, uint2 b) {
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 pack_p(const f32x16 &s, int base) {
  uint4 u;
  u.x = pack_bf16x2(s[base + 0], s[base + 1]);
  u.y = pack_bf16x2(s[base + 2], s[base + 3]);
  u.z = pack_bf16x2(s[base + 4], s[base + 5]);
  u.w = pack_bf16x2(s[base + 6], s[base + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float max16(const f32x16 &s) {
  float m0 = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  float m1 = fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]));
  float m2 = fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11]));
  float m3 = fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]));
  return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}

// Key index (within a 32-key tile) of accumulator register r in lane half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

constexpr float kRescale = 8.0f;   // log2 growth of the running max that forces a rescale

// ------------------------------------------------------------------------- //
// Long sequences                                                            //
// ------------------------------------------------------------------------- //
template <int D, int NT>
struct LongCfg {
  typedef Dims<D> DM;
  static constexpr int KB = 64;                  // keys per LDS tile
  static constexpr int QW = 32 * NT;             // queries per wave
  static constexpr int QB = 4 * QW;              // queries per workgroup
  static constexpr int K_LD = DM::DQK + 8;       // LDS row stride of K (u16)
  static constexpr int V_LD = KB + 4;            // LDS row stride of V^T (u16)
  static constexpr int K_TILE = KB * K_LD;
  static constexpr int V_TILE = DM::DV * V_LD;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int K_CHUNKS = KB * DM::CH;
  static constexpr int K_PER_T = (K_CHUNKS + 255) / 256;
  static constexpr int V_TASKS = (KB / 4) * DM::CH;   // (4 keys x 8 dims) per task
  static constexpr int V_PER_T = (V_TASKS + 255) / 256;
};

template <int D, int NT>
__global__ void __launch_bounds__(256, 2) attn_long_kernel(AttnArgs a, uint32_t nqb, uint32_t nblocks) {
  typedef LongCfg<D, NT> C;
  typedef Dims<D> DM;
  __shared__ __attribute__((aligned(16))) u16 lds[2 * C::STAGE];

  const uint32_t tile = xcd_remap(blockIdx.x, nblocks);
  const uint32_t qb = tile % nqb;
  const uint32_t seq = tile / nqb;
  const int h = (int)(seq % (uint32_t)a.H);
  const int64_t outer = seq / (uint32_t)a.H;
  const int64_t rs = (int64_t)a.H * D;                  // row stride (elements)
  const int64_t base = outer * a.L * rs + (int64_t)h * D;
  const u16 *qp = a.q + base, *kp = a.k + base, *vp = a.v + base;
  u16 *op = a.o + base;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int L = a.L, nv = a.n_valid;

  // Constant parts of both stages: K pad columns [D, DQK) = 0; V^T rows [D, DV) = 0,
  // except the ones row.
  for (int i = t; i < 2 * C::KB; i += 256) {
    u16 *row = lds + (i / C::KB) * C::STAGE + (i % C::KB) * C::K_LD;
    for (int dd = D; dd < DM::DQK; ++dd) row[dd] = 0;
  }
  for (int i = t; i < 2 * (DM::DV - D) * C::V_LD; i += 256) {
    const int st = i / ((DM::DV - D) * C::V_LD);
    const int rem = i % ((DM::DV - D) * C::V_LD);
    const int dd = D + rem / C::V_LD;
    lds[st * C::STAGE + C::K_TILE + dd * C::V_LD + rem % C::V_LD] = (DM::ONES && dd == D) ? (u16)0x3F80 : (u16)0;
  }

  // Q operand fragments (B of S^T = K Q^T), held for the whole key loop.
  const int q0 = qb * C::QB + wave * C::QW;
  bf16x8 qf[NT][DM::KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int qi = q0 + nt * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < DM::KS; ++ks) {
      const int dd = ks * 16 + g * 8;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qi < L && dd < D) u = *reinterpret_cast<const uint4 *>(qp + (int64_t)qi * rs + dd);
      qf[nt][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 oacc[DM::DT][NT];
#pragma unroll
  for (int i = 0; i < DM::DT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][j][r] = 0.f;
  float mref[NT], lsum[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    mref[j] = -INFINITY;
    lsum[j] = 0.f;
  }

  const int nkt = (min(L, nv) + C::KB - 1) / C::KB;   // tiles past n_valid carry no weight
  uint4 rk[C::K_PER_T], rv[C::V_PER_T][4];

  auto gload = [&](int kt) {
    const int kb = kt * C::KB;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = t + 256 * i;
      const int key = c / DM::CH, ch = c % DM::CH;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (c < C::K_CHUNKS && kb + key < L) u = *reinterpret_cast<const uint4 *>(kp + (int64_t)(kb + key) * rs + ch * 8);
      rk[i] = u;
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int task = t + 256 * i;
      const int key4 = task % (C::KB / 4), ch = task / (C::KB / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kb + key4 * 4 + j;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (task < C::V_TASKS && key < L) u = *reinterpret_cast<const uint4 *>(vp + (int64_t)key * rs + ch * 8);
        rv[i][j] = u;
      }
    }
  };
  auto sstore = [&](int stage) {
    u16 *Ks = lds + stage * C::STAGE;
    u16 *Vs = Ks + C::K_TILE;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int c = t + 256 * i;
      if (c < C::K_CHUNKS) *reinterpret_cast<uint4 *>(Ks + (c / DM::CH) * C::K_LD + (c % DM::CH) * 8) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int task = t + 256 * i;
      if (task < C::V_TASKS) {
        const int key4 = task % (C::KB / 4), ch = task / (C::KB / 4);
        uint2 tr[8];
        transpose4x8(rv[i], tr);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint2 *>(Vs + (ch * 8 + j) * C::V_LD + key4 * 4) = tr[j];
      }
    }
  };

  if (nkt > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const u16 *Ks = lds + stage * C::STAGE;
    const u16 *Vs = Ks + C::K_TILE;
    const int kb = kt * C::KB;
    const bool masked = kb + C::KB > nv;

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 s[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DM::KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (sub * 32 + l32) * C::K_LD + ks * 16 + g * 8);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nt][ks], s[nt], 0, 0, 0);
      }
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool off = kb + sub * 32 + acc_row(r, g) >= nv;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) s[nt][r] = off ? -INFINITY : s[nt][r];
        }
      }
      float mx[NT];
      bool grow = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        mx[nt] = max16(s[nt]);
        mx[nt] = fmaxf(mx[nt], __shfl_xor(mx[nt], 32));
        grow |= (mx[nt] - mref[nt]) * a.c > kRescale;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float mnew = fmaxf(mref[nt], mx[nt]);
          const float alpha = __builtin_amdgcn_exp2f((mref[nt] - mnew) * a.c);
          mref[nt] = mnew;
          lsum[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][nt][r] *= alpha;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float mc = mref[nt] * a.c;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nt][r] = __builtin_amdgcn_exp2f(fmaf(s[nt][r], a.c, -mc));
        if constexpr (!DM::ONES) {
          float acc = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += s[nt][r];
          lsum[nt] += acc;
        }
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pf[nt] = pack_p(s[nt], ks2 * 8);
        const int kk = sub * 32 + ks2 * 16 + g * 4;
#pragma unroll
        for (int dt = 0; dt < DM::DT; ++dt) {
          const u16 *vrow = Vs + (dt * 32 + l32) * C::V_LD + kk;
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint2 *>(vrow), *reinterpret_cast<const uint2 *>(vrow + 8));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nt], oacc[dt][nt], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nkt) sstore(stage ^ 1);
    __syncthreads();
  }

  // normalise and store
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l;
    if constexpr (DM::ONES) {
      l = __shfl(oacc[DM::ONES_DT][nt][DM::ONES_R], l32);   // held by lane half 0
    } else {
      l = lsum[nt] + __shfl_xor(lsum[nt], 32);
    }
    const float inv = 1.0f / l;
    const int qi = q0 + nt * 32 + l32;
    if (qi >= L) continue;
    u16 *orow = op + (int64_t)qi * rs;
#pragma unroll
    for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int dd = dt * 32 + rb * 8 + g * 4;
        if (dd + 4 <= D) {
          uint2 w;
          w.x = pack_bf16x2(oacc[dt][nt][rb * 4 + 0] * inv, oacc[dt][nt][rb * 4 + 1] * inv);
          w.y = pack_bf16x2(oacc[dt][nt][rb * 4 + 2] * inv, oacc[dt][nt][rb * 4 + 3] * inv);
          *reinterpret_cast<uint2 *>(orow + dd) = w;
        }
      }
  }
}

// ------------------------------------------------------------------------- //
// Short sequences (L <= 32 * NT)                                             //
// ------------------------------------------------------------------------- //
template <int D, int NT>
struct ShortCfg {
  typedef Dims<D> DM;
  static constexpr int KL = 32 * NT;             // padded keys = queries
  static constexpr int V_LD = KL + 4;
  static constexpr int V_WAVE = DM::DV * V_LD;   // u16 per wave
  static constexpr int V_TASKS = (KL / 4) * DM::CH;
  static constexpr int V_PER_L = (V_TASKS + 63) / 64;
};

template <int D, int NT>
__global__ void __launch_bounds__(256, 2) attn_short_kernel(AttnArgs a, uint32_t nblocks) {
  typedef ShortCfg<D, NT> C;
  typedef Dims<D> DM;
  __shared__ __attribute__((aligned(16))) u16 lds[4 * C::V_WAVE];

  const int64_t outer = xcd_remap(blockIdx.x, nblocks);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int L = a.L, nv = min(a.n_valid, a.L);
  const int64_t rs = (int64_t)a.H * D;
  u16 *Vs = lds + wave * C::V_WAVE;

  // constant V^T rows [D, DV)
  for (int i = lane; i < (DM::DV - D) * C::V_LD; i += 64) {
    const int dd = D + i / C::V_LD;
    Vs[dd * C::V_LD + i % C::V_LD] = (DM::ONES && dd == D) ? (u16)0x3F80 : (u16)0;
  }

  for (int h = wave; h < a.H; h += 4) {
    const int64_t base = outer * L * rs + (int64_t)h * D;
    const u16 *qp = a.q + base, *kp = a.k + base, *vp = a.v + base;
    u16 *op = a.o + base;

    // V^T of this head into the wave's LDS slice
#pragma unroll
    for (int i = 0; i < C::V_PER_L; ++i) {
      const int task = lane + 64 * i;
      if (task < C::V_TASKS) {
        const int key4 = task % (C::KL / 4), ch = task / (C::KL / 4);
        uint4 kv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key4 * 4 + j;
          kv[j] = key < L ? *reinterpret_cast<const uint4 *>(vp + (int64_t)key * rs + ch * 8) : make_uint4(0, 0, 0, 0);
        }
        uint2 tr[8];
        transpose4x8(kv, tr);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint2 *>(Vs + (ch * 8 + j) * C::V_LD + key4 * 4) = tr[j];
      }
    }
    bf16x8 qf[NT][DM::KS], kf[NT][DM::KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = nt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < DM::KS; ++ks) {
        const int dd = ks * 16 + g * 8;
        uint4 uq = make_uint4(0, 0, 0, 0), uk = make_uint4(0, 0, 0, 0);
        if (row < L && dd < D) {
          uq = *reinterpret_cast<const uint4 *>(qp + (int64_t)row * rs + dd);
          uk = *reinterpret_cast<const uint4 *>(kp + (int64_t)row * rs + dd);
        }
        qf[nt][ks] = __builtin_bit_cast(bf16x8, uq);
        kf[nt][ks] = __builtin_bit_cast(bf16x8, uk);
      }
    }
    // S^T[mt][nt]: keys of tile mt x queries of tile nt
    f32x16 s[NT][NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][nt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DM::KS; ++ks)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][ks], qf[nt][ks], s[mt][nt], 0, 0, 0);
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (mt * 32 + acc_row(r, g) < nv) ? s[mt][nt][r] : -INFINITY;
          s[mt][nt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mc = mx * a.c;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][nt][r] = __builtin_amdgcn_exp2f(fmaf(s[mt][nt][r], a.c, -mc));
    }
    // V^T is complete in LDS once every lane's stores have issued (one wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x16 oacc[DM::DT][NT];
#pragma unroll
    for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][nt][r] = 0.f;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pf[nt] = pack_p(s[mt][nt], ks2 * 8);
        const int kk = mt * 32 + ks2 * 16 + g * 4;
#pragma unroll
        for (int dt = 0; dt < DM::DT; ++dt) {
          const u16 *vrow = Vs + (dt * 32 + l32) * C::V_LD + kk;
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint2 *>(vrow), *reinterpret_cast<const uint2 *>(vrow + 8));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nt], oacc[dt][nt], 0, 0, 0);
        }
      }
    float lsum[NT];
    if constexpr (!DM::ONES) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float acc = 0.f;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += s[mt][nt][r];
        lsum[nt] = acc + __shfl_xor(acc, 32);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float l;
      if constexpr (DM::ONES) {
        l = __shfl(oacc[DM::ONES_DT][nt][DM::ONES_R], l32);
      } else {
        l = lsum[nt];
      }
      const float inv = 1.0f / l;
      const int qi = nt * 32 + l32;
      if (qi >= L) continue;
      u16 *orow = op + (int64_t)qi * rs;
#pragma unroll
      for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int dd = dt * 32 + rb * 8 + g * 4;
          if (dd + 4 <= D) {
            uint2 w;
            w.x = pack_bf16x2(oacc[dt][nt][rb * 4 + 0] * inv, oacc[dt][nt][rb * 4 + 1] * inv);
            w.y = pack_bf16x2(oacc[dt][nt][rb * 4 + 2] * inv, oacc[dt][nt][rb * 4 + 3] * inv);
            *reinterpret_cast<uint2 *>(orow + dd) = w;
          }
        }
    }
    // the next head overwrites V^T: all lanes' reads of this head are done
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int D, int NT>
st_status launch_long(const AttnArgs &a, hipStream_t s) {
  typedef LongCfg<D, NT> C;
  const int64_t nqb = (a.L + C::QB - 1) / C::QB;
  const int64_t nb = nqb * a.outer * a.H;
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_long_kernel<D, NT>), dim3((uint32_t)nb), dim3(256), 0, s, a, (uint32_t)nqb,
                     (uint32_t)nb);
  return launch_status();
}

template <int D, int NT>
st_status launch_short(const AttnArgs &a, hipStream_t s) {
  if (a.outer >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_short_kernel<D, NT>), dim3((uint32_t)a.outer), dim3(256), 0, s, a, (uint32_t)a.outer);
  return launch_status();
}

AttnArgs make_args(const void *q, const void *k, const void *v, int64_t outer, int L, int n_valid, int H,
                   float scale, void *out) {
  AttnArgs a;
  a.q = static_cast<const u16 *>(q);
  a.k = static_cast<const u16 *>(k);
  a.v = static_cast<const u16 *>(v);
  a.o = static_cast<u16 *>(out);
  a.outer = outer;
  a.L = L;
  a.n_valid = n_valid;
  a.H = H;
  a.c = (float)((double)scale * 1.4426950408889634);
  return a;
}

}  // namespace

bool attn_bf16_supported(int d) { return d == 64 || d == 72 || d == 128; }
bool attn_short_supported(int L, int d) { return L <= 64 && (d == 64 || d == 72); }

st_status launch_attn_bf16(const void *q, const void *k, const void *v, int64_t outer, int L, int n_valid, int H,
                           int d, float scale, void *out, hipStream_t s) {
  if (outer == 0 || L == 0) return ST_OK;
  const AttnArgs a = make_args(q, k, v, outer, L, n_valid, H, scale, out);
  switch (d) {
    case 72: return launch_long<72, 2>(a, s);
    case 64: return launch_long<64, 2>(a, s);
    case 128: return launch_long<128, 1>(a, s);
    default: return ST_EUNSUPPORTED;
  }
}

st_status launch_attn_short_bf16(const void *q, const void *k, const void *v, int64_t outer, int L, int n_valid,
                                 int H, int d, float scale, void *out, hipStream_t s) {
  if (outer == 0 || L == 0) return ST_OK;
  const AttnArgs a = make_args(q, k, v, outer, L, n_valid, H, scale, out);
  if (d == 72) return L <= 32 ? launch_short<72, 1>(a, s) : launch_short<72, 2>(a, s);
  if (d == 64) return L <= 32 ? launch_short<64, 1>(a, s) : launch_short<64, 2>(a, s);
  return ST_EUNSUPPORTED;
}

}  // namespace st
