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
// Tiling: 8 waves as 2 (channels) x 4 (tokens); a wave owns 16*CT channels x
// 64 tokens (CT*4 accumulator tiles), a workgroup 32*CT channels x 256 tokens.
// Both operands reach LDS by direct global->LDS loads, K advancing 64 per step
// (whole 128-byte lines of both operands) through two LDS stages.  Moving
// operands from L2 into LDS, not the MFMAs, bounds this kernel, so the tile is
// as large as the LDS allows and every load instruction covers whole lines.
// The grid is remapped so the channel tiles of one token block run on the same
// XCD and share its L2 copy of the activations.
#include <type_traits>

#include "st_internal.h"

namespace st {
namespace {

constexpr int kBK = 64;          // K per pipeline step (128-byte rows in LDS)
constexpr int kTT = 4;           // 16-token MFMA tiles per wave
constexpr int kWM = 16 * kTT;    // tokens per wave
constexpr int kWavesM = 4;        // token-direction waves per workgroup
constexpr int kThreads = 64 * 2 * kWavesM;
constexpr int kBM = kWavesM * kWM;  // tokens per workgroup
constexpr int kStages = 2;       // LDS pipeline depth
constexpr uint32_t kGroupN = 16; // channel tiles sharing a token-block sweep

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

struct GemmArgs {
  const u16 *x;      // [M, K]
  const u16 *w;      // [N, K]
  int64_t M;
  int K, N;
  // plain output
  u16 *y;            // [M, N]
  RowMap ymap;       // MODE 0: row r of the product is stored at row map_row(r, ymap) of y
  RowMap xmap;       // with XMAP: row r of the product reads row map_row(r, xmap) of x
  // qkv output
  u16 *q, *k, *v;    // [M, H, D]
  int H;
  const float *g_q, *g_k;
  float eps;
  float q_scale;     // q is stored times q_scale
  RopeArgs rope;
};

template <int CT>
struct Tile {
  static constexpr int WN = 16 * CT;                 // channels per wave
  static constexpr int BN = 2 * WN;                  // channels per workgroup
  static constexpr int LDS_A = BN * kBK;             // u16 per stage: W rows
  static constexpr int LDS_B = kBM * kBK;            // u16 per stage: X rows
  static constexpr int STAGE = LDS_A + LDS_B;
  static constexpr int A_BLOCKS = LDS_A * 2 / 1024;  // 1 KB direct-to-LDS loads per stage
  static constexpr int B_BLOCKS = LDS_B * 2 / 1024;
  static constexpr int BLOCKS = A_BLOCKS + B_BLOCKS;
  static constexpr int NWAVES = kThreads / 64;
  static constexpr int PER_WAVE = (BLOCKS + NWAVES - 1) / NWAVES;
  static_assert(LDS_A * 2 % 1024 == 0 && LDS_B * 2 % 1024 == 0, "stage must be whole 1 KB blocks");
};

// LDS layout of a stage: rows of 64 bf16 (eight 16-byte chunks); chunk kc of row
// r sits in slot r*8 + (kc ^ (r & 7)), so the 16-byte operand reads of 8
// consecutive rows at one kc hit 8 disjoint bank quads.
__device__ __forceinline__ int slot_of(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

// Global -> LDS loads of one stage: 1 KB (8 whole rows) per wavefront
// instruction, lane l of block b filling slot 64 b + l.  Each lane's element offset inside the K
// window is fixed for the whole K loop and computed once; rows past M or N
// repeat the last row (their results are never stored).  With XMAP the x rows
// go through a.xmap and their offsets are from a.x (64-bit), else from the
// tile's first row.
template <int CT, bool XMAP>
struct GemmDma {
  typedef Tile<CT> TL;
  typedef typename std::conditional<XMAP, int64_t, int>::type Off;
  Off off[TL::PER_WAVE];

  __device__ __forceinline__ void init(const GemmArgs &a, int64_t m0, int n0, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < TL::PER_WAVE; ++i) {
      const int n = wave + TL::NWAVES * i;
      const bool isb = n >= TL::A_BLOCKS;
      const int sl = (isb ? n - TL::A_BLOCKS : n) * 64 + lane;
      const int row = sl >> 3;
      const int kc = (sl & 7) ^ (row & 7);
      if (XMAP && isb) {
        off[i] = map_row(min<int64_t>(m0 + row, a.M - 1), a.xmap) * a.K + 8 * kc;
      } else {
        const int r = isb ? (int)(min<int64_t>(m0 + row, a.M - 1) - m0) : min(n0 + row, a.N - 1);
        off[i] = r * a.K + 8 * kc;
      }
    }
  }

  __device__ __forceinline__ void issue(u16 *__restrict__ stage, int k0, const u16 *xb, const u16 *w, int wave) const {
#pragma unroll
    for (int i = 0; i < TL::PER_WAVE; ++i) {
      const int n = wave + TL::NWAVES * i;
      if (n < TL::BLOCKS) {
        const bool isb = n >= TL::A_BLOCKS;
        const int b = isb ? n - TL::A_BLOCKS : n;
        const u16 *src = (isb ? xb : w) + off[i] + k0;
        u16 *dst = stage + (isb ? TL::LDS_A : 0) + b * 512;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
      }
    }
  }
};

// One K step for one wave: issue the next step's loads into `nxt`, then
// 2 x CT x 4 MFMAs on the stage in As / Bs.  Stage pointers are restrict-qualified:
// the loads in flight never alias the stage being read.
template <int CT, bool XMAP>
__device__ __forceinline__ void gemm_step(const u16 *__restrict__ As, const u16 *__restrict__ Bs,
                                          u16 *__restrict__ nxt, bool prefetch, int k_next, const GemmDma<CT, XMAP> &dma,
                                          const u16 *xb, const u16 *w, int wave, int wn, int wm, int l16, int g4,
                                          f32x4 (&acc)[CT][kTT]) {
  typedef Tile<CT> TL;
  if (prefetch) dma.issue(nxt, k_next, xb, w, wave);
#pragma unroll
  for (int ks = 0; ks < kBK / 32; ++ks) {
    bf16x8 bf[kTT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
      bf[tt] = *reinterpret_cast<const bf16x8 *>(Bs + slot_of(wm * kWM + tt * 16 + l16, ks * 4 + g4) * 8);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const bf16x8 af = *reinterpret_cast<const bf16x8 *>(As + slot_of(wn * TL::WN + ct * 16 + l16, ks * 4 + g4) * 8);
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
        acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[tt], acc[ct][tt], 0, 0, 0);
    }
  }
}

template <int CT, int D, typename TabPtr>
__device__ __forceinline__ void epilogue_qkv(const GemmArgs &a, f32x4 (&acc)[CT][kTT], int64_t m0, int nw0, int wm,
                                             int l16, int g4, TabPtr tab);

// Floats of the RoPE table (npos positions x pairs x {cos, sin}); 0 without RoPE.
template <int D>
__device__ __forceinline__ int64_t rope_table_floats(const RopeArgs &r) {
  if (r.kind == ST_ROPE_NONE) return 0;
  return (int64_t)r.npos * (r.kind == ST_ROPE_2D ? D / 4 : D / 2) * 2;
}

// MODE 0: plain output y.  MODE 1: q/k/v with RMSNorm + RoPE on q, k (head dim D).
template <int CT, int MODE, int D, bool XMAP>
__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_kernel(GemmArgs a, uint32_t n_tiles_n, uint32_t nblocks) {
  typedef Tile<CT> TL;
  __shared__ __attribute__((aligned(16))) u16 lds[kStages * TL::STAGE];

  // Tile order: channel tiles in groups of kGroupN, token blocks running
  // fastest inside a group, and each XCD taking a contiguous range of that
  // order.  An XCD then streams activations past a ~2.6 MB slice of W that
  // stays in its L2, instead of cycling through all of W per token block.
  const uint32_t tile = xcd_remap(blockIdx.x, nblocks);
  const uint32_t n_tiles_m = nblocks / n_tiles_n;
  const uint32_t grp = tile / (kGroupN * n_tiles_m);
  const uint32_t gsz = min(kGroupN, n_tiles_n - grp * kGroupN);
  const uint32_t rem = tile - grp * kGroupN * n_tiles_m;
  const int64_t m0 = (int64_t)(rem / gsz) * kBM;
  const int n0 = (int)(grp * kGroupN + rem % gsz) * TL::BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;   // 2 channel waves x kWavesM token waves
  const int l16 = lane & 15, g4 = lane >> 4;

  f32x4 acc[CT][kTT];
#pragma unroll
  for (int i = 0; i < CT; ++i)
#pragma unroll
    for (int j = 0; j < kTT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  GemmDma<CT, XMAP> dma;
  dma.init(a, m0, n0, lane, wave);
  const u16 *xb = XMAP ? a.x : a.x + m0 * a.K;
  const int nk = a.K / kBK;
  // MODE 1: the RoPE table moves into the stage the last K step leaves free
  // (its loads overlap that step's MFMAs), so the epilogue's cos/sin reads are
  // LDS reads instead of dependent global loads.  Tables larger than a stage
  // are read from global memory.
  int64_t tab_floats = 0;
  if constexpr (MODE == 1) tab_floats = rope_table_floats<D>(a.rope);
  const bool tab_lds = tab_floats > 0 && tab_floats * 4 <= TL::STAGE * 2;
  dma.issue(lds, 0, xb, a.w, wave);
  wait_vmem_upto<0>();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    u16 *cur = lds + (kt & 1) * TL::STAGE;
    u16 *nxt = lds + ((kt & 1) ^ 1) * TL::STAGE;
    if (kt + 1 == nk && tab_lds) {
      // 1 KB per wave instruction; the last block's lanes past the end re-read the last 16 bytes
      const int blocks = (int)((tab_floats + 255) / 256);
      for (int b = wave; b < blocks; b += TL::NWAVES) {
        const int64_t f = min<int64_t>((int64_t)b * 256 + lane * 4, tab_floats - 4);
        __builtin_amdgcn_global_load_lds(a.rope.table + f, (__attribute__((address_space(3))) void *)(nxt + b * 512),
                                         16, 0, 0);
      }
    }
    gemm_step<CT, XMAP>(cur, cur + TL::LDS_A, nxt, kt + 1 < nk, (kt + 1) * kBK, dma, xb, a.w, wave, wn, wm, l16, g4,
                        acc);
    wait_vmem_upto<0>();
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  const int nw0 = n0 + wn * TL::WN;   // first channel of this wave
  if constexpr (MODE == 0) {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int64_t r = m0 + wm * kWM + tt * 16 + l16;
      if (r >= a.M) continue;
      u16 *yr = a.y + map_row(r, a.ymap) * a.N;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = nw0 + ct * 16 + g4 * 4;
        if (n >= a.N) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[ct][tt][0], acc[ct][tt][1]);
        o.y = pack_bf16x2(acc[ct][tt][2], acc[ct][tt][3]);
        *reinterpret_cast<uint2 *>(yr + n) = o;
      }
    }
  } else {
    if (tab_lds) {
      const float *t = reinterpret_cast<const float *>(lds + (nk & 1) * TL::STAGE);   // the last step's free stage
      epilogue_qkv<CT, D>(a, acc, m0, nw0, wm, l16, g4, t);
    } else {
      epilogue_qkv<CT, D>(a, acc, m0, nw0, wm, l16, g4, a.rope.table);
    }
  }
}

// MODE 1 epilogue: the wave's channels are HPW whole heads.
template <int CT, int D, typename TabPtr>
__device__ __forceinline__ void epilogue_qkv(const GemmArgs &a, f32x4 (&acc)[CT][kTT], int64_t m0, int nw0, int wm,
                                             int l16, int g4, TabPtr tab) {
  typedef Tile<CT> TL;
  constexpr int HPW = TL::WN / D;
  static_assert(TL::WN % D == 0, "wave channel range must hold whole heads");
  const int H = a.H;
  const int hd = H * D;
  const int gh0 = nw0 / D;   // global head index (over 3H) of the wave's first head
  const int npairs = a.rope.kind == ST_ROPE_2D ? D / 4 : D / 2;

  // A wave whose heads are all v heads stores the projection as it is.
  if (gh0 / H == 2 && (gh0 + HPW - 1) / H == 2) {
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int64_t r = m0 + wm * kWM + tt * 16 + l16;
      if (r >= a.M) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int cl = ct * 16 + g4 * 4;
        const int gh = gh0 + cl / D;
        if (gh >= 3 * H) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[ct][tt][0], acc[ct][tt][1]);
        o.y = pack_bf16x2(acc[ct][tt][2], acc[ct][tt][3]);
        *reinterpret_cast<uint2 *>(a.v + r * hd + (gh - 2 * H) * D + (cl - (cl / D) * D)) = o;
      }
    }
    return;
  }

  // Pass 1, per token row of the lane: 1 / RMS of each head of the wave, and
  // the token's RoPE position.  A lane's 4 channels of one MFMA tile belong to
  // one head; the head's sum of squares is completed over the 4 lanes that
  // share the token (lane groups 16 apart).
  float inv[kTT][HPW];
  int p0[kTT], p1[kTT];
  int64_t roff[kTT];         // element offset of the lane's token row in q, k, v; -1: past the last row
  const uint32_t period = (uint32_t)min<int64_t>(a.rope.period, 1ll << 30);
  const uint32_t base_i = a.rope.kind == ST_ROPE_NONE ? 0u : (uint32_t)(m0 % a.rope.period);   // one per workgroup
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt) {
    float ss[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) ss[hh] = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int hh = (ct * 16 + g4 * 4) / D;
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
      inv[tt][hh] = rsqrtf(ss[hh] * (1.0f / D) + a.eps);
    }
    const int64_t r = m0 + wm * kWM + tt * 16 + l16;
    roff[tt] = r < a.M ? r * hd : -1;
    p0[tt] = p1[tt] = 0;
    if (a.rope.kind != ST_ROPE_NONE) {
      if (a.rope.pos) {   // caller's positions, clamped into the table (out-of-range positions are undefined)
        const int2 pp = *reinterpret_cast<const int2 *>(a.rope.pos + 2 * min<int64_t>(r, a.M - 1));
        p0[tt] = min(max(pp.x, 0), a.rope.npos - 1);
        p1[tt] = min(max(pp.y, 0), a.rope.npos - 1);
      } else {
        const uint32_t i = (base_i + (uint32_t)(wm * kWM + tt * 16 + l16)) % period + (uint32_t)a.rope.offset;
        if (a.rope.kind == ST_ROPE_1D) {
          p0[tt] = (int)i;
        } else {
          p0[tt] = (int)(i / (uint32_t)a.rope.grid_w);
          p1[tt] = (int)(i - (uint32_t)p0[tt] * (uint32_t)a.rope.grid_w);
        }
      }
    }
  }

  // Pass 2, channel tile outer: the tile's head, section (q, k, v), gains and
  // rotation pair are fixed for all token rows.  GENERAL covers a wave with
  // rows past the last one, channel tiles past the last head or v heads
  // (by select, no divergent branch); every other wave takes the copy of the
  // loop without those checks.
  auto pass2 = [&](auto general) {
    constexpr bool GENERAL = decltype(general)::value;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int cl = ct * 16 + g4 * 4;
      const int hh = cl / D;
      const int gh = gh0 + hh;
      if (GENERAL && gh >= 3 * H) continue;
      const int which = gh / H;              // 0 q, 1 k, 2 v
      const int jd = cl - hh * D;            // dim within the head (multiple of 4)
      const bool norm = !GENERAL || which < 2;
      float4 g = *reinterpret_cast<const float4 *>((which == 0 ? a.g_q : a.g_k) + jd);
      if (which == 0) g = make_float4(g.x * a.q_scale, g.y * a.q_scale, g.z * a.q_scale, g.w * a.q_scale);
      const bool second = a.rope.kind == ST_ROPE_2D && jd >= D / 2;
      const int pair = (jd - (second ? D / 2 : 0)) >> 1;
      u16 *dst = (which == 0 ? a.q : (which == 1 ? a.k : a.v)) + (gh - which * H) * D + jd;
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
        if (GENERAL && roff[tt] < 0) continue;
        float invh = inv[tt][0];
#pragma unroll
        for (int h2 = 1; h2 < HPW; ++h2) invh = hh == h2 ? inv[tt][h2] : invh;
        float o[4] = {acc[ct][tt][0] * invh * g.x, acc[ct][tt][1] * invh * g.y, acc[ct][tt][2] * invh * g.z,
                      acc[ct][tt][3] * invh * g.w};
        if (a.rope.kind != ST_ROPE_NONE) {
          const int pos = second ? p1[tt] : p0[tt];
          const float4 cs = *reinterpret_cast<const float4 *>(tab + ((int64_t)pos * npairs + pair) * 2);
          const float x0 = o[0], x1 = o[1], x2 = o[2], x3 = o[3];
          o[0] = x0 * cs.x - x1 * cs.y;
          o[1] = x0 * cs.y + x1 * cs.x;
          o[2] = x2 * cs.z - x3 * cs.w;
          o[3] = x2 * cs.w + x3 * cs.z;
        }
        if (GENERAL)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = norm ? o[j] : acc[ct][tt][j];
        uint2 ov;
        ov.x = pack_bf16x2(o[0], o[1]);
        ov.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2 *>(dst + roff[tt]) = ov;
      }
    }
  };
  const bool full_rows = m0 + kBM <= a.M;       // whole workgroup
  if (full_rows && gh0 + HPW <= 2 * H) pass2(std::false_type{});   // q and k heads only, every row present
  else pass2(std::true_type{});
}

template <int CT, int MODE, int D, bool XMAP = false>
st_status launch_gemm(const GemmArgs &a, hipStream_t s) {
  typedef Tile<CT> TL;
  if (a.M == 0) return ST_OK;
  const int64_t mt = (a.M + kBM - 1) / kBM;
  const uint32_t nt = (a.N + TL::BN - 1) / TL::BN;
  const int64_t nb = mt * nt;
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((gemm_bf16_kernel<CT, MODE, D, XMAP>), dim3((uint32_t)nb), dim3(kThreads), 0, s, a, nt,
                     (uint32_t)nb);
  return launch_status();
}

}  // namespace

st_status launch_qkv_bf16(const void *x, int64_t rows, int c_in, const void *w, const float *g_q, const float *g_k,
                          float eps, float q_scale, const RopeArgs &rope, int H, int d, void *q, void *k, void *v,
                          hipStream_t s, RowMap xmap) {
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
  a.q_scale = q_scale;
  a.rope = rope;
  a.xmap = xmap;
  const bool mapped = xmap.n1 != 0;
  switch (d) {
    case 72: return mapped ? launch_gemm<9, 1, 72, true>(a, s) : launch_gemm<9, 1, 72>(a, s);   // 2 heads x 72
    case 64: return mapped ? launch_gemm<8, 1, 64, true>(a, s) : launch_gemm<8, 1, 64>(a, s);   // 2 heads x 64
    case 128: return mapped ? launch_gemm<8, 1, 128, true>(a, s) : launch_gemm<8, 1, 128>(a, s);   // 1 head x 128
    default: return ST_EUNSUPPORTED;
  }
}

st_status launch_linear_bf16(const void *a_, int64_t rows, int k_in, const void *w, int n_out, void *y,
                             hipStream_t s, RowMap ymap) {
  GemmArgs a{};
  a.x = static_cast<const u16 *>(a_);
  a.w = static_cast<const u16 *>(w);
  a.M = rows;
  a.K = k_in;
  a.N = n_out;
  a.y = static_cast<u16 *>(y);
  a.ymap = ymap;
  if (n_out % 288 == 0) return launch_gemm<9, 0, 0>(a, s);
  return launch_gemm<8, 0, 0>(a, s);
}

}  // namespace st
