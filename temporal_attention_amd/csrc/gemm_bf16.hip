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
#include <atomic>
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
constexpr uint32_t kGroupN = 16; // channel tiles per group of the tile order (tile_origin)

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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

// Epilogue staging.  A lane's accumulators hold 4 consecutive channels of one
// token, so stores straight from them write 32-byte pieces of 16 different
// rows per instruction.  Instead each wave converts ROWS tokens x WN channels
// at a time to bf16 into its own LDS slot, reads them back along the rows and
// stores 16 bytes per lane: a store instruction then covers whole stretches of
// 3.5 token rows.  The slots sit in LDS the K loop no longer needs (ROWS = 32
// when both stages are free, 16 when one already holds the next tile's first K
// slice) and need no workgroup barrier (a wave reads back only what it wrote).
// Rows of RS = 144 bf16 (288 bytes, 72 banks) put the 8-byte writes of 8
// consecutive rows x 4 lane groups on 64 distinct banks.
template <int CT, int ROWS>
struct Staging {
  static constexpr int WN = 16 * CT;
  static constexpr int RS = WN == 128 ? 144 : WN;   // row stride in bf16
  static constexpr int CH = WN / 8;                 // 16-byte chunks per token row
  static constexpr int SLOT = ROWS * RS;            // bf16 per wave slot
  static constexpr int TPR = ROWS / 16;             // 16-token MFMA tiles per round
  static constexpr int ROUNDS = kTT / TPR;
  static constexpr int IT = (ROWS * CH + 63) / 64;  // 64-lane read-back steps per round
  static_assert(RS * 2 % 32 == 0 && (RS * 2 / 4) % 64 == 8, "row stride must spread 8 rows over the banks");
  static_assert(ROWS == 16 || ROWS == 32, "one or two token tiles per round");
};

// Global -> LDS loads of one stage: 1 KB (8 whole rows) per wavefront
// instruction, lane l of block b filling slot 64 b + l.  Each lane's element
// offset inside a tile's K window is computed per tile; rows past M or N
// repeat the last row (their results are never stored).  With XMAP the x rows
// go through a.xmap and their offsets are from a.x (64-bit), else from the
// tile's first row.
template <int CT, bool XMAP>
struct GemmDma {
  typedef Tile<CT> TL;
  typedef typename std::conditional<XMAP, int64_t, int>::type Off;
  Off off[TL::PER_WAVE];
  const u16 *xb, *w;   // bases of the x offsets and of the W offsets

  __device__ __forceinline__ void set_tile(const GemmArgs &a, int64_t m0, int n0, int lane, int wave) {
    xb = XMAP ? a.x : a.x + m0 * a.K;
    w = a.w;
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

  __device__ __forceinline__ void issue(u16 *__restrict__ stage, int k0, int wave) const {
#pragma unroll
    for (int i = 0; i < TL::PER_WAVE; ++i) {
      const int n = wave + TL::NWAVES * i;
      if (n < TL::BLOCKS) {
        const bool isb = n >= TL::A_BLOCKS;
        const int b = isb ? n - TL::A_BLOCKS : n;
        __builtin_amdgcn_global_load_lds((isb ? xb : w) + off[i] + k0,
                                         (__attribute__((address_space(3))) void *)(stage + (isb ? TL::LDS_A : 0) +
                                                                                    b * 512),
                                         16, 0, 0);
      }
    }
  }
};

// The MFMAs of one K step for one wave: 2 x CT x 4 on the stage in As / Bs, in
// groups of one channel tile (4 MFMAs) whose A operand (and, at a K slice's
// first group, the 4 B operands) is read from LDS one group ahead.  The wait at
// the top of a group is explicit and comes before the next group's reads are
// issued: while direct-to-LDS loads are in flight the compiler only ever waits
// for all outstanding LDS reads, so a wait it placed after those reads would
// also wait for them.
template <int CT>
__device__ __forceinline__ void gemm_step(const u16 *__restrict__ As, const u16 *__restrict__ Bs, int wn, int wm,
                                          int l16, int g4, f32x4 (&acc)[CT][kTT]) {
  typedef Tile<CT> TL;
  constexpr int NG = (kBK / 32) * CT;   // groups (K slice ks, channel tile ct) of the step
  bf16x8 bfr[kBK / 32][kTT], afr[kBK / 32][CT];
  auto issue_reads = [&](int gi) {
    const int ks = gi / CT, ct = gi % CT;
    if (ct == 0)
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt)
        bfr[ks][tt] = *reinterpret_cast<const bf16x8 *>(Bs + slot_of(wm * kWM + tt * 16 + l16, ks * 4 + g4) * 8);
    afr[ks][ct] = *reinterpret_cast<const bf16x8 *>(As + slot_of(wn * TL::WN + ct * 16 + l16, ks * 4 + g4) * 8);
  };
  issue_reads(0);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    wait_lds_reads();
    __builtin_amdgcn_sched_barrier(0);
    if (gi + 1 < NG) issue_reads(gi + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int ks = gi / CT, ct = gi % CT;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
      acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ks][ct], bfr[ks][tt], acc[ct][tt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Orders a wave's LDS writes before its reads of other lanes' data (LDS executes
// one wave's instructions in order; this only keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Floats of the RoPE table (npos positions x pairs x {cos, sin}); 0 without RoPE.
template <int D>
__device__ __forceinline__ int64_t rope_table_floats(const RopeArgs &r) {
  if (r.kind == ST_ROPE_NONE) return 0;
  return (int64_t)r.npos * (r.kind == ST_ROPE_2D ? D / 4 : D / 2) * 2;
}

// MODE 1: LDS past the two pipeline stages holds g_q | g_k (1 KB, fp32) and the
// RoPE table when it fits, loaded once per workgroup; larger tables are read
// from global memory.
constexpr int kAuxU16 = 12288;    // 24 KB: 2 stages + aux stay within 160 KB
constexpr int kGainsU16 = 512;

// First token row and first channel of tile v.  Channel tiles go in groups of
// kGroupN; inside a group the channel tiles of one token block run back to
// back (they share the block's activations in the XCD's L2), then the next
// token block; each XCD takes a contiguous range of that order (xcd_remap).
// A 1152-wide projection (4 channel tiles, 2.6 MB of W) keeps its weights in
// L2; the 3456-wide QKV weights (8 MB) are re-read from the Infinity Cache per
// token block, which measured faster than orders that keep a 4-tile weight
// slice in L2 and re-read activations instead.
struct TileOrigin {
  int64_t m0;
  int n0;
};
template <int CT>
__device__ __forceinline__ TileOrigin tile_origin(uint32_t v, uint32_t n_tiles_n, uint32_t nblocks) {
  const uint32_t tile = xcd_remap(v, nblocks);
  const uint32_t n_tiles_m = nblocks / n_tiles_n;
  const uint32_t grp = tile / (kGroupN * n_tiles_m);
  const uint32_t gsz = min(kGroupN, n_tiles_n - grp * kGroupN);
  const uint32_t rem = tile - grp * kGroupN * n_tiles_m;
  return TileOrigin{(int64_t)(rem / gsz) * kBM, (int)(grp * kGroupN + rem % gsz) * Tile<CT>::BN};
}

// MODE 0 epilogue: the wave's 64 tokens x WN channels to y, through its slot.
template <int CT, int ROWS>
__device__ __forceinline__ void epilogue_plain(const GemmArgs &a, f32x4 (&acc)[CT][kTT], int64_t m0, int nw0,
                                               int wm, int lane, u16 *slot) {
  typedef Staging<CT, ROWS> SG;
  const int l16 = lane & 15, g4 = lane >> 4;
  if (a.N % 8 != 0 || (reinterpret_cast<uintptr_t>(a.y) & 15) != 0) {   // rows not 16-byte aligned: direct
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int64_t r = m0 + wm * kWM + tt * 16 + l16;
      if (r >= a.M) continue;
      u16 *yr = a.y + map_row(r, a.ymap) * a.N;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = nw0 + ct * 16 + g4 * 4;
        if (n >= a.N) continue;
        *reinterpret_cast<uint2 *>(yr + n) =
            uint2{pack_bf16x2(acc[ct][tt][0], acc[ct][tt][1]), pack_bf16x2(acc[ct][tt][2], acc[ct][tt][3])};
      }
    }
    return;
  }
  const int64_t rl = m0 + wm * kWM + lane;   // the lane's token row, mapped once
  const int64_t roff = rl < a.M ? map_row(rl, a.ymap) * a.N : -1;
#pragma unroll
  for (int rd = 0; rd < SG::ROUNDS; ++rd) {
#pragma unroll
    for (int t2 = 0; t2 < SG::TPR; ++t2)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const f32x4 &c = acc[ct][rd * SG::TPR + t2];
        *reinterpret_cast<uint2 *>(slot + (t2 * 16 + l16) * SG::RS + ct * 16 + g4 * 4) =
            uint2{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
      }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < SG::IT; ++it) {
      const int c = min(it * 64 + lane, ROWS * SG::CH - 1);
      const int tok = c / SG::CH, ch = c - tok * SG::CH;
      const int64_t ro = __shfl(roff, rd * ROWS + tok);
      const uint4 v = *reinterpret_cast<const uint4 *>(slot + tok * SG::RS + ch * 8);
      const int n = nw0 + ch * 8;
      if (it * 64 + lane < ROWS * SG::CH && ro >= 0 && n < a.N) *reinterpret_cast<uint4 *>(a.y + ro + n) = v;
    }
    wave_lds_sync();
  }
}

// MODE 1 epilogue: the wave's channels are HPW whole heads; the results go out
// through the wave's slot, ROWS tokens at a time.
template <int CT, int D, int ROWS, typename TabPtr>
__device__ __forceinline__ void epilogue_qkv(const GemmArgs &a, f32x4 (&acc)[CT][kTT], int64_t m0, int nw0, int wm,
                                             int lane, u16 *slot, const float *gains, TabPtr tab) {
  typedef Tile<CT> TL;
  typedef Staging<CT, ROWS> SG;
  constexpr int HPW = TL::WN / D;
  static_assert(TL::WN % D == 0, "wave channel range must hold whole heads");
  static_assert(D % 8 == 0, "a 16-byte chunk must not straddle two heads");
  const int l16 = lane & 15, g4 = lane >> 4;
  const int H = a.H;
  const int hd = H * D;
  const int gh0 = nw0 / D;   // global head index (over 3H) of the wave's first head
  const int npairs = a.rope.kind == ST_ROPE_2D ? D / 4 : D / 2;

  // Where each head of the wave starts in q, k or v (wave-uniform), and whether it exists.
  u16 *hbase[HPW];
  bool hok[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int gh = gh0 + hh, which = gh / H;
    hok[hh] = gh < 3 * H;
    hbase[hh] = (which == 0 ? a.q : (which == 1 ? a.k : a.v)) + (gh - which * H) * D;
  }
  // Stores round RD of the wave from its slot: chunk c is 8 channels of token
  // row c / CH of the round, inside one head.
  auto flush = [&](auto rd_c) {
    constexpr int RD = decltype(rd_c)::value;
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < SG::IT; ++it) {
      const int c = min(it * 64 + lane, ROWS * SG::CH - 1);
      const int tok = c / SG::CH, ch = c - tok * SG::CH;
      const int cl = ch * 8, hh = cl / D;
      const int64_t r = m0 + wm * kWM + RD * ROWS + tok;
      const uint4 v = *reinterpret_cast<const uint4 *>(slot + tok * SG::RS + cl);
      u16 *base = hbase[0];
      bool ok = hok[0];
#pragma unroll
      for (int h2 = 1; h2 < HPW; ++h2) {
        base = hh == h2 ? hbase[h2] : base;
        ok = hh == h2 ? hok[h2] : ok;
      }
      if (it * 64 + lane < ROWS * SG::CH && r < a.M && ok)
        *reinterpret_cast<uint4 *>(base + r * hd + (cl - hh * D)) = v;
    }
    wave_lds_sync();
  };
  auto put = [&](int t2, int ct, const uint2 &o) {
    *reinterpret_cast<uint2 *>(slot + (t2 * 16 + l16) * SG::RS + ct * 16 + g4 * 4) = o;
  };
  typedef std::integral_constant<int, 0> T0;
  typedef std::integral_constant<int, 1> T1;
  typedef std::integral_constant<int, 2> T2;
  typedef std::integral_constant<int, 3> T3;

  // Every round of the wave's tile, in order.
  auto rounds = [&](auto fn) {
    fn(T0{});
    fn(T1{});
    if constexpr (SG::ROUNDS == 4) {
      fn(T2{});
      fn(T3{});
    }
  };

  // A wave whose heads are all v heads stores the projection as it is.
  if (gh0 / H == 2 && (gh0 + HPW - 1) / H == 2) {
    rounds([&](auto rd_c) {
      constexpr int RD = decltype(rd_c)::value;
#pragma unroll
      for (int t2 = 0; t2 < SG::TPR; ++t2)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x4 &c = acc[ct][RD * SG::TPR + t2];
          put(t2, ct, uint2{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])});
        }
      flush(rd_c);
    });
    return;
  }

  // Pass 1, per token row of the lane: 1 / RMS of each head of the wave, and
  // the token's RoPE position.  A lane's 4 channels of one MFMA tile belong to
  // one head; the head's sum of squares is completed over the 4 lanes that
  // share the token (lane groups 16 apart).
  float inv[kTT][HPW];
  int p0[kTT], p1[kTT];
  const uint32_t period = (uint32_t)min<int64_t>(a.rope.period, 1ll << 30);
  const uint32_t base_i = a.rope.kind == ST_ROPE_NONE ? 0u : (uint32_t)(m0 % a.rope.period);   // one per tile
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

  // Pass 2, round RD, channel tile outer, into the slot: the tile's head,
  // section (q, k, v), gains and rotation pair are fixed for all token rows.
  // GENERAL covers a wave with channel tiles past the last head or v heads (by
  // select, no divergent branch); every other wave takes the copy of the loop
  // without those checks.  Rows past the last one are computed from the
  // repeated (or zero) last rows of x and never stored.
  auto pass2 = [&](auto general, auto rd_c) {
    constexpr bool GENERAL = decltype(general)::value;
    constexpr int RD = decltype(rd_c)::value;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int cl = ct * 16 + g4 * 4;
      const int hh = cl / D;
      const int gh = gh0 + hh;
      if (GENERAL && gh >= 3 * H) continue;
      const int which = gh / H;              // 0 q, 1 k, 2 v
      const int jd = cl - hh * D;            // dim within the head (multiple of 4)
      const bool norm = !GENERAL || which < 2;
      float4 g = *reinterpret_cast<const float4 *>(gains + (which == 0 ? 0 : D) + jd);   // LDS copy of g_q | g_k
      if (which == 0) g = make_float4(g.x * a.q_scale, g.y * a.q_scale, g.z * a.q_scale, g.w * a.q_scale);
      const bool second = a.rope.kind == ST_ROPE_2D && jd >= D / 2;
      const int pair = (jd - (second ? D / 2 : 0)) >> 1;
#pragma unroll
      for (int t2 = 0; t2 < SG::TPR; ++t2) {
        const int tt = RD * SG::TPR + t2;
        float invh = inv[tt][0];
#pragma unroll
        for (int h2 = 1; h2 < HPW; ++h2) invh = hh == h2 ? inv[tt][h2] : invh;
        const f32x4 &c = acc[ct][tt];
        float o[4] = {c[0] * invh * g.x, c[1] * invh * g.y, c[2] * invh * g.z, c[3] * invh * g.w};
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
          for (int j = 0; j < 4; ++j) o[j] = norm ? o[j] : c[j];
        put(t2, ct, uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
      }
    }
    flush(rd_c);
  };
  if (gh0 + HPW <= 2 * H) rounds([&](auto rd_c) { pass2(std::false_type{}, rd_c); });   // q and k heads only
  else rounds([&](auto rd_c) { pass2(std::true_type{}, rd_c); });
}

// MODE 0: plain output y.  MODE 1: q/k/v with RMSNorm + RoPE on q, k (head dim D).
// PERSIST (MODE 0 without XMAP): workgroup b takes tiles b, b + gridDim.x, ...
// (tile_origin order), and the K pipeline runs on across tiles: the last K
// step of a tile loads the next tile's first K slice into the free stage, and
// the next tile's second slice is issued right after the epilogue, so one
// tile's stores drain while the next one computes, and no workgroup waits for
// its stores to retire before the next tile's loads start.  The other kernels
// take one tile per workgroup (their longer epilogues need more registers
// than the tile loop leaves).
template <int CT, int MODE, int D, bool XMAP>
__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_kernel(GemmArgs a, uint32_t n_tiles_n, uint32_t nblocks) {
  typedef Tile<CT> TL;
  constexpr bool PERSIST = MODE == 0 && !XMAP;
  constexpr int ROWS = PERSIST ? 16 : 32;   // staging rows per round: one stage free, or both
  typedef Staging<CT, ROWS> SG;
  static_assert(8 * SG::SLOT <= (PERSIST ? 1 : kStages) * TL::STAGE, "the wave slots fit the free stages");
  __shared__ __attribute__((aligned(16))) u16 lds[kStages * TL::STAGE + (MODE == 1 ? kAuxU16 : 0)];
  typedef __attribute__((address_space(3))) void lds_void;

  uint32_t v = blockIdx.x;
  if (v >= nblocks) return;
  const int lane = threadIdx.x & 63;
  const int wave = PERSIST ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;   // 2 channel waves x kWavesM token waves
  const int nk = a.K / kBK;

  u16 *aux = lds + kStages * TL::STAGE;
  bool tab_lds = false;
  if constexpr (MODE == 1) {
    static_assert(D <= 128, "g_q and g_k fill one 1 KB load");
    const int64_t tab_floats = rope_table_floats<D>(a.rope);
    const int blocks = (int)((tab_floats + 255) / 256);   // 1 KB per wave instruction
    tab_lds = tab_floats > 0 && kGainsU16 + blocks * 512 <= kAuxU16;
    if (wave == TL::NWAVES - 1) {   // lanes past 2 D re-read g_k's last 16 bytes into the gains block's tail
      const float *g = lane < D / 4 ? a.g_q + 4 * lane : a.g_k + 4 * min(lane - D / 4, D / 4 - 1);
      __builtin_amdgcn_global_load_lds(g, (lds_void *)aux, 16, 0, 0);
    }
    if (tab_lds)   // the last block's lanes past the end re-read the last 16 bytes
      for (int b = wave; b < blocks; b += TL::NWAVES) {
        const int64_t f = min<int64_t>((int64_t)b * 256 + lane * 4, tab_floats - 4);
        __builtin_amdgcn_global_load_lds(a.rope.table + f, (lds_void *)(aux + kGainsU16 + b * 512), 16, 0, 0);
      }
  }

  TileOrigin o = tile_origin<CT>(v, n_tiles_n, nblocks);
  GemmDma<CT, XMAP> dma;
  dma.set_tile(a, o.m0, o.n0, lane, wave);
  dma.issue(lds, 0, wave);
  wait_vmem_upto<0>();
  __syncthreads();

  int st = 0;                   // stage holding the current K slice
  bool second_loaded = false;   // the tile's second K slice was issued before its first step
  f32x4 acc[CT][kTT];
  while (true) {
    const uint32_t vn = v + gridDim.x;
    const bool has_next = PERSIST && vn < nblocks;
    // The lane index, opaque to the compiler once per tile: keeps it from
    // hoisting the epilogue's per-lane address arithmetic out of the tile loop
    // and holding dozens of such values live across the K loop.
    int ln = lane;
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (PERSIST) asm volatile("" : "+v"(ln));
#endif
    const int l16 = ln & 15, g4 = ln >> 4;
    TileOrigin on = o;
#pragma unroll
    for (int i = 0; i < CT; ++i)
#pragma unroll
      for (int j = 0; j < kTT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt + 1 < nk; ++kt) {
      u16 *cur = lds + st * TL::STAGE;
      if (kt > 0 || !second_loaded) dma.issue(lds + (st ^ 1) * TL::STAGE, (kt + 1) * kBK, wave);
      gemm_step<CT>(cur, cur + TL::LDS_A, wn, wm, l16, g4, acc);
      wait_vmem_upto<0>();
      __syncthreads();
      st ^= 1;
    }
    {   // the last K step loads the next tile's first K slice
      u16 *cur = lds + st * TL::STAGE;
      if (has_next) {
        on = tile_origin<CT>(vn, n_tiles_n, nblocks);
        dma.set_tile(a, on.m0, on.n0, ln, wave);   // ln: recomputed per tile, not hoisted
        dma.issue(lds + (st ^ 1) * TL::STAGE, 0, wave);
      }
      gemm_step<CT>(cur, cur + TL::LDS_A, wn, wm, l16, g4, acc);
      wait_vmem_upto<0>();
      __syncthreads();
      st ^= 1;
    }

    // Epilogue: PERSIST, in the stage the last step has left free (st ^ 1;
    // stage st holds the next tile's first K slice); otherwise in both stages.
    u16 *slot = (PERSIST ? lds + (st ^ 1) * TL::STAGE : lds) + wave * SG::SLOT;
    const int nw0 = o.n0 + wn * TL::WN;   // first channel of this wave
    if constexpr (MODE == 0) {
      epilogue_plain<CT, ROWS>(a, acc, o.m0, nw0, wm, ln, slot);
    } else {
      const float *gl = reinterpret_cast<const float *>(aux);
      if (tab_lds)
        epilogue_qkv<CT, D, ROWS>(a, acc, o.m0, nw0, wm, ln, slot, gl,
                                  reinterpret_cast<const float *>(aux + kGainsU16));
      else
        epilogue_qkv<CT, D, ROWS>(a, acc, o.m0, nw0, wm, ln, slot, gl, a.rope.table);
    }
    if (!has_next) break;
    __syncthreads();   // every wave has read back its slot: the stage takes the next tile's second K slice
    second_loaded = nk > 1;
    if (second_loaded) dma.issue(lds + (st ^ 1) * TL::STAGE, kBK, wave);
    v = vn;
    o = on;
  }
}

// Every kernel the launchers below use, instantiated explicitly so that the
// host pass emits all of their launch stubs.
template __global__ void gemm_bf16_kernel<9, 1, 72, false>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<9, 1, 72, true>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<8, 1, 64, false>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<8, 1, 64, true>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<8, 1, 128, false>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<8, 1, 128, true>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<9, 0, 0, false>(GemmArgs, uint32_t, uint32_t);
template __global__ void gemm_bf16_kernel<8, 0, 0, false>(GemmArgs, uint32_t, uint32_t);

// Compute units of the current device (cached per device; concurrent first
// calls store the same value): the persistent grid.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int CT, int MODE, int D, bool XMAP = false>
st_status launch_gemm(const GemmArgs &a, hipStream_t s) {
  typedef Tile<CT> TL;
  if (a.M == 0) return ST_OK;
  const int64_t mt = (a.M + kBM - 1) / kBM;
  const uint32_t nt = (a.N + TL::BN - 1) / TL::BN;
  const int64_t nb = mt * nt;
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  // persistent: one workgroup per CU (LDS-bound); otherwise one tile per workgroup
  const bool persist = MODE == 0 && !XMAP;
  const uint32_t grid = persist ? (uint32_t)std::min<int64_t>(nb, device_cus()) : (uint32_t)nb;
  hipLaunchKernelGGL((gemm_bf16_kernel<CT, MODE, D, XMAP>), dim3(grid), dim3(kThreads), 0, s, a, nt, (uint32_t)nb);
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
  // the epilogue stores 16-byte pieces of q, k, v rows
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) return ST_EALIGN;
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
