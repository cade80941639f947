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
// Long sequences (attn_long_kernel): a workgroup of 8 waves owns 32*NT
// queries per wave; K and V tiles of 128 keys (64 for d = 128) go from
// global memory straight into three rotating LDS stages, V^T is read from
// them with transpose reads, and the online softmax only rescales the
// accumulator when a query's running maximum grows by more than 8 (in log2
// units), so exponentials stay <= 2^8 in between.
// Short sequences (attn_short_kernel, L <= 64): one wave per (outer, head)
// loads its whole Q and K straight into operand registers and copies V
// global -> LDS into a private slice, read back as V^T by transpose reads; a
// workgroup covers four adjacent heads of one outer index, so its loads share
// cache lines, and every wave has exactly one head to do, so all of them are
// in flight at once.  For d = 72 the output rows go back out through the same
// slice, 16 bytes per lane along whole rows.
#include <math.h>

#include "st_internal.h"

namespace st {
namespace {

struct AttnArgs {
  const u16 *q, *k, *v;
  u16 *o;
  float *lse;          // optional [outer, H, L]: natural log-sum-exp of the scaled scores per query
  int acc;             // o and lse hold a partial result over other keys: merge this one into it, in place
  int64_t outer;
  int L, Lk, n_valid, H;   // L queries, Lk keys per sequence (equal except for chunk attention)
  float c;             // scale * log2(e)
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
  // Long kernel: when the rows past the last whole 32-row tile (the tail of
  // d, the ones row) fit in 16, they form one 16-row tile on the 16x16x32 MFMA.
  static constexpr bool PV16 = ONES && (D % 32) < 16;
  static constexpr int DT32 = PV16 ? D / 32 : DT;   // 32-row P.V tiles
  // Long kernel, d = 64 or 128: K and V rows of 128 or 256 bytes would put
  // chunk c of every row on the same LDS banks, so the 16-byte chunks of a
  // row are stored permuted: physical chunk = logical chunk ^ swizzle(row).
  // K: the 16 rows that one operand read visits at a logical chunk land on
  // 16 different bank groups.  V (transpose reads, 4 rows x 64 bytes per
  // read): the XOR moves whole 64-byte windows, so those rows differ there.
  static constexpr bool SWZ = D % 64 == 0;
  static constexpr int RPS = SWZ ? 128 / D : 1;   // rows per 256-byte bank span
  __host__ __device__ static constexpr int kswz(int r) { return SWZ ? (r / RPS) % CH : 0; }
  __host__ __device__ static constexpr int vswz(int r) { return SWZ ? 4 * ((r / RPS) % (CH / 4)) : 0; }
};

// Two LDS transpose reads, 8 keys apart, as one 8 x bf16 MFMA operand.
template <int D>
__device__ __forceinline__ uint4 tr_read_pair(const u16 *p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p + 8 * D));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
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
  float m = __builtin_fmaxf(__builtin_fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, s[i]), s[i + 1]);
  return __builtin_fmaxf(m, s[15]);
}

// max(x[l], x[l ^ 32]): the two half-waves hold the two halves of a query's keys.
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes
// 0..31 of its second, so with both operands = x the two results hold x and
// its partner in some order, and their max is the same in every lane.
__device__ __forceinline__ float max_across_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Key index (within a 32-key tile) of accumulator register r in lane half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

constexpr float kRescale = 8.0f;   // log2 growth of the running max that forces a rescale
// Keys per LDS tile of the long kernel for d <= 72: one workgroup barrier per
// tile, so larger tiles mean fewer barriers (d = 128 keeps 64 keys so three
// stages fit in LDS).
constexpr int kLongKeys = 128;
// Waves per workgroup of the long kernel: every workgroup streams all keys of
// its sequence through LDS, so more queries per workgroup means less L2->LDS
// traffic per flop.
constexpr int kLongWaves = 8;

// ------------------------------------------------------------------------- //
// Long sequences                                                            //
// ------------------------------------------------------------------------- //
template <int D, int NT, int W = kLongWaves>
struct LongCfg {
  typedef Dims<D> DM;
  static constexpr int WAVES = W;                 // waves per workgroup
  static constexpr int KB = D <= 72 ? kLongKeys : 64;  // keys per LDS tile
  static constexpr int QW = 32 * NT;              // queries per wave
  static constexpr int QB = WAVES * QW;           // queries per workgroup
  static constexpr int TILE = KB * D;             // u16 per K or V tile: rows packed as in memory
  static constexpr int SLACK = 32;                // u16 after a tile: operand reads run past the last row
  static constexpr int REGION = TILE + SLACK;
  static constexpr int STAGE = 2 * REGION;        // K tile, then V tile
  static constexpr int NSTAGE = 3;                // tiles in LDS at once
  static constexpr int BLOCKS = TILE * 2 / 1024;  // 1 KB direct-to-LDS loads per tile
  static_assert((TILE * 2) % 1024 == 0, "tile must be whole 1 KB blocks");
};

// Wait until this wave's outstanding global->LDS loads have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// K and V tiles go global -> LDS directly, 1 KB per wavefront instruction:
// lane l of block b carries 16-byte chunk 64 b + l of the packed [key][d]
// tile.  The 2 * BLOCKS blocks of a stage are dealt round-robin to the
// workgroup's waves; each lane's element offset inside a tile (key * row stride + dim) is
// fixed for the whole key loop, so it is computed once.  Keys past L repeat
// row L-1 (their scores are masked).
template <int D>
struct LongDma {
  typedef LongCfg<D, 1> C;
  static constexpr int PER_WAVE = (2 * C::BLOCKS + C::WAVES - 1) / C::WAVES;
  int off[PER_WAVE];   // element offset of this lane's chunk within a tile

  __device__ __forceinline__ static int chunk_key(int n, int lane) {
    const int b = n >= C::BLOCKS ? n - C::BLOCKS : n;
    return (b * 64 + lane) / Dims<D>::CH;
  }

  __device__ __forceinline__ void init(int64_t rs, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int n = wave + C::WAVES * i;
      const bool isv = n >= C::BLOCKS;
      const int b = isv ? n - C::BLOCKS : n;
      const int c = b * 64 + lane;
      const int row = c / Dims<D>::CH, p = c % Dims<D>::CH;   // LDS row and physical chunk
      const int chunk = p ^ (isv ? Dims<D>::vswz(row) : Dims<D>::kswz(row));
      off[i] = (int)(row * rs) + chunk * 8;
    }
  }

  __device__ __forceinline__ void issue(u16 *__restrict__ dst_stage, int kb, const u16 *kp, const u16 *vp, int64_t rs,
                                        int L, int lane, int wave) const {
    const bool tail = kb + C::KB > L;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int n = wave + C::WAVES * i;
      if (n < 2 * C::BLOCKS) {
        const bool isv = n >= C::BLOCKS;
        const int b = isv ? n - C::BLOCKS : n;
        const u16 *base = (isv ? vp : kp) + (int64_t)kb * rs;
        int o = off[i];
        if (tail) {   // repeat row L-1 for keys past L
          const int key = chunk_key(n, lane);
          if (kb + key >= L) o += (int)((L - 1 - kb - key) * rs);
        }
        u16 *dst = dst_stage + (isv ? C::REGION : 0) + b * 512;
        __builtin_amdgcn_global_load_lds(base + o, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
      }
    }
  }
};

// Per-wave state and steps of the long kernel.  The key loop runs in units of
// 32 keys and is software-pipelined: one step issues S^T = K Q^T of unit u+1,
// then the exponentials of unit u (whose rescale is already settled), then
// O^T += V^T P^T of unit u, and only then the rescale test of unit u+1.  The
// matrix products of one unit and the vector work of the other are
// independent, so the MFMA pipe and the vector ALU stay busy together.
//
// d = 72 (FOLD): the Q.K contraction is padded to 80 dimensions, and two of
// the spare ones carry the softmax bookkeeping into the MFMA.  Q dim 72 holds
// -m (the running max, kept bf16-exact) against K dim 72 = 1, and Q dim 73
// holds -1 against K dim 73 = 0 for a valid key or 2^120 for a masked one, so
// the accumulator is already the score minus the max (or about -2^120), and
// masking costs nothing in the loop.
//   PRE (c = scale * log2(e) a power of two): Q is multiplied by c exactly, so
//   the accumulator is the exp2 argument itself and a probability is one exp2.
//   The layer pair stores q already multiplied by scale * log2(e) (a gain of
//   its RMSNorm epilogue, rounded to bf16 once) and attends with c = 1.
//   Otherwise Q enters the contraction as stored and the exponent is c * acc:
//   one multiply more per score.  Rounding c * Q to bf16 in the kernel instead
//   would add a second rounding of up to 2^-8 relative to every element, which
//   peaked softmaxes turn into output errors of several 1e-2.
constexpr uint32_t kBf16One = 0x3F80u, kBf16NegOne = 0xBF80u, kBf16Big = 0x7B80u;   // 1, -1, 2^120

__device__ __forceinline__ float round_bf16(float x) { return __uint_as_float(pack_bf16x2(x, 0.f) << 16); }

template <int D, int NT, bool PRE>
struct LongWave {
  typedef LongCfg<D, NT> C;
  typedef Dims<D> DM;
  static constexpr bool FOLD = DM::DQK > D;
  static_assert(!FOLD || D % 16 == 8, "the folded terms sit in the upper half of the last Q.K step");

  bf16x8 qf[NT][DM::KS];     // Q^T operand (B of S^T = K Q^T)
  f32x16 oacc[DM::DT32][NT]; // O^T accumulator, 32-row tiles
  f32x4 oacc16[NT][2];       // PV16: last 16 rows of O^T, queries 0..15 and 16..31 of a tile
  float m[NT];               // running max (FOLD: in accumulator units, bf16-exact; else raw scores)
  float lsum[NT];            // softmax denominator when V^T has no ones row
  float c;                   // scale * log2(e)
  float thr;                 // FOLD: the rescale threshold in accumulator units (kRescale, or kRescale / c)
  int nv, l32, g, q16, v_off, v_off16;
  int koff[DM::SWZ ? DM::KS : 1];     // SWZ: K operand offset of each 16-dim step within a unit's rows
  int voff[DM::SWZ ? DM::DT32 : 1];   // SWZ: V^T read offset of each 32-row tile within a unit's rows
  bool vkeep;                // lane's row of the last P.V tile is a real V^T row
  uint32_t vconst;           // otherwise its constant (ones row or zero)

  // K operand of the 32 keys of unit u, whose K rows start at Ks.
  __device__ __forceinline__ void kfrag(bf16x8 (&kf)[DM::KS], const u16 *__restrict__ Ks, int u) const {
    uint32_t kfix = 0;
    if constexpr (FOLD) kfix = u * 32 + l32 < nv ? kBf16One : (kBf16One | kBf16Big << 16);
#pragma unroll
    for (int ks = 0; ks < DM::KS; ++ks) {
      uint4 ku;
      if constexpr (DM::SWZ)
        ku = *reinterpret_cast<const uint4 *>(Ks + koff[ks]);
      else
        ku = *reinterpret_cast<const uint4 *>(Ks + l32 * D + ks * 16 + g * 8);
      if constexpr (FOLD)
        if (ks == DM::KS - 1 && g) ku.x = kfix;
      kf[ks] = __builtin_bit_cast(bf16x8, ku);
    }
  }

  // S^T of one 32-query tile.
  __device__ __forceinline__ void qk(f32x16 &s, const bf16x8 (&kf)[DM::KS], int nt) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DM::KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[nt][ks], s, 0, 0, 0);
  }

  __device__ __forceinline__ void qk(f32x16 (&s)[NT], const u16 *__restrict__ Ks, int u) const {
    bf16x8 kf[DM::KS];
    kfrag(kf, Ks, u);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qk(s[nt], kf, nt);
  }

  // Keys of unit u at or past nv get score -inf (the FOLD path masks in qk).
  __device__ __forceinline__ void mask(f32x16 (&s)[NT], int u) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool off = u * 32 + acc_row(r, g) >= nv;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt][r] = off ? -INFINITY : s[nt][r];
    }
  }

  // Lane-local maxima of a unit's scores; true when some query's running
  // max must move (its scores exceed it by more than 2^kRescale).
  __device__ __forceinline__ bool needs_rescale(const f32x16 (&s)[NT], float (&lm)[NT]) const {
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lm[nt] = max16(s[nt]);
      if constexpr (FOLD) grow |= lm[nt] > thr;
      else grow |= (lm[nt] - m[nt]) * c > kRescale;
    }
    return __builtin_amdgcn_ballot_w64(grow) != 0;
  }

  // Move the running max to cover unit s; `first`: nothing is accumulated yet.
  __device__ __forceinline__ void rescale(f32x16 (&s)[NT], const float (&lm)[NT], bool first) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mx = max_across_halves(lm[nt]);
      if constexpr (FOLD) {
        // s holds (scaled) score - m; the new max is bf16-exact so -m fits Q dim 72.
        const float mnew = round_bf16(m[nt] + (first ? mx : fmaxf(mx, 0.f)));
        const float delta = mnew - m[nt];
        if (!first) scale_acc(nt, __builtin_amdgcn_exp2f(PRE ? -delta : -delta * c));
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nt][r] -= delta;
        m[nt] = mnew;
        uint4 qu = __builtin_bit_cast(uint4, qf[nt][DM::KS - 1]);
        if (g) qu.x = (kBf16NegOne << 16) | ((__float_as_uint(mnew) >> 16) ^ 0x8000u);
        qf[nt][DM::KS - 1] = __builtin_bit_cast(bf16x8, qu);
      } else {
        const float mnew = fmaxf(m[nt], mx);
        const float alpha = __builtin_amdgcn_exp2f((m[nt] - mnew) * c);   // 0 when first
        m[nt] = mnew;
        lsum[nt] *= alpha;
        scale_acc(nt, alpha);
      }
    }
  }

  // Whole-vector multiplies: element-wise ones make the register allocator
  // copy the MFMA accumulators on every path through the rescale branch.
  __device__ __forceinline__ void scale_acc(int nt, float alpha) {
#pragma unroll
    for (int dt = 0; dt < DM::DT32; ++dt) oacc[dt][nt] = oacc[dt][nt] * alpha;
    if constexpr (DM::PV16) {
      // the 16x16 accumulator holds query (lane & 15) + 16 h in every lane;
      // alpha is per query in lane (query) of the 32x32 layout
      oacc16[nt][0] = oacc16[nt][0] * __shfl(alpha, q16);
      oacc16[nt][1] = oacc16[nt][1] * __shfl(alpha, q16 + 16);
    }
  }

  // Probabilities of query tile nt of a settled unit, as the bf16 B operand
  // of O^T = V^T P^T.
  __device__ __forceinline__ void probs(f32x16 &s, bf16x8 (&pf)[2][NT], int nt) {
    if constexpr (FOLD) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(PRE ? s[r] : s[r] * c);
    } else {
      const float mc = m[nt] * c;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -mc));
    }
    if constexpr (!DM::ONES) {
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc += s[r];
      lsum[nt] += acc;
    }
    pf[0][nt] = pack_p(s, 0);
    pf[1][nt] = pack_p(s, 8);
  }

  // O^T += V^T P^T for one unit whose V rows start at Vs.
  __device__ __forceinline__ void pv(const bf16x8 (&pf)[2][NT], const u16 *__restrict__ Vs) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const u16 *vb = Vs + ks2 * 16 * D + v_off;
#pragma unroll
      for (int dt = 0; dt < DM::DT32; ++dt) {
        uint4 u = tr_read_pair<D>(DM::SWZ ? Vs + ks2 * 16 * D + voff[dt] : vb + dt * 32);
        if (!DM::PV16 && DM::DV != D && dt == DM::DT - 1 && !vkeep) u = make_uint4(vconst, vconst, vconst, vconst);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks2][nt], oacc[dt][nt], 0, 0, 0);
      }
    }
    if constexpr (DM::PV16) {
      // The 16x16x32 B operand wants, per 16-lane row, 8 keys of 16 queries.
      // v_permlane16_swap of the two 16-key halves of P^T regroups the score
      // layout into exactly that: queries 0..15 (first result) and 16..31
      // (second) of the tile, key groups {0-3,8-11}, {16-19,24-27},
      // {4-7,12-15}, {20-23,28-31} by row; V^T is read in the same order.
      uint4 u = tr_read_pair<D>(Vs + v_off16);
      if (!vkeep) u = make_uint4(vconst, vconst, vconst, vconst);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint4 x0 = __builtin_bit_cast(uint4, pf[0][nt]), x1 = __builtin_bit_cast(uint4, pf[1][nt]);
        const auto w0 = __builtin_amdgcn_permlane16_swap(x0.x, x1.x, false, false);
        const auto w1 = __builtin_amdgcn_permlane16_swap(x0.y, x1.y, false, false);
        const auto w2 = __builtin_amdgcn_permlane16_swap(x0.z, x1.z, false, false);
        const auto w3 = __builtin_amdgcn_permlane16_swap(x0.w, x1.w, false, false);
        const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w1[0], w2[0], w3[0]));
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w0[1], w1[1], w2[1], w3[1]));
        oacc16[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pa, oacc16[nt][0], 0, 0, 0);
        oacc16[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, oacc16[nt][1], 0, 0, 0);
      }
    }
  }

  // One pipeline step: unit u (settled, scores in slot CUR of sb, V rows at
  // Vs) and, when NEXT, unit un (K rows at Kn), whose scores go to the other
  // slot.  Steps alternate slots, so no scores are ever copied.  Phase nt
  // pairs the S^T MFMAs of query tile nt of unit un with the exponentials of
  // the same tile of unit u, so only one tile of each is in flight at once;
  // the last phase pairs O^T += V^T P^T with the rescale test.  With PREF the
  // K operand of unit up is read into kf after P.V, one step before the
  // S^T MFMAs that use it, so that read's latency is off the critical path.
  template <bool NEXT, int CUR, bool PREF>
  __device__ __forceinline__ void step(f32x16 (&sb)[2][NT], bf16x8 (&kf)[DM::KS], const u16 *__restrict__ Vs, int un,
                                       bool mask_next, const u16 *__restrict__ Kp, int up) {
    bf16x8 pf[2][NT];
    // Raised issue priority while this wave interleaves S^T MFMAs with
    // exponentials: when the other wave of the SIMD is in its P.V phase
    // (MFMA-heavy, waiting on V^T reads), this one's vector work goes first
    // and fills the matrix pipe's shadow.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (NEXT) qk(sb[CUR ^ 1][nt], kf, nt);
      probs(sb[CUR][nt], pf, nt);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    pv(pf, Vs);
    if constexpr (PREF) kfrag(kf, Kp, up);
    if constexpr (NEXT) {
      if constexpr (!FOLD)
        if (mask_next) mask(sb[CUR ^ 1], un);
      float lm[NT];
      if (needs_rescale(sb[CUR ^ 1], lm)) rescale(sb[CUR ^ 1], lm, false);
    }
  }
};

template <int D, int NT, bool PRE>
__global__ void __launch_bounds__(64 * kLongWaves, 8 / kLongWaves) attn_long_kernel(AttnArgs a, uint32_t nqb,
                                                                                  uint32_t nblocks) {
  typedef LongCfg<D, NT> C;
  typedef Dims<D> DM;
  typedef LongWave<D, NT, PRE> W;
  __shared__ __attribute__((aligned(16))) u16 lds[C::NSTAGE * C::STAGE];

  const uint32_t tile = xcd_remap(blockIdx.x, nblocks);
  const uint32_t qb = tile % nqb;
  const uint32_t seq = tile / nqb;
  const int h = (int)(seq % (uint32_t)a.H);
  const int64_t outer = seq / (uint32_t)a.H;
  const int64_t rs = (int64_t)a.H * D;                  // row stride (elements)
  const int64_t qbase = outer * a.L * rs + (int64_t)h * D;
  const int64_t kvbase = outer * a.Lk * rs + (int64_t)h * D;
  const u16 *qp = a.q + qbase, *kp = a.k + kvbase, *vp = a.v + kvbase;
  u16 *op = a.o + qbase;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int L = a.L, Lk = a.Lk;

  W w;
  w.c = a.c;
  w.thr = PRE ? kRescale : kRescale / a.c;
  w.nv = min(Lk, a.n_valid);
  w.l32 = lane & 31;
  w.g = lane >> 5;
  w.q16 = lane & 15;

  // Slack after every tile is zero, so operand reads that run past the last
  // row multiply finite values by the zero padding of Q (K) or get replaced (V).
  for (int i = t; i < 2 * C::NSTAGE * C::SLACK; i += 64 * C::WAVES)
    lds[(i / C::SLACK) * C::REGION + C::TILE + i % C::SLACK] = 0;

  // Q operand fragments, held for the whole key loop (FOLD: PRE multiplies
  // by c, exactly; the -m and -1 terms in dims 72 and 73, m starts at 0).
  const int q0 = qb * C::QB + wave * C::QW;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int qi = q0 + nt * 32 + w.l32;
#pragma unroll
    for (int ks = 0; ks < DM::KS; ++ks) {
      const int dd = ks * 16 + w.g * 8;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qi < L && dd < D) u = *reinterpret_cast<const uint4 *>(qp + (int64_t)qi * rs + dd);
      if constexpr (W::FOLD && PRE) {
        uint32_t x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[j] = pack_bf16x2(__uint_as_float(x[j] << 16) * w.c, __uint_as_float(x[j] & 0xFFFF0000u) * w.c);
        u = make_uint4(x[0], x[1], x[2], x[3]);
      }
      if constexpr (W::FOLD)
        if (ks == DM::KS - 1 && w.g) u.x = kBf16NegOne << 16;
      w.qf[nt][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
#pragma unroll
  for (int i = 0; i < DM::DT32; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.oacc[i][j][r] = 0.f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) w.oacc16[j][h][r] = 0.f;
    w.m[j] = W::FOLD ? 0.f : -INFINITY;
    w.lsum[j] = 0.f;
  }

  // V^T operand via LDS transpose reads (ds_read_b64_tr_b16): in each 16-lane
  // group, lane i receives element (i & 3) of the 8 bytes addressed by lanes
  // 4j + (i >> 2), j = 0..3.  Lane 4j + q of group G addresses V[key0 + j][dg + 4q]
  // with dg = 32 dt + 16 (G & 1), so lane i of the group gets 4 consecutive keys
  // of dimension dg + i: exactly the A-operand layout (row = lane % 32).
  const int grp = lane >> 4, gi = lane & 15;
  w.v_off = (gi >> 2) * D + 16 * (grp & 1) + 4 * (gi & 3) + 4 * (grp >> 1) * D;
  if constexpr (DM::SWZ) {
    // Swizzled rows (see Dims): the XORs are per lane and per step, so the
    // offsets are computed once.  A lane's V rows are (gi >> 2) + 4 (grp >> 1)
    // plus multiples of 8, which all share one swizzle.
    const int vsw = DM::vswz((gi >> 2) + 4 * (grp >> 1)) / 4;
#pragma unroll
    for (int ks = 0; ks < DM::KS; ++ks) w.koff[ks] = w.l32 * D + ((ks * 2 + w.g) ^ DM::kswz(w.l32)) * 8;
#pragma unroll
    for (int dt = 0; dt < DM::DT32; ++dt) w.voff[dt] = w.v_off + (dt ^ vsw) * 32;
  }
  // rows past D in the last P.V tile: the ones row, then zeros
  const int dlast = 32 * (DM::DT - 1) + w.l32;
  w.vkeep = dlast < D;
  w.vconst = (DM::ONES && dlast == D) ? 0x3F803F80u : 0u;
  if constexpr (DM::PV16) {
    // 16-row tile: group G of 16 lanes holds keys {0,16,4,20}[G] + {0..3, 8..11};
    // lane 4j + q of the group addresses V[key0 + j][d16 + 4q], d16 = first row of the tile.
    constexpr int d16 = D - D % 32;
    w.v_off16 = ((grp & 1) * 16 + (grp >> 1) * 4 + (gi >> 2)) * D + d16 + 4 * (gi & 3);
    w.vkeep = gi < D % 32;
    w.vconst = (gi == D % 32) ? 0x3F803F80u : 0u;
  }

  // Units of 32 keys up to n_valid (later keys carry no weight), KB / 32 per
  // LDS tile.  Tiles rotate through NSTAGE stages: tile j+1 is in flight
  // while tile j is read, and tile j+2 is issued into tile j-1's stage once
  // the barrier that opens tile j has passed.
  constexpr int UPT = C::KB / 32;   // 32-key units per tile
  const int nu = (w.nv + 31) / 32;
  const int ntl = (nu + UPT - 1) / UPT;
  const bool partial = (w.nv & 31) != 0;
  LongDma<D> dma;
  dma.init(rs, lane, wave);
  if (ntl == 0) return;   // whole workgroup: n_valid is uniform (the host never launches with none)
  dma.issue(lds, 0, kp, vp, rs, Lk, lane, wave);
  wait_vmem();
  __syncthreads();
  if (ntl > 1) dma.issue(lds + C::STAGE, C::KB, kp, vp, rs, Lk, lane, wave);

  // A wave whose queries all lie past L (the last query block of a sequence
  // whose length is not a multiple of the block) computes nothing: it only
  // issues its share of every tile's loads and meets the same barriers as
  // the key loop below, then leaves.
  if (__builtin_amdgcn_readfirstlane(q0) >= L) {
    for (int p = 0; 2 * p + 2 < nu; ++p) {
      const int u = 2 * p;
      if (u % UPT == 0) {
        const int kt = u / UPT;
        wait_vmem();
        __syncthreads();
        if (kt + 2 < ntl) dma.issue(lds + ((kt + 2) % C::NSTAGE) * C::STAGE, (kt + 2) * C::KB, kp, vp, rs, Lk, lane, wave);
      }
    }
    return;
  }

  // K (and, + REGION, V) rows of unit u
  auto unit_rows = [&](int u) { return lds + ((u / UPT) % C::NSTAGE) * C::STAGE + (u % UPT) * 32 * D; };
  f32x16 sb[2][NT];
  bf16x8 kf[DM::KS];
  {
    w.kfrag(kf, lds, 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) w.qk(sb[0][nt], kf, nt);
    if constexpr (!W::FOLD)
      if (partial && nu == 1) w.mask(sb[0], 0);
    float lm[NT];
    w.needs_rescale(sb[0], lm);
    w.rescale(sb[0], lm, true);
    if (nu > 1) w.kfrag(kf, lds + 32 * D, 1);
  }

  // Units in pairs; one barrier per tile, at the top of its first pair:
  // tile kt+1 has landed (K is read one unit ahead, possibly from it) and
  // tile kt-1's stage is free for tile kt+2.
  int p = 0;
  for (; 2 * p + 2 < nu; ++p) {
    const int u = 2 * p;
    if (u % UPT == 0) {
      const int kt = u / UPT;
      wait_vmem();
      __syncthreads();
      if (kt + 2 < ntl) dma.issue(lds + ((kt + 2) % C::NSTAGE) * C::STAGE, (kt + 2) * C::KB, kp, vp, rs, Lk, lane, wave);
    }
    w.template step<true, 0, true>(sb, kf, unit_rows(u) + C::REGION, u + 1, partial && u + 1 == nu - 1,
                                   unit_rows(u + 2), u + 2);
    w.template step<true, 1, true>(sb, kf, unit_rows(u + 1) + C::REGION, u + 2, partial && u + 2 == nu - 1,
                                   unit_rows(u + 3), u + 3);
  }
  {
    // the last one or two units: their tile has landed (waited at the previous
    // tile's barrier, or before the loop), and nothing is prefetched
    const int u = 2 * p;
    if (u + 2 == nu) {
      w.template step<true, 0, false>(sb, kf, unit_rows(u) + C::REGION, u + 1, partial, nullptr, 0);
      w.template step<false, 1, false>(sb, kf, unit_rows(u + 1) + C::REGION, 0, false, nullptr, 0);
    } else {
      w.template step<false, 0, false>(sb, kf, unit_rows(u) + C::REGION, 0, false, nullptr, 0);
    }
  }

  // normalise and store
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l;
    float lh[2] = {0.f, 0.f};   // PV16: denominators of the two query halves (ones row = row D % 32)
    if constexpr (DM::PV16) {
      static_assert(DM::PV16 == false || (D % 32) % 4 == 0, "ones row starts a 4-row lane group");
      lh[0] = __shfl(w.oacc16[nt][0][0], 16 * ((D % 32) / 4) + (lane & 15));
      lh[1] = __shfl(w.oacc16[nt][1][0], 16 * ((D % 32) / 4) + (lane & 15));
      l = w.l32 < 16 ? lh[0] : lh[1];
    } else if constexpr (DM::ONES) {
      l = __shfl(w.oacc[DM::ONES_DT][nt][DM::ONES_R], w.l32);   // held by lane half 0
    } else {
      l = w.lsum[nt] + __shfl_xor(w.lsum[nt], 32);
    }
    const int qi = q0 + nt * 32 + w.l32;
    // Output = fa * (accumulated row) + fp * (this result); without a.acc,
    // fa = 0 and fp = 1.  The merge weights are exp(lse_part - lse_union).
    float fa = 0.f, fp = 1.f;
    if (a.lse) {
      // sum_j exp(scale s_j) = 2^M * l, M = the running max in scaled log2 units
      const float M = (W::FOLD && PRE) ? w.m[nt] : w.m[nt] * w.c;
      float lse = (M + log2f(l)) * 0.69314718055994531f;
      const int64_t li = (outer * a.H + h) * (int64_t)L + qi;
      if (a.acc) {
        const float la = qi < L ? a.lse[li] : -INFINITY;   // read by both lane halves before g == 0 writes
        const float mm = fmaxf(la, lse);
        const float wa = expf(la - mm), wp = expf(lse - mm);
        const float tot = wa + wp;
        fa = wa / tot;
        fp = wp / tot;
        lse = mm + logf(tot);
      }
      if (qi < L && w.g == 0) a.lse[li] = lse;
    }
    const float inv = fp / l;
    if (qi < L) {
      u16 *orow = op + (int64_t)qi * rs;
#pragma unroll
      for (int dt = 0; dt < DM::DT32; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int dd = dt * 32 + rb * 8 + w.g * 4;
          if (dd + 4 <= D) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = w.oacc[dt][nt][rb * 4 + j] * inv;
            if (a.acc && fa > 0.f) {   // an empty accumulator contributes nothing, whatever its row holds
              const uint2 pv = *reinterpret_cast<const uint2 *>(orow + dd);
              x[0] = fmaf(fa, __uint_as_float(pv.x << 16), x[0]);
              x[1] = fmaf(fa, __uint_as_float(pv.x & 0xFFFF0000u), x[1]);
              x[2] = fmaf(fa, __uint_as_float(pv.y << 16), x[2]);
              x[3] = fmaf(fa, __uint_as_float(pv.y & 0xFFFF0000u), x[3]);
            }
            uint2 o;
            o.x = pack_bf16x2(x[0], x[1]);
            o.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2 *>(orow + dd) = o;
          }
        }
    }
    if constexpr (DM::PV16) {
      // 16x16 accumulator: lane l holds rows 4 (l / 16) .. +3 for query (l & 15) of each half
      // merge weights of query (lane & 15) + 16 h live in the lane of the 32x32 layout that holds it
      float fa16[2], fp16[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        fa16[h] = __shfl(fa, h * 16 + (lane & 15));
        fp16[h] = __shfl(fp, h * 16 + (lane & 15));
      }
      const int dd = D - D % 32 + 4 * (lane >> 4);
      if (dd + 4 <= D) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qh = q0 + nt * 32 + h * 16 + (lane & 15);
          const float fah = fa16[h], fph = fp16[h];
          if (qh < L) {
            const float ih = fph / lh[h];
            u16 *orow = op + (int64_t)qh * rs + dd;
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = w.oacc16[nt][h][j] * ih;
            if (a.acc && fah > 0.f) {
              const uint2 pv = *reinterpret_cast<const uint2 *>(orow);
              x[0] = fmaf(fah, __uint_as_float(pv.x << 16), x[0]);
              x[1] = fmaf(fah, __uint_as_float(pv.x & 0xFFFF0000u), x[1]);
              x[2] = fmaf(fah, __uint_as_float(pv.y << 16), x[2]);
              x[3] = fmaf(fah, __uint_as_float(pv.y & 0xFFFF0000u), x[3]);
            }
            uint2 o;
            o.x = pack_bf16x2(x[0], x[1]);
            o.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2 *>(orow) = o;
          }
        }
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
  static constexpr int KL = 32 * NT;                        // padded keys = queries
  static constexpr int V_BLOCKS = (KL * DM::CH + 63) / 64;  // 1 KB direct-to-LDS loads of V
  static constexpr int V_WAVE = V_BLOCKS * 512 + 64;        // u16 per wave: V rows, then transpose-read slack
  // u16 of LDS per workgroup.  With two query tiles it is padded to 54 KB so
  // that at most two workgroups (two waves per SIMD) share a CU: timed at
  // 1080p, three waves per SIMD ran 4-13% slower and one wave 10% slower (more
  // scattered Q/K row loads in flight than the memory system serves well).
  static constexpr int LDS = NT == 2 && 4 * V_WAVE < 27648 ? 27648 : 4 * V_WAVE;
};

// At least two waves per SIMD: keeps the compiler from splitting the registers
// into AGPR accumulators plus VGPRs, which would cost occupancy.
template <int D, int NT>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256), amdgpu_waves_per_eu(2)))
attn_short_kernel(AttnArgs a, uint32_t nblocks) {
  typedef ShortCfg<D, NT> C;
  typedef Dims<D> DM;
  __shared__ __attribute__((aligned(16))) u16 lds[C::LDS];

  const uint32_t hg_n = (uint32_t)(a.H + 3) / 4;
  const uint32_t blk = xcd_remap(blockIdx.x, nblocks);
  const int64_t outer = blk / hg_n;
  const int h0 = (int)(blk % hg_n) * 4, h1 = min(a.H, h0 + 4);
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int L = a.L, nv = min(a.n_valid, a.L);
  const int64_t rs = (int64_t)a.H * D;
  u16 *Vs = lds + wave * C::V_WAVE;

  // V^T operand by transpose reads of V stored [key][d] (the layout of the
  // long kernel): lane 4j + q of 16-lane group G addresses V[key0 + j][dg + 4q].
  const int grp = lane >> 4, gi = lane & 15;
  const int v_off = (gi >> 2) * D + 16 * (grp & 1) + 4 * (gi & 3) + 4 * (grp >> 1) * D;
  const int dlast = 32 * (DM::DT - 1) + l32;   // O^T row of this lane in the last tile
  const bool vkeep = dlast < D;
  const uint32_t vconst = (DM::ONES && dlast == D) ? 0x3F803F80u : 0u;

  // Blocks of V rows wholly past L are never loaded: they are zeroed once, so
  // the P.V products of those (masked) keys are 0 * 0.
  const int vblk = min(C::V_BLOCKS, (L * DM::CH + 63) / 64);   // blocks loaded per head
  for (int i = vblk * 64 + lane; i < C::V_BLOCKS * 64; i += 64) reinterpret_cast<uint4 *>(Vs)[i] = make_uint4(0, 0, 0, 0);

  for (int h = h0 + wave; h < h1; h += 4) {
    const int64_t base = outer * L * rs + (int64_t)h * D;
    const u16 *qp = a.q + base, *kp = a.k + base, *vp = a.v + base;
    u16 *op = a.o + base;

    // Q and K go straight into operand registers; all loads are issued before
    // any is used.  Rows past L re-read row L-1 (those queries are not stored,
    // those keys are masked); chunks past d re-read the last chunk and are
    // zeroed below.
    uint4 qraw[NT][DM::KS], kraw[NT][DM::KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t row = min(nt * 32 + l32, L - 1);
#pragma unroll
      for (int ks = 0; ks < DM::KS; ++ks) {
        const int dd = min(ks * 16 + g * 8, D - 8);
        qraw[nt][ks] = *reinterpret_cast<const uint4 *>(qp + row * rs + dd);
        kraw[nt][ks] = *reinterpret_cast<const uint4 *>(kp + row * rs + dd);
      }
    }
    // V rows go global -> LDS directly: 16-byte chunk n of the packed
    // [key][d] tile is chunk n % (d/8) of key n / (d/8); keys past L re-read
    // row L-1 (their probabilities are 0) and chunks past the tile land in
    // the slack.
#pragma unroll
    for (int b = 0; b < C::V_BLOCKS; ++b) {
      if (b >= vblk) break;
      const int n = 64 * b + lane;
      const int key = min(n / DM::CH, L - 1), ch = n % DM::CH;
      __builtin_amdgcn_global_load_lds(vp + (int64_t)key * rs + ch * 8,
                                       (__attribute__((address_space(3))) void *)(Vs + b * 512), 16, 0, 0);
    }
    bf16x8 qf[NT][DM::KS], kf[NT][DM::KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int ks = 0; ks < DM::KS; ++ks) {
        const bool pad = ks * 16 + g * 8 >= D;
        qf[nt][ks] = __builtin_bit_cast(bf16x8, pad ? make_uint4(0, 0, 0, 0) : qraw[nt][ks]);
        kf[nt][ks] = __builtin_bit_cast(bf16x8, pad ? make_uint4(0, 0, 0, 0) : kraw[nt][ks]);
      }

    // One query tile at a time: S^T of its key tiles, softmax, bf16 P^T.
    bf16x8 pf[NT][NT][2];   // [query tile][key tile][16-key half]
    float lsum[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x16 s[NT];   // keys of tile mt x the queries of tile nt
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DM::KS; ++ks) s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][ks], qf[nt][ks], s[mt], 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (mt * 32 + acc_row(r, g) < nv) ? s[mt][r] : -INFINITY;
          s[mt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_across_halves(mx);
      const float mc = mx * a.c;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][r] = __builtin_amdgcn_exp2f(fmaf(s[mt][r], a.c, -mc));
      if constexpr (!DM::ONES) {
        float acc = 0.f;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += s[mt][r];
        lsum[nt] = acc + __shfl_xor(acc, 32);
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        pf[nt][mt][0] = pack_p(s[mt], 0);
        pf[nt][mt][1] = pack_p(s[mt], 8);
      }
    }
    // V has landed in this wave's slice
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if constexpr (D % 64 != 0) {
      // d = 72 (rows of 144 bytes, 36 banks apart): O^T of both query tiles, then
      // the normalised rows through this wave's V slice (free once the last P.V
      // MFMA has read it), stored 16 bytes per lane along whole rows instead of
      // 8-byte pieces of 32 rows.  For d = 64 or 128 the rows would all start on
      // the same LDS banks; those store from the accumulators directly.
      f32x16 oacc[NT][DM::DT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nt][dt][r] = 0.f;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            const u16 *vb = Vs + (mt * 32 + ks2 * 16) * D + v_off;
#pragma unroll
            for (int dt = 0; dt < DM::DT; ++dt) {
              uint4 u = tr_read_pair<D>(vb + dt * 32);
              if (DM::DV != D && dt == DM::DT - 1 && !vkeep) u = make_uint4(vconst, vconst, vconst, vconst);
              oacc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[nt][mt][ks2],
                                                                     oacc[nt][dt], 0, 0, 0);
            }
          }
      }
      float inv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float l;
        if constexpr (DM::ONES) {
          l = __shfl(oacc[nt][DM::ONES_DT][DM::ONES_R], l32);
        } else {
          l = lsum[nt];
        }
        inv[nt] = 1.0f / l;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int dd = dt * 32 + rb * 8 + g * 4;
            if (dd + 4 <= D) {
              uint2 w;
              w.x = pack_bf16x2(oacc[nt][dt][rb * 4 + 0] * inv[nt], oacc[nt][dt][rb * 4 + 1] * inv[nt]);
              w.y = pack_bf16x2(oacc[nt][dt][rb * 4 + 2] * inv[nt], oacc[nt][dt][rb * 4 + 3] * inv[nt]);
              *reinterpret_cast<uint2 *>(Vs + (nt * 32 + l32) * D + dd) = w;
            }
          }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int kRowChunks = DM::CH;                        // 16-byte chunks per row of O
      constexpr int kIt = (C::KL * kRowChunks + 63) / 64;
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int c = it * 64 + lane;
        const int row = c / kRowChunks, ch = c - row * kRowChunks;
        if (row < L) {
          const uint4 w = *reinterpret_cast<const uint4 *>(Vs + row * D + ch * 8);
          *reinterpret_cast<uint4 *>(op + (int64_t)row * rs + ch * 8) = w;
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x16 oacc[DM::DT];
#pragma unroll
        for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            const u16 *vb = Vs + (mt * 32 + ks2 * 16) * D + v_off;
#pragma unroll
            for (int dt = 0; dt < DM::DT; ++dt) {
              uint4 u = tr_read_pair<D>(vb + dt * 32);
              if (DM::DV != D && dt == DM::DT - 1 && !vkeep) u = make_uint4(vconst, vconst, vconst, vconst);
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[nt][mt][ks2], oacc[dt],
                                                                 0, 0, 0);
            }
          }
        float l;
        if constexpr (DM::ONES) {
          l = __shfl(oacc[DM::ONES_DT][DM::ONES_R], l32);
        } else {
          l = lsum[nt];
        }
        const float inv = 1.0f / l;
        const int qi = nt * 32 + l32;
        if (qi < L) {
          u16 *orow = op + (int64_t)qi * rs;
#pragma unroll
          for (int dt = 0; dt < DM::DT; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
              const int dd = dt * 32 + rb * 8 + g * 4;
              if (dd + 4 <= D) {
                uint2 w;
                w.x = pack_bf16x2(oacc[dt][rb * 4 + 0] * inv, oacc[dt][rb * 4 + 1] * inv);
                w.y = pack_bf16x2(oacc[dt][rb * 4 + 2] * inv, oacc[dt][rb * 4 + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + dd) = w;
              }
            }
        }
      }
    }
    // the next head overwrites V: all lanes' reads of this head are done
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int D, int NT, bool PRE = false>
st_status launch_long(const AttnArgs &a, hipStream_t s) {
  typedef LongCfg<D, NT> C;
  const int64_t nqb = (a.L + C::QB - 1) / C::QB;
  const int64_t nb = nqb * a.outer * a.H;
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_long_kernel<D, NT, PRE>), dim3((uint32_t)nb), dim3(64 * C::WAVES), 0, s, a, (uint32_t)nqb,
                     (uint32_t)nb);
  return launch_status();
}

template <int D, int NT>
st_status launch_short(const AttnArgs &a, hipStream_t s) {
  const int64_t nb = a.outer * ((a.H + 3) / 4);
  if (nb >= (1ll << 31)) return ST_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_short_kernel<D, NT>), dim3((uint32_t)nb), dim3(256), 0, s, a, (uint32_t)nb);
  return launch_status();
}

// c is a power of two: multiplying bf16 values by it is exact (no overflow at attention scales).
bool pow2(float c) {
  int e;
  return c > 0.f && frexpf(c, &e) == 0.5f && e > -100 && e < 100;
}

AttnArgs make_args(const void *q, const void *k, const void *v, int64_t outer, int L, int Lk, int n_valid, int H,
                   float scale, void *out, float *lse, bool acc = false) {
  AttnArgs a;
  a.q = static_cast<const u16 *>(q);
  a.k = static_cast<const u16 *>(k);
  a.v = static_cast<const u16 *>(v);
  a.o = static_cast<u16 *>(out);
  a.lse = lse;
  a.acc = acc ? 1 : 0;
  a.outer = outer;
  a.L = L;
  a.Lk = Lk;
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
  return launch_attn_chunk_bf16(q, k, v, outer, L, L, n_valid, H, d, scale, out, nullptr, s);
}

st_status launch_attn_chunk_bf16(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk,
                                 int n_valid, int H, int d, float scale, void *out, float *lse, hipStream_t s,
                                 bool accumulate) {
  if (outer == 0 || Lq == 0) return ST_OK;
  const AttnArgs a = make_args(q, k, v, outer, Lq, Lk, n_valid, H, scale, out, lse, accumulate);
  switch (d) {
    case 72: return pow2(a.c) ? launch_long<72, 2, true>(a, s) : launch_long<72, 2, false>(a, s);
    case 64: return launch_long<64, 2>(a, s);
    case 128: return launch_long<128, 1>(a, s);
    default: return ST_EUNSUPPORTED;
  }
}

st_status launch_attn_short_bf16(const void *q, const void *k, const void *v, int64_t outer, int L, int n_valid,
                                 int H, int d, float scale, void *out, hipStream_t s) {
  if (outer == 0 || L == 0) return ST_OK;
  const AttnArgs a = make_args(q, k, v, outer, L, L, n_valid, H, scale, out, nullptr);
  if (d == 72) return L <= 32 ? launch_short<72, 1>(a, s) : launch_short<72, 2>(a, s);
  if (d == 64) return L <= 32 ? launch_short<64, 1>(a, s) : launch_short<64, 2>(a, s);
  return ST_EUNSUPPORTED;
}

}  // namespace st
