// Internal declarations shared by the HIP sources of libst.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/st.h"

namespace st {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// blockIdx.x -> logical tile id such that consecutive logical ids run on the
// same XCD.  The dispatcher hands workgroup i to XCD i % 8; tiles that share
// data (the N tiles of one GEMM row block, the query blocks of one attention
// sequence) then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = nblocks / kXcd;          // full round-robin rows
  const uint32_t full = per * kXcd;
  if (bid >= full) return bid;                  // ragged tail keeps its id
  return (bid % kXcd) * per + bid / kXcd;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels are compiled for gfx950 only.  Every call that launches work
// checks the current device after its argument checks (cached per device) and
// refuses any other architecture with ST_EUNSUPPORTED rather than failing at
// the launch.
inline st_status device_ok() {
  static std::atomic<int> arch[64];   // 0 not looked up, 1 gfx950, 2 another architecture
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ST_ELAUNCH;
  int a = dev < 64 ? arch[dev].load(std::memory_order_relaxed) : 0;
  if (a == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return ST_ELAUNCH;
    const char *n = p.gcnArchName;   // e.g. "gfx950:sramecc+:xnack-"
    a = (strncmp(n, "gfx950", 6) == 0 && (n[6] == '\0' || n[6] == ':')) ? 1 : 2;
    if (dev < 64) arch[dev].store(a, std::memory_order_relaxed);
  }
  return a == 1 ? ST_OK : ST_EUNSUPPORTED;
}

inline st_status launch_status() {
  return hipGetLastError() == hipSuccess ? ST_OK : ST_ELAUNCH;
}

// Launchers (each validates nothing; the C ABI layer has done it).
st_status launch_rope_table(int d, int kind, double base, int n_pos, float *table, hipStream_t s);

st_status launch_relayout(const void *src, const int64_t *src_str, void *dst, const int64_t *dst_str,
                          const int64_t *dims, int ndim, int elem_bytes, hipStream_t s);

struct RopeArgs {
  int kind;             // st_rope_kind
  int npos;
  const float *table;   // [npos][pairs][2]
  int64_t period, offset;
  int grid_w;
  const int32_t *pos = nullptr;   // [rows][2] positions ((t, 0) or (h, w)); null: periodic rule
};

// Row map of a linear layer's input or output rows: row r, read as the
// digits (r0, r1, r2, r3) of the mixed radix [*, n1, n2, n3] (r3 fastest),
// goes to row base + r0*s0 + r1*s1 + r2*s2 + r3*s3.  n1 = 0 is the identity.
struct RowMap {
  int64_t n1 = 0, n2 = 1, n3 = 1;
  int64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0, base = 0;
};
__host__ __device__ inline int64_t map_row(int64_t r, const RowMap &m) {
  if (m.n1 == 0) return r;
  const int64_t q3 = r / m.n3, d3 = r - q3 * m.n3;
  const int64_t q2 = q3 / m.n2, d2 = q3 - q2 * m.n2;
  const int64_t d0 = q2 / m.n1, d1 = q2 - d0 * m.n1;
  return m.base + d0 * m.s0 + d1 * m.s1 + d2 * m.s2 + d3 * m.s3;
}
// Rows in [outer, n1, n2] order go to [outer, n2, n1].
inline RowMap row_swap(int64_t n1, int64_t n2) {
  RowMap m;
  m.n1 = n1;
  m.n2 = n2;
  m.s0 = n1 * n2;
  m.s1 = 1;
  m.s2 = n1;
  return m;
}

// q is stored multiplied by q_scale (its RMSNorm gain times q_scale).
st_status launch_qkv_bf16(const void *x, int64_t rows, int c_in, const void *w, const float *g_q,
                          const float *g_k, float eps, float q_scale, const RopeArgs &rope, int H, int d, void *q,
                          void *k, void *v, hipStream_t s, RowMap xmap = {});
st_status launch_linear_bf16(const void *a, int64_t rows, int k_in, const void *w, int n_out, void *y,
                             hipStream_t s, RowMap ymap = {});
st_status launch_qkv_f32(const float *x, int64_t rows, int c_in, const float *w, const float *g_q,
                         const float *g_k, float eps, float q_scale, const RopeArgs &rope, int H, int d, float *q,
                         float *k, float *v, hipStream_t s);
st_status launch_linear_f32(const float *a, int64_t rows, int k_in, const float *w, int n_out, float *y,
                            hipStream_t s, RowMap ymap = {});

// Attention over the middle axis L of [outer, L, H, d] tensors, keys j >= n_valid masked.
st_status launch_attn_bf16(const void *q, const void *k, const void *v, int64_t outer, int L, int n_valid,
                           int H, int d, float scale, void *out, hipStream_t s);
st_status launch_attn_short_bf16(const void *q, const void *k, const void *v, int64_t outer, int L,
                                 int n_valid, int H, int d, float scale, void *out, hipStream_t s);
st_status launch_attn_f32(const float *q, const float *k, const float *v, int64_t outer, int L, int n_valid,
                          int H, int d, float scale, float *out, hipStream_t s);
// Attention of Lq queries over a chunk of Lk keys (keys j >= n_valid masked, n_valid >= 1), optionally
// writing the natural log-sum-exp of the scaled scores per query to lse [outer, H, Lq].  With
// accumulate, out and lse hold a partial result over other keys (lse -inf: none) and receive the
// merge of it with this chunk's result.
st_status launch_attn_chunk_bf16(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk,
                                 int n_valid, int H, int d, float scale, void *out, float *lse, hipStream_t s,
                                 bool accumulate = false);
st_status launch_attn_chunk_f32(const float *q, const float *k, const float *v, int64_t outer, int Lq, int Lk,
                                int n_valid, int H, int d, float scale, float *out, float *lse, hipStream_t s,
                                bool accumulate = false);
// o = 0 and lse = -inf for a chunk without valid keys; elem_bytes 2 or 4.
st_status launch_attn_empty(void *o, float *lse, int64_t outer, int L, int H, int d, int elem_bytes, hipStream_t s);
// Merge of two chunk results over [outer, L, H, d] with [outer, H, L] log-sum-exps (in place allowed).
st_status launch_attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t outer,
                            int L, int H, int d, int elem_bytes, void *o, float *lse, hipStream_t s);

// V-Major change detection: mask[v] = sum_j |v_new - v_cache| > threshold per row of d elements
// (d * elem_bytes a multiple of 16, at most 512 bytes); active rows compacted into idx (order
// unspecified, may be null), their count into *n_active; update != 0 refreshes the cache rows.
st_status launch_v_change(const void *v_new, void *v_cache, int64_t nvec, int d, int elem_bytes, float threshold,
                          uint8_t *mask, int32_t *idx, int64_t *n_active, int update, hipStream_t s);

bool attn_bf16_supported(int d);
bool attn_short_supported(int L, int d);

}  // namespace st
