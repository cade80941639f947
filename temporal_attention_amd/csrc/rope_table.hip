// Cosine/sine table of the rotary position encoding applied to Q and K
// (CoCoDiff page, "V-First compute scheduling").  Pair i of an axis segment
// of length m rotates by theta = p * base^(-2i/m); the angle and its cosine
// and sine are evaluated in double precision, then rounded to fp32, so the
// projection kernels only do table lookups.
#include "st_internal.h"

namespace st {
namespace {

__global__ void rope_table_kernel(int pairs, int m, double log2_base, int n_pos, float *table) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pos * pairs) return;
  const int p = i / pairs, pair = i % pairs;
  const double inv_freq = exp2(-2.0 * (double)pair / (double)m * log2_base);
  const double theta = (double)p * inv_freq;
  double sn, cs;
  sincos(theta, &sn, &cs);
  table[2 * i] = (float)cs;
  table[2 * i + 1] = (float)sn;
}

}  // namespace

st_status launch_rope_table(int d, int kind, double base, int n_pos, float *table, hipStream_t s) {
  const int m = kind == ST_ROPE_2D ? d / 2 : d;
  const int pairs = m / 2;
  const int n = n_pos * pairs;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, pairs, m, log2(base), n_pos,
                     table);
  return launch_status();
}

}  // namespace st
