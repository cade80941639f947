// Local pack and unpack around the P-way all-to-all between the two shardings
// of the layer pair (ScaleFusion review, "Technical architecture": the layer
// table gives each rank a patch block [B, T, S/P, C] for the temporal layer
// and a frame block [B, T/P, S, C] for the spatial layer, and an all-to-all
// converts between them; the algorithm pseudocode in "Core innovations"
// places it between the layers).
//
// A collective moves one contiguous chunk per peer, so each direction is
// pack -> all-to-all -> unpack.  The chunk layout on the wire is
// [P, B, T/P, S/P, C] in both directions, chunk q contiguous:
//   S2T  pack:   x [B, T, S/P, C]    -> send[q] = frames q*T/P.. of this rank's patches
//        unpack: recv[r] = rank r's patch block of this rank's frames -> y [B, T/P, S, C]
//   T2S  pack:   x [B, T/P, S, C]    -> send[q] = patches q*S/P.. of this rank's frames
//        unpack: recv[r] = rank r's frame block of this rank's patches -> y [B, T, S/P, C]
// Each is one strided copy (the relayout kernel); this file only builds the
// index maps: the 5-D dims [P, B, T/P, S/P, C] and the strides of each side.
#include "st_internal.h"

using namespace st;

namespace {

struct A2AMap {
  int64_t dims[5], chunk[5], side[5];
};

// chunk: strides of the contiguous [P, B, T/P, S/P, C] buffer; side: strides of the
// rank's own tensor, indexed by (peer, b, t, s, c) of the chunk layout.
A2AMap a2a_map(int dir, bool pack, int64_t B, int64_t T, int64_t S, int64_t C, int64_t P) {
  const int64_t tp = T / P, sp = S / P;
  A2AMap m;
  const int64_t d[5] = {P, B, tp, sp, C};
  const int64_t ch[5] = {B * tp * sp * C, tp * sp * C, sp * C, C, 1};
  for (int i = 0; i < 5; ++i) m.dims[i] = d[i], m.chunk[i] = ch[i];
  if (dir == ST_A2A_S2T) {
    if (pack) {   // x [B, T, S/P, C]: peer q gets frames q*tp + t
      const int64_t s[5] = {tp * sp * C, T * sp * C, sp * C, C, 1};
      for (int i = 0; i < 5; ++i) m.side[i] = s[i];
    } else {      // y [B, T/P, S, C]: rank r's patches at r*sp + s
      const int64_t s[5] = {sp * C, tp * S * C, S * C, C, 1};
      for (int i = 0; i < 5; ++i) m.side[i] = s[i];
    }
  } else {
    if (pack) {   // x [B, T/P, S, C]: peer q gets patches q*sp + s
      const int64_t s[5] = {sp * C, tp * S * C, S * C, C, 1};
      for (int i = 0; i < 5; ++i) m.side[i] = s[i];
    } else {      // y [B, T, S/P, C]: rank r's frames at r*tp + t
      const int64_t s[5] = {tp * sp * C, T * sp * C, sp * C, C, 1};
      for (int i = 0; i < 5; ++i) m.side[i] = s[i];
    }
  }
  return m;
}

st_status a2a_common(const void *src, void *dst, int dir, int B, int T, int S, int C, int P, int elem_bytes, bool pack,
                     hipStream_t s) {
  if (!src || !dst) return ST_EINVAL;
  if (dir != ST_A2A_S2T && dir != ST_A2A_T2S) return ST_EINVAL;
  if (B < 0 || T < 0 || S < 0 || C < 0 || P < 1 || T % P || S % P) return ST_EINVAL;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return ST_EINVAL;
  if ((uintptr_t)src % elem_bytes || (uintptr_t)dst % elem_bytes) return ST_EALIGN;
  const int64_t n = (int64_t)B * T * S * C / P;   // elements of one rank's share
  if (n == 0) return ST_OK;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, len = (uintptr_t)n * elem_bytes;
  if (a < b + len && b < a + len) return ST_EINVAL;
  const A2AMap m = a2a_map(dir, pack, B, T, S, C, P);
  if (const st_status dc = device_ok(); dc != ST_OK) return dc;
  return pack ? launch_relayout(src, m.side, dst, m.chunk, m.dims, 5, elem_bytes, s)
              : launch_relayout(src, m.chunk, dst, m.side, m.dims, 5, elem_bytes, s);
}

}  // namespace

extern "C" {

st_status st_a2a_pack(const void *x, void *send, int dir, int B, int T, int S, int C, int P, int elem_bytes,
                      void *stream) {
  return a2a_common(x, send, dir, B, T, S, C, P, elem_bytes, true, (hipStream_t)stream);
}

st_status st_a2a_unpack(const void *recv, void *y, int dir, int B, int T, int S, int C, int P, int elem_bytes,
                        void *stream) {
  return a2a_common(recv, y, dir, B, T, S, C, P, elem_bytes, false, (hipStream_t)stream);
}

}  // extern "C"
