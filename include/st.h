/*
 * st.h -- C ABI of the ST-DiT attention block on AMD MI355X (gfx950).
 *
 * The block, as the pages state it:
 *   - ScaleFusion review, "Technical architecture": an ST-DiT alternates a
 *     spatial layer (attention over the S patch tokens of each frame, input
 *     [B, T, S, C]) and a temporal layer (attention over the T frames of each
 *     patch); between them the tensor is redistributed between the
 *     [B, T, S, C] and [B, S, T, C] orders (an all-to-all across GPUs, a local
 *     permutation on one GPU).  Spatial-temporal independence: slicing along T
 *     commutes with the spatial layer, slicing along S with the temporal layer.
 *   - ScaleFusion review, "Core innovations", algorithm pseudocode: the input is
 *     rearranged to [B, N_T, N_S, T/N_T, S/N_S, C] and each layer runs slice by
 *     slice; the output returns to [B, T, S, C].
 *   - CoCoDiff page, "V-First compute scheduling": Q, K, V come from a linear
 *     projection; Q and K then get RMSNorm and RoPE, V gets neither.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless the
 *     comment says "host".  The library never allocates, frees, or keeps state
 *     between calls.  Scratch space, where needed, is a caller-provided
 *     workspace whose size the matching *_workspace() query returns.
 *   - dtype: ST_BF16 (bf16 storage, fp32 arithmetic and accumulation, outputs
 *     rounded to nearest-even) or ST_F32 (fp32 storage and arithmetic).
 *     RMSNorm gains and RoPE tables are always fp32.
 *   - Row-major layouts; the last listed dimension is contiguous.
 *   - Weights are "out-features major": w_qkv [3*H*d, c_in], w_o [c_out, H*d];
 *     y = x . w^T.  Rows 0..H*d-1 of w_qkv produce q (channel h*d + j), the
 *     next H*d produce k, the last H*d produce v.
 *   - stream is a hipStream_t (NULL: the default stream).  Calls validate
 *     their arguments on the host, enqueue kernels on the stream and return;
 *     they never synchronise.  Device faults surface at the caller's sync.
 *   - Errors are return codes only.  Argument validation happens before any
 *     HIP call, so an invalid call has no side effect.  A valid call with work
 *     to do then checks the current device: the kernels are built for gfx950,
 *     and any other device gives ST_EUNSUPPORTED before anything is enqueued.
 *     Outputs must not alias inputs (ST_EINVAL).  Pointers must be 16-byte
 *     aligned (ST_EALIGN) except for st_relayout, which needs element
 *     alignment only.
 *   - Calls are reentrant; concurrent calls on different streams are safe as
 *     long as their output buffers and workspaces do not overlap.
 *   - Sizes: activations may exceed 2^31 elements (every activation offset is
 *     64-bit).  ST_EUNSUPPORTED marks the index ranges the kernels do not
 *     cover: a weight matrix (3*H*d x c_in, n_out x k_in, c_out x H*d) of 2^31
 *     elements or more, 2^40 rows or sequences or more, a sequence length of
 *     2^30 or more, B*T*S of 2^31 or more in st_block_sliced*, a RoPE table of
 *     2^31 floats or more, and st_relayout copies of 2^32 vectors or more.
 */
#ifndef ST_H
#define ST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ST_OK = 0,
  ST_EINVAL = 1,        /* bad shape, NULL pointer, aliasing, unknown enum     */
  ST_EUNSUPPORTED = 2,  /* valid request the library has no kernel for        */
  ST_EALIGN = 3,        /* pointer not aligned as required                     */
  ST_EWORKSPACE = 4,    /* workspace NULL or smaller than the query returned   */
  ST_ELAUNCH = 5        /* a HIP launch reported an error                      */
} st_status;

typedef enum { ST_F32 = 0, ST_BF16 = 1 } st_dtype;

typedef enum {
  ST_A2A_S2T = 0,       /* patch blocks [B, T, S/P, C] -> frame blocks [B, T/P, S, C]  */
  ST_A2A_T2S = 1        /* frame blocks [B, T/P, S, C] -> patch blocks [B, T, S/P, C]  */
} st_a2a_dir;

typedef enum {
  ST_ROPE_NONE = 0,     /* no rotation                                         */
  ST_ROPE_1D = 1,       /* one segment over all d channels, position p = t     */
  ST_ROPE_2D = 2        /* axial: channels [0, d/2) by patch row h,
                           [d/2, d) by patch column w                          */
} st_rope_kind;

/* Human-readable name of a status code (static string). */
const char *st_status_str(int status);

/*
 * st_rope_table -- cosine/sine table of the rotary position encoding.
 * CoCoDiff page, "V-First compute scheduling" (RoPE on Q and K).  The rotation
 * of channel pair (2i, 2i+1) inside an axis segment of length m is
 * theta = p * base^(-2i/m): m = d for ST_ROPE_1D, m = d/2 for ST_ROPE_2D.
 *
 *   table  out  fp32 [n_pos][m/2][2] = (cos theta, sin theta) for p = 0..n_pos-1,
 *               computed in double precision on the device, rounded to fp32.
 *               Holds st_rope_table_floats(d, kind, n_pos) floats.
 * Errors: ST_EINVAL if kind is not 1D/2D, d is not even (1D) or not a multiple
 * of 4 (2D), n_pos < 1, base <= 0, table NULL.
 */
size_t st_rope_table_floats(int d, int kind, int n_pos);
st_status st_rope_table(int d, int kind, float base, int n_pos, float *table, void *stream);

/*
 * st_qkv_norm_rope -- QKV projection, then per-head RMSNorm and RoPE on q and k.
 * CoCoDiff page, "V-First compute scheduling": projection -> RMSNorm -> RoPE
 * for Q and K; V is the projection only.
 *
 *   x        in   [rows, c_in]           (dtype)
 *   w_qkv    in   [3*H*d, c_in]          (dtype)
 *   g_q,g_k  in   fp32 [d]               RMSNorm gains, shared by the heads
 *   eps           RMSNorm epsilon: t_j * g_j / sqrt(mean_j t_j^2 + eps), per (row, head)
 *   q_scale       > 0: q is stored multiplied by q_scale (1: plain q).  A layer that
 *                 passes (1/sqrt(d)) * log2(e) here and calls the attention with
 *                 scale = ln 2 computes the same softmax with q rounded once, here;
 *                 st_layer_scales() returns the pair the layer pair uses.
 *   rope_kind     st_rope_kind.  ST_ROPE_NONE ignores the arguments below up to H.
 *   rope_table in fp32 table from st_rope_table() (for the same d, kind and base)
 *   rope_npos     positions in the table
 *   pos      in   int32 [rows, 2], 8-byte aligned, or NULL.  Non-NULL: the position of
 *                 row r is pos[r] = (t, unused) for 1D, (h, w) for 2D -- any position set,
 *                 each value in [0, rope_npos) (values outside are clamped into the
 *                 table; the result is then unspecified, never a fault).
 *   pos_period, pos_offset, grid_w
 *                 used when pos is NULL: position of row r: i = r % pos_period + pos_offset;
 *                 1D: p = i;  2D: h = i / grid_w, w = i % grid_w.  Rows in [.., S] order
 *                 with pos_period = S give a frame's patches; rows in [.., T] order with
 *                 pos_period = T give frames.  Every position must be < rope_npos (ST_EINVAL).
 *   H, d          heads and head dim; dtype ST_BF16 supports d in {64, 72, 128},
 *                 ST_F32 supports even d <= 128 (multiple of 4 for 2D RoPE).
 *   q, k, v  out  [rows, H, d]           (dtype); must not overlap x, w_qkv, pos or each other
 * bf16: c_in must be a multiple of 64 (the K step of the MFMA pipeline).  rows may be 0 (no work).
 */
st_status st_qkv_norm_rope(const void *x, int64_t rows, int c_in, const void *w_qkv,
                           const float *g_q, const float *g_k, float eps, float q_scale,
                           int rope_kind, const float *rope_table, int rope_npos, const int32_t *pos,
                           int64_t pos_period, int64_t pos_offset, int grid_w,
                           int H, int d, int dtype, void *q, void *k, void *v, void *stream);

/*
 * st_layer_scales -- the q scale and attention scale a layer of st_block_sliced
 * uses for head dim d (host call, no GPU work).  The attention is
 * softmax(q.k / sqrt(d)) either way (ScaleFusion review, "Technical
 * architecture": the layers are attention layers of the transformer):
 *   ST_BF16: q_scale = (1/sqrt(d)) * log2(e), attn_scale = ln 2 -- q is stored
 *            pre-scaled, so the attention kernel's base-2 exponent is the
 *            score itself and needs no multiply;
 *   ST_F32:  q_scale = 1, attn_scale = 1/sqrt(d).
 * q_scale, attn_scale: host pointers to one float each.  ST_EINVAL for d < 1,
 * an unknown dtype or a NULL pointer.
 */
st_status st_layer_scales(int d, int dtype, float *q_scale, float *attn_scale);

/*
 * st_out_proj -- output projection of the attention result: y = a . w^T.
 * The pages do not spell the layer's output projection out; the layer is read
 * as projection -> norm/RoPE -> attention -> output projection.
 *
 *   a  in  [rows, k_in]   w in [n_out, k_in]   y out [rows, n_out]   (dtype)
 * bf16: k_in must be a multiple of 64.  n_out must be a multiple of 4.
 */
st_status st_out_proj(const void *a, int64_t rows, int k_in, const void *w, int n_out,
                      int dtype, void *y, void *stream);

/*
 * st_out_proj_relayout -- st_out_proj with the spatial <-> temporal relayout
 * (ScaleFusion review, "Technical architecture", execution flow) fused into
 * its stores: the rows of a, taken as [outer, n1, n2], are written to y as
 * [outer, n2, n1].  n1 = T, n2 = S turns the spatial layer's [B, T, S, C]
 * output into the temporal layer's [B, S, T, C] input; n1 = S, n2 = T turns
 * it back.  Every output element is bit-identical to st_out_proj followed by
 * st_relayout of the same rows; the relayout costs no extra pass over HBM.
 *
 *   a  in  [rows, k_in]   w in [n_out, k_in]   y out [rows, n_out]   (dtype)
 *   n1, n2 >= 1, rows a multiple of n1 * n2 (else ST_EINVAL; rows may be 0).
 * bf16: k_in must be a multiple of 64.  n_out must be a multiple of 4.
 */
st_status st_out_proj_relayout(const void *a, int64_t rows, int k_in, const void *w, int n_out,
                               int dtype, int64_t n1, int64_t n2, void *y, void *stream);

/*
 * st_attn_spatial -- spatial attention: for every (b, t, h),
 *   O = softmax(Q K^T * scale) V over the S patch tokens of frame t.
 * ScaleFusion review, "Technical architecture" (the spatial layer attends over
 * S); the cost is quadratic in S (PipeFusion summary, "Problem definition").
 *
 *   q, k, v  in   [B, T, S, H, d]   (the [rows, H, d] output of st_qkv_norm_rope
 *                                     for rows in [B, T, S] order)
 *   scale         usually 1/sqrt(d); passed by the caller.  bf16, d = 72: when
 *                 scale * log2(e) is a power of two (scale = ln 2 with q stored
 *                 pre-scaled, see st_layer_scales) the kernel needs no multiply
 *                 in the exponent; any other scale costs one multiply per score
 *                 (about 8% at 1080p), same precision
 *   w_o      in   NULL, or the layer's output projection [c_out, H*d]
 *   c_out         output channels when w_o is given (multiple of 4)
 *   out      out  w_o NULL: O [B, T, S, H, d];  else O . w_o^T [B, T, S, c_out]
 *   ws, ws_bytes  w_o given: device workspace of at least st_attn_workspace(B*T*S, H, d,
 *                 dtype) bytes, where O is staged (else ignored; may be NULL)
 * Same d support as st_qkv_norm_rope; bf16 with w_o needs H*d % 64 == 0.  S >= 1.
 */
st_status st_attn_spatial(const void *q, const void *k, const void *v, int B, int T, int S,
                          int H, int d, float scale, int dtype, const void *w_o, int c_out,
                          void *out, void *ws, size_t ws_bytes, void *stream);
/* Bytes of workspace an attention call with w_o needs for `rows` query rows (0 if invalid). */
size_t st_attn_workspace(int64_t rows, int H, int d, int dtype);

/*
 * st_attn_temporal -- temporal attention: for every (b, s, h),
 *   O = softmax(Q K^T * scale) V over the T frames of patch s,
 * where keys at frames t >= t_valid get weight exactly 0 (frames appended to
 * make T a multiple of the slice count N_T; their query rows are computed
 * but carry no meaning).
 * ScaleFusion review, "Technical architecture" (the temporal layer attends over T).
 *
 *   q, k, v  in   [B, S, T, H, d]
 *   1 <= t_valid <= T.
 *   scale, w_o, c_out, ws, ws_bytes   as st_attn_spatial (rows = B*S*T)
 *   out      out  w_o NULL: O [B, S, T, H, d];  else O . w_o^T [B, S, T, c_out]
 */
st_status st_attn_temporal(const void *q, const void *k, const void *v, int B, int S, int T,
                           int t_valid, int H, int d, float scale, int dtype, const void *w_o,
                           int c_out, void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * st_attn_chunk -- attention of queries over ONE chunk of keys/values, with the
 * log-sum-exp of the chunk's scores.  Ring attention (PipeFusion summary,
 * "Problem definition": sequence parallelism splits the sequence; SwiftFusion,
 * "Topology-Aware Communication Scheduling") and Torus attention (SwiftFusion,
 * "Torus Attention") compute attention of the local queries against one
 * key/value chunk at a time and combine the partial results; st_attn_merge is
 * the combination.  For every (o, h) and query i:
 *   out[o, i, h] = softmax_j(scale * q_i . k_j) v_j   over keys j < kv_valid of the chunk
 *   lse[o, h, i] = log sum_j exp(scale * q_i . k_j)    (natural log, same keys)
 *
 *   q        in   [outer, Lq, H, d]
 *   k, v     in   [outer, Lk, H, d]   (the chunk)
 *   kv_valid      keys j >= kv_valid of the chunk are excluded; 0 <= kv_valid <= Lk.
 *                 kv_valid = 0 gives out = 0 and lse = -inf (an empty chunk).
 *   out      out  [outer, Lq, H, d]   (dtype)
 *   lse      out  fp32 [outer, H, Lq], 4-byte aligned
 * Same d support as st_attn_spatial.  Outputs must not overlap the inputs or
 * each other (ST_EINVAL).  Lq = Lk with kv_valid = Lk is st_attn_spatial plus lse.
 */
st_status st_attn_chunk(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk, int kv_valid,
                        int H, int d, float scale, int dtype, void *out, float *lse, void *stream);

/*
 * st_attn_chunk_acc -- st_attn_chunk and st_attn_merge in one pass: the step
 * Ring and Torus attention repeat as each key/value chunk arrives (same
 * passages as st_attn_chunk).  acc_o / acc_lse hold the result over the keys
 * seen so far and receive the result over those keys and this chunk:
 *   lse_c = log sum_j exp(scale * q_i . k_j)          over this chunk's keys
 *   acc_lse' = log(exp(acc_lse) + exp(lse_c))
 *   acc_o'   = exp(acc_lse - acc_lse') acc_o + exp(lse_c - acc_lse') softmax_j(..) v_j
 * The chunk's own output never leaves the kernel (fp32 in registers), so the
 * merge costs one read of the accumulator instead of a separate pass over two
 * partial results.  acc_lse = -inf marks an empty accumulator: its acc_o row
 * is then ignored (any contents) and the call writes this chunk's result,
 * bit-identical to st_attn_chunk.  kv_valid = 0 leaves the accumulator as it is.
 *
 *   q, k, v, kv_valid   as st_attn_chunk
 *   acc_o     in/out  [outer, Lq, H, d]   (dtype)
 *   acc_lse   in/out  fp32 [outer, H, Lq], 4-byte aligned
 * Same validation and error codes as st_attn_chunk (acc_o, acc_lse in the
 * roles of out, lse).
 */
st_status st_attn_chunk_acc(const void *q, const void *k, const void *v, int64_t outer, int Lq, int Lk, int kv_valid,
                            int H, int d, float scale, int dtype, void *acc_o, float *acc_lse, void *stream);

/*
 * st_attn_merge -- the attention result over the union of two disjoint key
 * chunks, from the two chunk results (st_attn_chunk or earlier merges):
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   out = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
 * per (o, i, h), computed in fp32.  A part with lse = -inf (no keys) has weight
 * 0; two empty parts give out = 0, lse = -inf.
 *
 *   o_a, o_b  in   [outer, L, H, d]   (dtype)     lse_a, lse_b  in  fp32 [outer, H, L]
 *   out       out  [outer, L, H, d]   (dtype)     lse           out fp32 [outer, H, L]
 * out may be o_a or o_b itself and lse may be lse_a or lse_b itself (a running
 * merge in place); any other overlap is ST_EINVAL.  d >= 1 (any size).
 */
st_status st_attn_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int64_t outer, int L,
                        int H, int d, int dtype, void *out, float *lse, void *stream);

/*
 * st_v_change -- V-Major change detection (CoCoDiff page, "V-Major selective
 * communication"): per denoising step, a V vector whose L1 change against the
 * cached vector of the previous step exceeds a threshold is active (its Q, K,
 * V are communicated); the others are read from the cache.  A vector is one
 * (token, head) row of V:
 *   dist[v] = sum_j |v_new[v, j] - v_cache[v, j]|   (fp32)
 *   mask[v] = dist[v] > threshold
 *
 *   v_new     in      [rows, H, d]   (dtype)     v_cache  in/out  [rows, H, d]
 *   threshold         >= 0 (or +inf); the page gives no value, so the caller chooses it
 *   mask      out     uint8 [rows, H]: 1 active, 0 not (16-byte aligned)
 *   active_idx out    int32 [rows * H] capacity, or NULL: the first *n_active entries are
 *                     the flat indices r * H + h of the active vectors, increasing within
 *                     each run of 1024 vectors, runs in unspecified order
 *   n_active  out     device int64: number of active vectors (8-byte aligned)
 *   update_cache      nonzero: v_cache rows of active vectors are overwritten with v_new
 * d * element size must be a multiple of 16 bytes and at most 512 (bf16 d % 8 == 0,
 * d <= 256; fp32 d % 4 == 0, d <= 128).  Outputs must not overlap inputs or each other;
 * v_new and v_cache must not overlap.  The whole-step refresh the page describes (every
 * 10 steps, all vectors) is the caller's: pass threshold 0 or copy v_new.
 */
st_status st_v_change(const void *v_new, void *v_cache, int64_t rows, int H, int d, float threshold, int dtype,
                      uint8_t *mask, int32_t *active_idx, int64_t *n_active, int update_cache, void *stream);

/*
 * st_relayout -- strided N-D copy, the one-GPU form of the spatial <-> temporal
 * redistribution (ScaleFusion review, "Technical architecture", execution flow)
 * and of the blocked rearranges and slice gathers/scatters of the algorithm
 * pseudocode ("Core innovations").
 *
 * For every multi-index i with 0 <= i_k < dims[k]:
 *     dst[sum_k i_k * dst_strides[k]] = src[sum_k i_k * src_strides[k]]
 * dims, src_strides, dst_strides are HOST arrays of ndim int64 values;
 * strides are in elements.  1 <= ndim <= 6, elem_bytes in {1, 2, 4, 8, 16}.
 * The destination index map must be one-to-one and must not overlap the
 * source (not checked beyond src != dst).  Bit-exact copy.
 */
st_status st_relayout(const void *src, const int64_t *src_strides, void *dst,
                      const int64_t *dst_strides, const int64_t *dims, int ndim,
                      int elem_bytes, void *stream);

/*
 * st_a2a_pack / st_a2a_unpack -- one rank's local pack before, and unpack after,
 * the P-way all-to-all between the two shardings of the layer pair (ScaleFusion
 * review, "Technical architecture": the layer table gives each rank [B, T, S/P, C]
 * for the temporal layer and [B, T/P, S, C] for the spatial layer, and an
 * all-to-all converts between them; "Core innovations", algorithm pseudocode:
 * the exchange sits between the layers).  A collective moves one contiguous
 * chunk per peer, so the exchange is pack -> all-to-all -> unpack.  Chunk layout
 * on the wire, both directions: [P, B, T/P, S/P, C], chunk q contiguous.
 *
 *   dir = ST_A2A_S2T (before the spatial layer):
 *     pack    x    [B, T, S/P, C]   this rank's patch block  -> send [P, B, T/P, S/P, C],
 *                                   chunk q = frames q*T/P .. (q+1)*T/P - 1
 *     unpack  recv [P, B, T/P, S/P, C], chunk r from rank r  -> y [B, T/P, S, C],
 *                                   rank r's patches at r*S/P ..
 *   dir = ST_A2A_T2S (before the temporal layer):
 *     pack    x    [B, T/P, S, C]   this rank's frame block  -> send [P, B, T/P, S/P, C],
 *                                   chunk q = patches q*S/P .. (q+1)*S/P - 1
 *     unpack  recv [P, B, T/P, S/P, C], chunk r from rank r  -> y [B, T, S/P, C],
 *                                   rank r's frames at r*T/P ..
 *   T, S        the GLOBAL frame and patch counts; T % P == 0 and S % P == 0
 *               (pad T with masked frames first, as for the slicing schedule)
 *   elem_bytes  1, 2, 4 or 8; pointers aligned to it
 * Both buffers hold B*T*S*C/P elements and must not overlap (ST_EINVAL).
 * Bit-exact copies (one st_relayout pass each).  P = 1 is a plain copy.
 */
st_status st_a2a_pack(const void *x, void *send, int dir, int B, int T, int S, int C, int P,
                      int elem_bytes, void *stream);
st_status st_a2a_unpack(const void *recv, void *y, int dir, int B, int T, int S, int C, int P,
                        int elem_bytes, void *stream);

/* Weights of one layer (all device pointers). */
typedef struct {
  const void *w_qkv;   /* [3*H*d, C] */
  const void *w_o;     /* [C, H*d]   */
  const float *g_q;    /* [d] */
  const float *g_k;    /* [d] */
} st_layer_weights;

/*
 * st_block_sliced -- the spatial + temporal layer pair under the slicing
 * schedule at one GPU (ScaleFusion review, "Core innovations": intra-layer
 * scheduling and the algorithm pseudocode; N_T = N_S = 4 in "Experimental
 * results").  x [B, T, S, C] is rearranged to [B, N_T, N_S, T/N_T, S/N_S, C];
 * the spatial layer runs once per time slice (T/N_T frames, all S patches,
 * 2D RoPE with global (h, w)), the temporal layer once per space slice
 * (S/N_S patches, all T frames, 1D RoPE with global t, keys t >= t_valid
 * masked); the result is rearranged back to y [B, T, S, C].
 * n_t = n_s = 1 is the unsliced layer pair.  In bf16 the rearranges and the
 * per-slice gathers and scatters move no data of their own: each slice's QKV
 * projection reads its rows from where they lie and its output projection
 * stores them where the next phase (or y) expects them.  fp32 runs them as
 * explicit copies.
 *
 *   x         in   [B, T, S, C]   bf16: C and H*d multiples of 64.
 *                                 T % n_t == 0, S % n_s == 0 (the caller pads T
 *                                 with zero frames and passes t_valid)
 *   grid_w         patch-grid width; S % grid_w == 0; s = h * grid_w + w
 *   spatial, temporal   host pointers to the two layers' weights
 *   y         out  [B, T, S, C]
 *   ws             device workspace of at least st_block_sliced_workspace() bytes
 *                  (bf16: the blocked intermediate [B, T, S, C] when sliced, or the
 *                  [B, S, T, C] temporal-layer input when not, plus q, k, v and the
 *                  attention output for the largest slice; fp32 adds the explicit
 *                  copies' slice buffers)
 * Each output element is computed by the same arithmetic in the same order
 * whatever n_t and n_s are, so sliced and unsliced results are bit-identical.
 */
st_status st_block_sliced(const void *x, int B, int T, int t_valid, int S, int grid_w, int C,
                          int H, int d, int n_t, int n_s, const st_layer_weights *spatial,
                          const st_layer_weights *temporal, float eps, float rope_base,
                          int dtype, void *y, void *ws, size_t ws_bytes, void *stream);
size_t st_block_sliced_workspace(int B, int T, int S, int grid_w, int C, int H, int d,
                                 int n_t, int n_s, int dtype);

/*
 * st_block_sliced_2s -- st_block_sliced with the slicing schedule pipelined on
 * two streams, the one-GPU form of the overlap the ScaleFusion review describes
 * ("Core innovations", intra-layer scheduling: while one slice is computed, the
 * next slice's data moves).  The layer computations (projections, attention)
 * run on `stream`; the slice gathers, scatters and the two blocked rearranges
 * run on `side_stream`, so slice i's gather overlaps slice i-1's computation
 * and its scatter overlaps slice i+1's.  Slice buffers are double-buffered in
 * the workspace, whose size st_block_sliced_2s_workspace() returns (larger than
 * st_block_sliced's in bf16: the copies need the blocked input and output and
 * two sets of slice buffers).
 *
 *   stream, side_stream  two distinct, non-NULL hipStream_t (ST_EINVAL
 *                        otherwise).  The call orders side_stream after the
 *                        work already on stream, and stream after everything
 *                        the call puts on side_stream: y is complete in
 *                        stream order, exactly as for st_block_sliced.
 * The result is bit-identical to st_block_sliced with the same arguments.  The
 * call creates and releases HIP events (no device memory).  n_t = n_s = 1 runs
 * entirely on `stream`.
 */
st_status st_block_sliced_2s(const void *x, int B, int T, int t_valid, int S, int grid_w, int C,
                             int H, int d, int n_t, int n_s, const st_layer_weights *spatial,
                             const st_layer_weights *temporal, float eps, float rope_base,
                             int dtype, void *y, void *ws, size_t ws_bytes, void *stream,
                             void *side_stream);
size_t st_block_sliced_2s_workspace(int B, int T, int S, int grid_w, int C, int H, int d,
                                    int n_t, int n_s, int dtype);

/*
 * st_block_sliced_noalloc -- st_block_sliced for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, which is
 * taken from a fixed device array inside the library instead.  The call
 * allocates nothing and frees nothing; the result is bit-identical to
 * st_block_sliced on the same arguments.
 *
 *   Limit: the workspace st_block_sliced_workspace() reports for the arguments
 *   must be at most st_block_sliced_noalloc_max() bytes (256 MiB), else
 *   ST_EWORKSPACE before any GPU work.  For example the layer pair of 16 heads
 *   x 72, C = 1152, fits up to about 23,000 tokens per call (B*T*S).
 *   The array exists once per GPU the library runs on and stays allocated
 *   until the process ends.  Every call on one GPU uses that GPU's copy, so
 *   calls that overlap in time on one GPU (other streams, other host threads)
 *   race on it: the caller must order them.  Nothing in it needs to start at
 *   zero; a call overwrites what it reads.
 * Validation and error codes as st_block_sliced, plus ST_ELAUNCH if the
 * array's device address cannot be obtained.
 */
st_status st_block_sliced_noalloc(const void *x, int B, int T, int t_valid, int S, int grid_w, int C,
                                  int H, int d, int n_t, int n_s, const st_layer_weights *spatial,
                                  const st_layer_weights *temporal, float eps, float rope_base,
                                  int dtype, void *y, void *stream);
size_t st_block_sliced_noalloc_max(void);

#ifdef __cplusplus
}
#endif
#endif /* ST_H */
