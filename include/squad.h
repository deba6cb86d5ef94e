/*
 * squad.h - C ABI of libsquad, the SQuad-Attention forward path for AMD MI355X (gfx950).
 *
 * SQuad-Attention replaces full softmax self-attention over the n latent tokens of
 * a video diffusion transformer by two softmax passes of O(n*sqrt(n)) total cost
 * (pages titled "SQuad: Sub-Quadratic Attention Distillation for Efficient Video
 * Generation"; the operator is defined in the gist.science technical summary,
 * section "Methodologie: SQuad", item "1. SQuad-Attention Operator"):
 *
 *   local pass  Attn_L : softmax attention among the tokens of each fixed window;
 *   global pass Attn_G : softmax attention among the tokens at the same relative
 *                        position (offset) inside their windows, across all windows;
 *   composition        : the local output is the value stream of the global pass,
 *                        out = Attn_G(q, k, Attn_L(q, k, v)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tokens are the cells of a T x H x W latent grid (grid[3] = {T, H, W}), numbered
 * row-major over (t, h, w); n = T*H*W.  A window is a tt x th x tw tile
 * (tile[3] = {tt, th, tw}); Wn = tt*th*tw tokens per window, G = n / Wn windows.
 * Windows are numbered row-major over the window grid (T/tt, H/th, W/tw) and the
 * offset of a token inside its window row-major over (tt, th, tw).
 *
 * Cut tilings (squad_attn_forward, its two halves, squad_local_pass and
 * squad_global_pass): a grid that is not a
 * whole number of tiles (each tile no larger than the grid) is read as padded up to
 * one with absent tokens.  The window grid is (ceil(T/tt), ceil(H/th), ceil(W/tw));
 * the tiles on the far edges are cut by the grid, so their windows hold fewer
 * tokens and an offset group holds one token per window that has that offset.
 * Absent tokens are neither keys nor queries.  (The pages use whole tiles only;
 * this is the plainest extension, and on whole tiles it is the operator above.)
 * The permutation entry points return SQUAD_ERR_SHAPE for cut tilings.  Outputs in token order cover exactly
 * the n present tokens.
 *
 * Token-order tensors are contiguous [batch, n, heads, head_dim] (= [B, n, hidden]).
 * Window-major tensors are contiguous [batch, heads, G, Wn, head_dim]; group-major
 * tensors are contiguous [batch, heads, Wn, G, head_dim].
 *
 * dtype: SQUAD_DTYPE_F32 (all tensors fp32, fp32 arithmetic throughout) or
 * SQUAD_DTYPE_BF16 (bf16 tensors; fp32 accumulation and softmax; the attention
 * weights are rounded to the value type for the weights-times-values product).
 * Inside squad_attn_forward the local output is held in fp16 between the two
 * passes (same bytes as bf16, three more significand bits); values of magnitude
 * 65504 or more overflow there and surface as inf/nan in the output.
 * head_dim must be 64 or 128.
 * scale <= 0 selects the softmax scale 1/sqrt(head_dim).
 * Sizes: G * Wn (tile cells, absent ones included) below 2^31, and per batch
 * element G * Wn * heads below 2^32 - 1 head rows (a bf16 tensor of up to 2^39
 * bytes at head_dim 128); SQUAD_ERR_SHAPE beyond.  Rows of tensors below 2^31
 * elements per batch element are located with 32-bit element offsets; larger
 * ones with offsets in head rows and 64-bit addresses (the 16-bit engine then
 * takes its table-free, per-block presence form).  The k-level entry points
 * keep the first limit (n * heads * head_dim below 2^31), as do
 * squad_window_attn (len * head_dim) and squad_dense_attn_forward
 * (n * heads * head_dim).
 *
 * Pointers are device pointers that the caller owns; base pointers must be 16-byte
 * aligned.  The library never allocates or frees device memory and never
 * synchronises: work is enqueued on `stream` (NULL = the null stream) and kernel
 * faults surface at the caller's next synchronisation.  Inputs are read-only;
 * outputs may not overlap inputs or the workspace.  Every argument check runs on
 * the host before anything is enqueued, so a nonzero status leaves the outputs
 * untouched.  The library is reentrant.  Exceptions, noted where they are
 * declared: squad_attn_forward_noalloc keeps the address of its own scratch array
 * per device, and squad_blas_create creates a rocBLAS handle (which owns whatever
 * device memory rocBLAS allocates for it) for the caller to pass to
 * squad_block_forward and to release with squad_blas_destroy.
 */
#ifndef SQUAD_H
#define SQUAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* squad_stream_t; /* the same type as hipStream_t */
typedef struct _rocblas_handle* squad_blas_t;  /* the same type as rocblas_handle */

enum squad_status {
  SQUAD_OK = 0,
  SQUAD_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, unknown selector          */
  SQUAD_ERR_SHAPE = 2,       /* tile larger than the grid, a cut tiling where only
                                whole tilings are accepted, or sizes too large       */
  SQUAD_ERR_UNSUPPORTED = 3, /* head_dim not 64/128 or dtype unknown                 */
  SQUAD_ERR_ALIAS = 4,       /* an output overlaps an input or the workspace         */
  SQUAD_ERR_ALIGN = 5,       /* a base pointer is not 16-byte aligned                */
  SQUAD_ERR_WORKSPACE = 6,   /* workspace null or smaller than required             */
  SQUAD_ERR_HIP = 7,         /* a HIP call failed (no device, launch failure)        */
  SQUAD_ERR_SCRATCH = 8      /* squad_attn_forward_noalloc: one (batch, head)'s local
                                output exceeds SQUAD_NOALLOC_SCRATCH_BYTES          */
};

/* Bytes of device scratch squad_attn_forward_noalloc keeps per device. */
#define SQUAD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum squad_dtype { SQUAD_DTYPE_F32 = 0, SQUAD_DTYPE_BF16 = 1 };

/* Static, human-readable text for a status code. */
const char* squad_status_string(int status);

/*
 * SQuad-Attention forward (local pass, then global pass with the local output as
 * its value stream; technical summary, "1. SQuad-Attention Operator").
 *   q, k, v, out : token order [batch, n, heads, head_dim], dtype `dtype`.
 *   workspace    : device scratch of at least squad_attn_workspace_size(...) bytes;
 *                  holds the local output, group-major [batch, heads, Wn, G,
 *                  head_dim] (fp16 for bf16 calls, fp32 for fp32 calls); on cut
 *                  tilings G counts every window of the rounded-up window grid and
 *                  the rows of absent tokens are left unwritten.
 * Enqueues two kernels on `stream`: squad_attn_forward_local, then
 * squad_attn_forward_global.
 */
int squad_attn_forward(const void* q, const void* k, const void* v,
                       const int32_t grid[3], const int32_t tile[3], int32_t heads,
                       void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                       float scale, void* workspace, size_t workspace_bytes,
                       squad_stream_t stream);

/*
 * First half of squad_attn_forward: the local pass ("1. SQuad-Attention Operator",
 * Local Pass), writing its output into `workspace` in the layout described above.
 */
int squad_attn_forward_local(const void* q, const void* k, const void* v,
                             const int32_t grid[3], const int32_t tile[3], int32_t heads,
                             int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                             void* workspace, size_t workspace_bytes, squad_stream_t stream);

/*
 * Second half of squad_attn_forward: the global pass ("1. SQuad-Attention
 * Operator", Global Pass and Compositie) over the local output that
 * squad_attn_forward_local left in `workspace`, writing `out` in token order.
 */
int squad_attn_forward_global(const void* q, const void* k,
                              const int32_t grid[3], const int32_t tile[3], int32_t heads,
                              void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                              float scale, const void* workspace, size_t workspace_bytes,
                              squad_stream_t stream);

/* Bytes of workspace squad_attn_forward needs (batch*heads*G*Wn*head_dim elements of
 * `dtype`, = batch*heads*n*head_dim on whole tilings); 0 if the arguments are
 * invalid. */
size_t squad_attn_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads,
                                 int32_t batch, int32_t head_dim, int32_t dtype);

/*
 * squad_attn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, layout, precision and statuses as squad_attn_forward, without the
 * workspace: the local output lives in a device array of
 * SQUAD_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one copy per device,
 * held until the process ends.  When batch * heads * G * Wn * head_dim elements of
 * the local output (fp16 for bf16 calls, fp32 for fp32) exceed it, the call runs
 * the two passes over slices of the heads of one batch element at a time, one
 * after the other on `stream`; one (batch, head)'s local output must fit
 * (SQUAD_ERR_SCRATCH otherwise: at head_dim 128, G * Wn <= 262,144 cells in bf16,
 * 131,072 in fp32).  Results are bit-identical to squad_attn_forward's.  Nothing
 * in the scratch needs to start at zero (every cell the global pass reads is
 * written by the local pass first).  Every call on a device shares that device's
 * array: calls that overlap in time on one device (different streams, or
 * different host threads without ordering) race on it and must not be issued.
 * The first call on a device looks up the array's address (hipGetSymbolAddress)
 * and keeps it; no call allocates or frees memory.
 */
int squad_attn_forward_noalloc(const void* q, const void* k, const void* v,
                               const int32_t grid[3], const int32_t tile[3], int32_t heads,
                               void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                               float scale, squad_stream_t stream);

/*
 * Training.  The distillation the pages run (flow-matching SFT, then DMD2;
 * technical summary, "Methodologie") fine-tunes the model through the operator, so
 * it needs the gradients of out = Attn_G(q, k, Attn_L(q, k, v)).  The pages give no
 * formula; these entry points compute the chain rule of the two softmax passes:
 * with o1 = Attn_L(q, k, v) and the upstream gradient dout,
 *   (dq_G, dk_G, do1) = gradients of Attn_G at (q, k, o1) given dout,
 *   (dq_L, dk_L, dv)  = gradients of Attn_L at (q, k, v) given do1,
 *   dq = dq_G + dq_L,  dk = dk_G + dk_L.
 * Inside one pass, for a unit's softmax P and output o: dv = P^T dout;
 * dS_ij = P_ij (<dout_i, v_j> - <dout_i, o_i>); dq = scale dS k; dk = scale dS^T q.
 *
 * squad_attn_train_workspace_size: bytes of the one workspace both calls take
 * (the local output, each pass's per-row softmax statistic, and the backward's
 * scratch: the local output's gradient, per-row <dout, o>, and for bf16 calls
 * one scale per head row of dq and of dk); 0 if the arguments are invalid.
 *
 * squad_attn_forward_train: squad_attn_forward (same arguments and checks) that
 * also keeps, in `workspace`, what squad_attn_backward needs.  `out` is the same
 * as squad_attn_forward's.
 *
 * squad_attn_backward: q, k, v, out (the training forward's output) and dout,
 * token order [batch, n, heads, head_dim] in `dtype`; writes dq, dk, dv (same
 * layout and dtype).  `workspace` must hold what squad_attn_forward_train wrote
 * with the same q, k, v, grid, tile, heads, batch, head_dim, dtype and scale (its
 * scratch part is overwritten).  bf16 calls compute in fp32 with bf16 MFMA
 * operands (P and dS rounded to bf16; the global pass's <dout, o1> products on
 * fp16 operands, dout scaled per row by a power of two) and round the gradients
 * to bf16 once.  Between the passes, bf16 calls keep the global pass's dq and dk
 * parts in dq and dk themselves, as fp16 rows scaled per row by a power of two
 * (each element within 2^-12 of its row's largest magnitude); dq and dk are
 * therefore written twice.
 * Statuses as for squad_attn_forward; the three outputs must not overlap each
 * other, an input or the workspace.  Work is enqueued on `stream`: four kernel
 * launches, no allocation, no synchronisation.
 */
size_t squad_attn_train_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads,
                                       int32_t batch, int32_t head_dim, int32_t dtype);
int squad_attn_forward_train(const void* q, const void* k, const void* v,
                             const int32_t grid[3], const int32_t tile[3], int32_t heads,
                             void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                             float scale, void* workspace, size_t workspace_bytes,
                             squad_stream_t stream);
int squad_attn_backward(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const int32_t grid[3], const int32_t tile[3],
                        int32_t heads, void* dq, void* dk, void* dv, int32_t batch,
                        int32_t head_dim, int32_t dtype, float scale, void* workspace,
                        size_t workspace_bytes, squad_stream_t stream);

/*
 * Tile planner.  The pages choose windows of about sqrt(n) tokens (technical
 * summary, "1. SQuad-Attention Operator", Complexiteit: w = sqrt(n) gives
 * O(n sqrt n)).  On a 3-D grid this picks the tile (tt <= T, th <= H, tw <= W)
 * that minimises the forward's product work, proportional to
 * Gp * Wn * (Wn + Gp) with Wn = tt*th*tw and Gp the number of windows of the
 * (possibly cut) tiling; ties go to the tiling with fewer absent tokens, then to
 * the most compact window (per axis, the tile extent closest to the number of
 * windows along that axis: least sum of squared log ratios), then to the first
 * in ascending (tt, th, tw) order.  Host-only; writes tile_out[3].
 * Returns SQUAD_ERR_INVALID_ARG for null pointers or sizes <= 0, SQUAD_ERR_SHAPE
 * for grids of 2^31 tokens or more.
 */
int squad_plan_tile(const int32_t grid[3], int32_t tile_out[3]);

/*
 * The attention block around the operator.  The pages time the attention per
 * block of a 5B video DiT (technical summary, "Experimentele Resultaten": the
 * per-block attention latency falls from 47.10 ms to 4.27 ms, about 11x).  This runs the block's attention path with given
 * weights (no bias, no normalisation; the pages describe neither):
 *   qkv = x w_qkv^T   (x [batch, n, hidden], w_qkv [3 hidden, hidden], nn.Linear
 *                      layout; q, k, v are qkv's column blocks, each [n, heads, d])
 *   a   = SQuad-Attention(q, k, v) (dense = 1: full softmax attention instead,
 *                      the comparator)
 *   y   = a w_out^T   (w_out [hidden, hidden]; y [batch, n, hidden])
 * hidden = heads * head_dim.  The projections are plain GEMMs on rocBLAS (fp32
 * accumulation, outputs rounded to `dtype`) on the caller's handle `blas`, whose
 * stream this call sets to `stream`; the attention kernels read q, k and v in place
 * from the projection's output rows (row stride 3 hidden).  `workspace` holds qkv,
 * the operator's workspace and a (squad_block_workspace_size bytes).  Statuses as
 * for squad_attn_forward (SQUAD_ERR_INVALID_ARG for a null handle), plus
 * SQUAD_ERR_SHAPE if dense = 1 and n * 3 * hidden reaches 2^31 (the comparator
 * keeps 32-bit element offsets).  The call keeps no state of
 * its own; rocBLAS may allocate device memory on the handle, which the handle owns.
 *
 * squad_blas_create: a rocBLAS handle on the current device for squad_block_forward
 * (SQUAD_ERR_HIP if rocBLAS cannot create one); squad_blas_destroy releases it and
 * whatever rocBLAS allocated for it.
 */
int squad_blas_create(squad_blas_t* handle);
int squad_blas_destroy(squad_blas_t handle);
size_t squad_block_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads, int32_t batch,
                                  int32_t head_dim, int32_t dtype);
int squad_block_forward(const void* x, const void* w_qkv, const void* w_out, const int32_t grid[3],
                        const int32_t tile[3], int32_t heads, void* y, int32_t batch, int32_t head_dim,
                        int32_t dtype, float scale, int32_t dense, squad_blas_t blas, void* workspace,
                        size_t workspace_bytes, squad_stream_t stream);

/*
 * More than two passes.  The pages name composing more than two passes as future
 * work, trading depth for efficiency (technical summary, "Betekenis en Claims").  The reading taken here: `levels` = k passes over nested tiles
 * t1 | t2 | ... | t(k-1) | grid (tiles holds (k-1) x 3 int32 {tt, th, tw}, each
 * tile dividing the next and the last dividing the grid, per axis).  Each axis
 * coordinate splits into k digits (digit j: the position among the t(j)-tiles
 * inside the t(j+1)-tile, t0 = one cell, tk = the grid); pass j is the standard
 * softmax attention among the tokens that differ only in digit j, with the same
 * q and k, and its output is the value stream of pass j + 1:
 *   o_0 = v,  o_(j+1) = Attn_j(q, k, o_j),  out = o_k.
 * k = 2 is squad_attn_forward with tile = t1.  With unit sizes about n^(1/k)
 * the work is O(k n^(1+1/k)).  Whole tilings only (SQUAD_ERR_SHAPE if the tiles
 * do not nest); 2 <= levels <= 8 (else SQUAD_ERR_INVALID_ARG).
 * q, k, v, out token order [batch, n, heads, head_dim]; `workspace` holds the
 * intermediate outputs in token order (fp16 for bf16 calls, fp32 for fp32),
 * squad_kpass_workspace_size bytes (0 for invalid arguments).  One kernel
 * launch per pass; other statuses as for squad_attn_forward.
 */
size_t squad_kpass_workspace_size(const int32_t grid[3], const int32_t* tiles, int32_t levels,
                                  int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype);
int squad_kpass_forward(const void* q, const void* k, const void* v, const int32_t grid[3],
                        const int32_t* tiles, int32_t levels, int32_t heads, void* out,
                        int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                        void* workspace, size_t workspace_bytes, squad_stream_t stream);

/*
 * Training the k-level operator: the chain rule over the levels, from the last
 * down (level j's backward at (q, k, o_j) given the gradient of o_(j+1) yields
 * its parts of dq and dk and the gradient of o_j; dv is the gradient of o_0).
 * squad_kpass_train_workspace_size: bytes of the workspace both calls share (the
 * intermediate outputs, each level's row statistics, and the backward's scratch).
 * squad_kpass_forward_train: squad_kpass_forward keeping that state.
 * squad_kpass_backward: dq, dk, dv ([batch, n, heads, head_dim], the call's dtype)
 * from q, k, v, the training forward's out and dout, with its workspace (same
 * grid, tiles, heads, batch, head_dim, dtype and scale).  Precision and statuses
 * as for squad_attn_backward; two kernel launches per level.
 */
size_t squad_kpass_train_workspace_size(const int32_t grid[3], const int32_t* tiles, int32_t levels,
                                        int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype);
int squad_kpass_forward_train(const void* q, const void* k, const void* v, const int32_t grid[3],
                              const int32_t* tiles, int32_t levels, int32_t heads, void* out,
                              int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                              void* workspace, size_t workspace_bytes, squad_stream_t stream);
int squad_kpass_backward(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const int32_t grid[3], const int32_t* tiles, int32_t levels,
                         int32_t heads, void* dq, void* dk, void* dv, int32_t batch, int32_t head_dim,
                         int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                         squad_stream_t stream);

/*
 * Local pass alone (Attn_L): o1 = softmax attention inside each window.
 * q, k, v, o1 token order [batch, n, heads, head_dim].
 */
int squad_local_pass(const void* q, const void* k, const void* v,
                     const int32_t grid[3], const int32_t tile[3], int32_t heads,
                     void* o1, int32_t batch, int32_t head_dim, int32_t dtype,
                     float scale, squad_stream_t stream);

/*
 * Global pass alone (Attn_G): out = softmax attention among same-offset tokens
 * across windows, with `vstream` as the value stream (in the operator, the local
 * output).  All four tensors token order [batch, n, heads, head_dim].
 */
int squad_global_pass(const void* q, const void* k, const void* vstream,
                      const int32_t grid[3], const int32_t tile[3], int32_t heads,
                      void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                      float scale, squad_stream_t stream);

/*
 * Tile gather: token order [batch, n, heads, head_dim] -> window-major
 * [batch, heads, G, Wn, head_dim] (the tensor reshaping the method is built from;
 * technical summary, "Belangrijkste Bijdragen").  An exact copy.
 */
int squad_tile_gather(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                      int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                      squad_stream_t stream);

/* Tile scatter: the inverse of squad_tile_gather (window-major -> token order). */
int squad_tile_scatter(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                       int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                       squad_stream_t stream);

/*
 * Window-to-group transpose: window-major [batch, heads, G, Wn, head_dim] ->
 * group-major [batch, heads, Wn, G, head_dim], the regrouping between the local
 * and the global pass ("1. SQuad-Attention Operator", Global Pass).  Exact copy.
 */
int squad_window_to_group(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                          int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                          squad_stream_t stream);

/*
 * Batched short-sequence softmax attention, one independent attention per unit:
 * q, k, v, out contiguous [units, len, head_dim].  The engine behind both passes,
 * each of which is standard softmax attention over its units ("1. SQuad-Attention
 * Operator", Complexiteit).
 */
int squad_window_attn(const void* q, const void* k, const void* v, void* out,
                      int32_t units, int32_t len, int32_t head_dim, int32_t dtype,
                      float scale, squad_stream_t stream);

/*
 * Dense full softmax self-attention over all n tokens (the quadratic operator the
 * method replaces; abstract).  Comparator only.  q, k, v, out token order
 * [batch, n, heads, head_dim].
 */
int squad_dense_attn_forward(const void* q, const void* k, const void* v, void* out,
                             int32_t batch, int32_t n, int32_t heads, int32_t head_dim,
                             int32_t dtype, float scale, squad_stream_t stream);

/*
 * Host-only: the element offsets the six-digit map of pass `level` of a k-level
 * operator gives, in the order [batch][heads][units][rows] (rows = the level's
 * digits row-major over (t, h, w); units = the other digits).  offsets must
 * hold batch*heads*n entries.  The middle passes of squad_kpass_forward use
 * this map; its first and last passes use the two-pass maps.
 */
int squad_debug_kpass_offsets(const int32_t grid[3], const int32_t* tiles, int32_t levels, int32_t level,
                              int32_t heads, int32_t batch, int32_t head_dim, int64_t* offsets);

/*
 * Measuring kernel (not part of the operator): `blocks` workgroups of 256 threads,
 * each wave running `iters` (rounded up to a multiple of 4) rounds of four
 * independent 32x32x16 bf16 MFMAs on
 * hash-drawn operands, 4 * 32768 flops per wave and round.  Timed by the caller,
 * it gives the sustained MFMA rate of the card with random data, the ceiling
 * against which the attention kernels' rate is read.  out holds blocks * 256
 * floats (a checksum per lane).  SQUAD_ERR_INVALID_ARG for null out or sizes <= 0.
 */
int squad_debug_mfma_probe(float* out, int32_t blocks, int32_t iters, squad_stream_t stream);

/*
 * Host-only inspection of the address maps the kernels use (no device needed).
 * Writes, for every (batch, head, unit, row) in the kernels' enumeration order
 * [batch][heads][units][rows], the element offset that row occupies in the tensor:
 *   which = 0: local-pass rows in token order   (units = G windows, rows = Wn offsets)
 *   which = 1: global-pass rows in token order  (units = Wn offsets, rows = G windows)
 *   which = 2: local output in the group-major workspace (units = G, rows = Wn)
 *   which = 3: global-pass value rows in the workspace   (units = Wn, rows = G)
 * offsets must hold batch*heads*G*Wn entries (= batch*heads*n on whole tilings).
 * On a cut tiling, absent rows of the two token maps read -1 (the test the
 * kernels use to skip them).
 */
int squad_debug_row_offsets(int32_t which, const int32_t grid[3], const int32_t tile[3],
                            int32_t heads, int32_t batch, int32_t head_dim, int64_t* offsets);

#ifdef __cplusplus
}
#endif

#endif /* SQUAD_H */
