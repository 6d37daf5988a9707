/*
 * nabla.h -- C ABI of libnabla: NABLA (Neighborhood Adaptive Block-Level
 * Attention) self-attention for AMD Instinct MI355X (gfx950).
 *
 * Method sources (pages as titled; sections named):
 *   [GZ] "NABLA: Neighborhood Adaptive Block-Level Attention", gist.science
 *        (Chinese), technical summary, section "Methodology: NABLA".
 *   [LS] lsdiaocha.cn article on NABLA (Sber AI), section 2 (core
 *        innovations), section 4 (technical principles), section 5
 *        (comparison with existing techniques).
 *
 * One call of the method, in order:
 *   nabla_flatten     token reordering into P x P patches        [GZ] token reordering
 *   nabla_pool        average-pool Q and K into block delegates   [GZ] downsampling
 *   nabla_mask        reduced softmax map, CDF cut, STA union      [GZ] reduced attention,
 *                                                                  CDF thresholding, hybrid STA
 *   nabla_compact     per-head compressed (CSR) kept-block lists   [LS] sec. 5
 *   nabla_attn_fwd    exact attention on kept N x N token blocks   [GZ] expansion; [LS] sec. 2
 *   nabla_transpose_v V in the per-block transposed operand layout
 *   nabla_attn_fwd_vt nabla_attn_fwd reading that layout (faster)
 *   nabla_dense_attn_fwd  full attention (the baseline)   [GZ] experimental results 1
 *   nabla_qkv_split   QKV projection output -> q, k, V^T and block means
 *   nabla_unflatten   inverse reorder of the output
 *   nabla_mask_build  pool + mask + compact in one call (same outputs)
 *   nabla_forward     mask_build -> (transpose_v) -> attn_fwd in one call
 *   nabla_forward_noalloc  the same on a library-owned scratch array
 *
 * Gradients with the kept-block mask held fixed (training with NABLA:
 * [GZ] core contributions and experimental results 2, pre-training;
 * [LS] sec. 3):
 *   nabla_attn_fwd_lse / nabla_attn_fwd_vt_lse   forward that also writes the
 *                     log-sum-exp of every query's scores
 *   nabla_mask_transpose  key-major (transposed) mask, compacted by nabla_compact
 *   nabla_attn_bwd_dq     dQ and D = rowsum(dO * O), query-block lists
 *   nabla_attn_bwd_dkdv   dK and dV, key-block (transposed) lists
 *
 * Conventions for every entry point
 *   - All pointers except `geom`, `sta` and `bytes`/`offsets` outputs are
 *     DEVICE pointers, allocated and owned by the caller.  The library
 *     allocates no memory and keeps no state between calls apart from the
 *     thread-local last HIP error and, for nabla_forward_noalloc, its
 *     static per-GPU scratch array and that array's device address.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; it never synchronizes.
 *   - Return value: NABLA_OK (0) or a negative NABLA_E_* code.  All argument
 *     checks run before anything is enqueued: a call that returns an error
 *     has launched nothing.  A failed launch returns NABLA_E_HIP and keeps the
 *     hipError_t for nabla_last_hip_error().  No call aborts or throws.
 *   - batch == 0 or heads == 0 is a valid empty call: NABLA_OK, no launch.
 *
 * Geometry and layouts
 *   The latent is T x H x W tokens (valid extents).  Blocks are P x P spatial
 *   patches of one frame, P = 8, so a block holds N = P*P = 64 tokens.
 *   H and W are padded up to Hp, Wp (multiples of P); the block grid is
 *   T x (Hp/P) x (Wp/P) and nb = T * (Hp/P) * (Wp/P).  Block b has frame
 *   t = b / ((Hp/P)(Wp/P)), block row hb and block column wb (row-major);
 *   slot s of the block is patch row s / P and patch column s % P.
 *
 *   NABLA_LAYOUT_THW:     tensor [B, heads, T, H, W, d]  (natural order,
 *                         valid tokens only; the reorder is applied inside
 *                         the kernels' address computation)
 *   NABLA_LAYOUT_BLOCKED: tensor [B, heads, nb, 64, d]   (already flattened;
 *                         pad slots present in memory and ignored on input)
 *   Q, K, V and O of one call share one layout, contiguous; Q, K, V share
 *   `dtype` and O has `out_dtype`.
 *   Pooled queries qbar: float32 [B, heads, nb, d] (row c = block c).
 *   Pooled keys kbar: 3 * nb16 * d bf16 values per head, [B, heads] heads
 *        in a row, nb16 = 16 * ceil(nb / 16).  Each float32 mean x is held
 *        exactly as three bf16 parts h = bf16(x), m = bf16(x - h),
 *        l = bf16(x - h - m) (round to nearest even; the two differences are
 *        exact in float32 and l equals the last one, so h + m + l == x, and
 *        (h + m) + l evaluated in float32 gives x back).  The parts sit in the
 *        mask kernel's matrix-core operand order: part p of block 16 j + i,
 *        channel c at bf16 offset
 *        (((j * (d / 32) + c / 32) * 3 + p) * 64 + ((c / 8) % 4) * 16 + i) * 8 + c % 8,
 *        so that each 16-byte-per-lane load of a wavefront is 1 KB contiguous.
 *        Rows past nb are ignored on input and left unwritten on output.
 *   Masks: uint32 [B, heads, nb, nw], nw = ceil(nb / 32); block c of row r is
 *   kept iff bit (c % 32) of word (c / 32) is set.  Bits >= nb are zero.
 *   Row counts: int32 [B, heads, nb].
 *   CSR: row_ptr int32 [B*heads, nb + 1] (offsets inside that head's list);
 *        col_idx int32 [B*heads, nb * nb] capacity; head i's list starts at
 *        col_idx + i * nb * nb; kept block indices of a row are ascending.
 *   V^T (bf16 only): [B, heads, nb, d, 64]; row c of block b holds channel c
 *        of the block's 64 key slots, in the order that swaps bits 2 and 3 of
 *        the slot index (positions 0-3, 4-7, 8-11, 12-15 of every 16 hold
 *        slots 0-3, 8-11, 4-7, 12-15); pad slots are zero.
 */
#ifndef NABLA_H
#define NABLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NABLA_ABI_VERSION 5

enum nabla_status {
  NABLA_OK = 0,
  NABLA_E_NULL = -1,        /* a required pointer is NULL */
  NABLA_E_SHAPE = -2,       /* batch/heads < 0, T/H/W < 1, or sizes overflow the limits */
  NABLA_E_DTYPE = -3,       /* dtype / out_dtype not supported (see nabla_geom) */
  NABLA_E_HEAD_DIM = -4,    /* head_dim not 64 or 128 */
  NABLA_E_PATCH = -5,       /* P != 8 */
  NABLA_E_THR = -6,         /* thr not in (0, 1] (or 0 without STA), or not finite */
  NABLA_E_STA = -7,         /* STA window not all-zero or all positive odd */
  NABLA_E_WORKSPACE = -8,   /* workspace smaller than nabla_forward_workspace_size */
  NABLA_E_LAYOUT = -9,      /* layout not NABLA_LAYOUT_THW / NABLA_LAYOUT_BLOCKED */
  NABLA_E_HIP = -10,        /* a HIP launch failed; see nabla_last_hip_error() */
  NABLA_E_SCALE = -11,      /* softmax scale not finite and > 0 */
  NABLA_E_TOO_LARGE = -12   /* nb above NABLA_MAX_BLOCKS */
};

enum nabla_dtype { NABLA_DTYPE_F32 = 0, NABLA_DTYPE_BF16 = 1 };
enum nabla_layout { NABLA_LAYOUT_THW = 0, NABLA_LAYOUT_BLOCKED = 1 };

/* Largest number of blocks per head (the mask kernel keeps one row of
 * nb scores in registers across a wavefront). */
#define NABLA_MAX_BLOCKS 4096

typedef struct nabla_geom {
  int64_t batch;     /* B >= 0 */
  int64_t heads;     /* heads >= 0 */
  int32_t T, H, W;   /* valid latent extents, each >= 1 */
  int32_t P;         /* patch side; must be 8 */
  int32_t head_dim;  /* d: 64 or 128 */
  int32_t dtype;     /* enum nabla_dtype: element type of Q, K, V */
  int32_t layout;    /* enum nabla_layout: layout of Q, K, V, O */
  int32_t out_dtype; /* enum nabla_dtype: element type of O; float32 inputs
                        need float32 output, bf16 inputs may write either (the
                        bf16 output is the float32 result rounded once, RNE) */
} nabla_geom;

/* Number of blocks per head, nb (see Geometry above). */
int nabla_num_blocks(const nabla_geom* geom, int64_t* nb);

/* Fractal flatten ([GZ] Methodology, token reordering): every P x P spatial
 * patch of a frame becomes one contiguous run of 64 tokens, patches in
 * row-major order over the frame, frames in temporal order.
 * x: [B, heads, T, H, W, d] (geom->layout is ignored) -> x_blocked:
 * [B, heads, nb, 64, d]; pad slots are written as zeros.  Bit-exact copy. */
int nabla_flatten(const nabla_geom* geom, const void* x, void* x_blocked, void* stream);

/* Inverse of nabla_flatten on valid slots: [B, heads, nb, 64, d] ->
 * [B, heads, T, H, W, d].  Bit-exact copy. */
int nabla_unflatten(const nabla_geom* geom, const void* x_blocked, void* x, void* stream);

/* Block average pooling of Q and K ([GZ] Methodology, downsampling;
 * [LS] sec. 2 and 4): qbar[b, h, c, :] = mean of the valid tokens of block c,
 * accumulated in float32, and the same for kbar in its split, tiled encoding
 * (see the layouts above).  q, k in geom's layout and dtype. */
int nabla_pool(const nabla_geom* geom, const void* q, const void* k,
               float* qbar, void* kbar, void* stream);

/* Adaptive block mask ([GZ] Methodology, reduced attention + CDF
 * thresholding + hybrid integration with STA).  For every row r of every
 * head: s_c = qbar_r . kbar_c * (1 / sqrt(d)) to float32 accuracy (six
 * bf16 products of the three-part splits of qbar and kbar, float32
 * accumulation), p = softmax(s);
 * the kept set is the smallest set of blocks taken in order of decreasing p
 * (ties: lower block index first) whose total probability reaches thr
 * (thr = 1 keeps every block).  If sta = {wt, wh, ww} is non-zero, every
 * block within wt/2 frames, wh/2 block rows and ww/2 block columns of the
 * row's own block is added (window clipped at the borders).
 *   thr            in (0, 1]; 0 turns the adaptive part off, which leaves
 *                  the pure STA window ([GZ] experimental results 3, the
 *                  static baseline) and needs a non-zero sta
 *   sta            host array of 3 ints; NULL or {0,0,0} = no STA;
 *                  otherwise three positive odd numbers
 *   mask_bits      out, uint32 [B, heads, nb, nw]: union mask
 *   row_count      out, int32 [B, heads, nb]: kept blocks per row (union)
 *   adaptive_bits  optional out (may be NULL), uint32 [B, heads, nb, nw]:
 *                  the CDF-threshold mask before the STA union */
int nabla_mask(const nabla_geom* geom, const float* qbar, const void* kbar,
               float thr, const int32_t* sta, uint32_t* mask_bits,
               int32_t* row_count, uint32_t* adaptive_bits, void* stream);

/* Compressed kept-block lists ([LS] sec. 5, storing only the compressed
 * sparse matrix): per head, row_ptr = exclusive prefix sum of row_count and
 * col_idx = the kept block indices of each row in ascending order.
 * mask_bits, row_count as produced by nabla_mask; row_ptr int32
 * [B*heads, nb + 1]; col_idx int32 with capacity B*heads*nb*nb. */
int nabla_compact(const nabla_geom* geom, const uint32_t* mask_bits,
                  const int32_t* row_count, int32_t* row_ptr, int32_t* col_idx,
                  void* stream);

/* Mask construction in one call: nabla_pool, nabla_mask and nabla_compact
 * in that order on `stream` ([GZ] Methodology, downsampling + reduced
 * attention + CDF thresholding + hybrid integration with STA; [LS] sec. 5,
 * compressed storage).  Writes exactly what those three calls write, bit for
 * bit: qbar, kbar, mask_bits, row_count, adaptive_bits (optional, may be
 * NULL), row_ptr and col_idx, with the shapes given there; q, k in geom's
 * layout and dtype; thr and sta as for nabla_mask.  Arguments are checked
 * before anything is enqueued.  No workspace. */
int nabla_mask_build(const nabla_geom* geom, const void* q, const void* k, float thr,
                     const int32_t* sta, float* qbar, void* kbar, uint32_t* mask_bits,
                     int32_t* row_count, uint32_t* adaptive_bits, int32_t* row_ptr,
                     int32_t* col_idx, void* stream);

/* Block-sparse attention forward ([GZ] Methodology, expansion of the block
 * mask to token resolution; [LS] sec. 2, step 3): for each valid query token
 * i of block r, o_i = sum_j softmax_j(q_i . k_j * scale) v_j over the valid
 * key tokens j of the kept blocks listed for row r.  bf16 inputs use bf16
 * matrix cores with float32 accumulation and a float32 online softmax;
 * float32 inputs compute in float32.  q, k, v in geom's layout and dtype, o
 * in geom's layout and out_dtype;
 * in NABLA_LAYOUT_BLOCKED pad query slots of o are written as zeros.  A row
 * with an empty list produces zeros.  scale > 0 (usually 1/sqrt(d)).
 * col_idx entries must lie in [0, nb); the kernels do not fault on bad lists:
 * an entry outside [0, nb) is skipped, and a row whose pointers are negative,
 * decreasing or past nb * nb is treated as empty. */
int nabla_attn_fwd(const nabla_geom* geom, const void* q, const void* k,
                   const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                   float scale, void* o, void* stream);

/* V in the V^T layout above (bf16 inputs only): the attention kernel reads
 * it as matrix-core operands with plain 16-byte loads instead of transposing
 * V on chip.  v in geom's layout; vt [B, heads, nb, d, 64].  Bit-exact copy. */
int nabla_transpose_v(const nabla_geom* geom, const void* v, void* vt, void* stream);

/* nabla_attn_fwd with V given as nabla_transpose_v's output (bf16 inputs
 * only).  Same arguments otherwise; the result is bit-identical to
 * nabla_attn_fwd's. */
int nabla_attn_fwd_vt(const nabla_geom* geom, const void* q, const void* k,
                      const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                      float scale, void* o, void* stream);

/* Layout pass after a transformer layer's fused QKV projection, for a
 * network that keeps its token sequence in the blocked (fractal-flattened)
 * order throughout ([GZ] Methodology, token reordering and downsampling):
 * splits the projection output into the head-major tensors the other calls
 * take and computes the block means on the way, so no pooling or V
 * transpose pass of its own is needed.  geom: layout NABLA_LAYOUT_BLOCKED
 * (NABLA_E_LAYOUT otherwise), dtype bf16 (NABLA_E_DTYPE otherwise).
 *   qkv        bf16 [B, nb * 64, 3, heads, d]: for every token of the blocked
 *              order (pad slots included) its q, k and v rows of every head
 *   q, k       out, bf16 [B, heads, nb * 64, d]: copies, blocked layout
 *   vt         out, bf16 [B, heads, nb, d, 64]: as nabla_transpose_v of v
 *   qbar, kbar out, layouts as for nabla_pool: bit-identical to nabla_pool
 *              of q and k (means over the valid tokens; pad slots ignored)
 * Bit-exact otherwise. */
int nabla_qkv_split(const nabla_geom* geom, const void* qkv, void* q, void* k,
                    void* vt, float* qbar, void* kbar, void* stream);

/* Dense (full) attention, the baseline that the method's speed-ups are
 * measured against ([GZ] experimental results 1, speed-up over full
 * attention; [LS] sec. 3, generation time against full attention): every
 * valid query attends to every valid key of its head, with no mask and no
 * kept lists.  bf16 inputs only (NABLA_E_DTYPE otherwise); q, k in geom's
 * layout, vt from nabla_transpose_v; o in geom's layout and out_dtype; lse
 * optional (may be NULL), float32 [B, heads, nb, 64] as for
 * nabla_attn_fwd_lse.  Equal, up to float rounding order, to nabla_attn_fwd
 * on the all-kept mask. */
int nabla_dense_attn_fwd(const nabla_geom* geom, const void* q, const void* k,
                         const void* vt, float scale, void* o, float* lse, void* stream);

/* Gradients ([GZ] core contributions, "dual-stage acceleration" of training
 * and inference, and experimental results 2, pre-training a 2B DiT with
 * NABLA; [LS] sec. 3).  The kept-block mask is a threshold on pooled scores,
 * so it is held fixed and only the exact attention over the kept blocks is
 * differentiated: with p = softmax(q k^T * scale) over the kept valid keys,
 * o = p v and incoming gradient dO,
 *   dV = p^T dO,  dP = dO V^T,  dS = p (dP - D),  D = rowsum(dO * o),
 *   dQ = dS K * scale,  dK = dS^T Q * scale.
 * Shared conventions: lse and delta are float32 [B, heads, nb, 64], indexed by
 * block and slot (slot = row-in-patch * 8 + column-in-patch) whatever the
 * tensor layout; the gradient calls need geom->out_dtype == geom->dtype
 * (NABLA_E_DTYPE otherwise), and o, dout, dq, dk, dv are in geom's layout and
 * dtype.  Pad slots of dq, dk, dv are not written in the THW layout and are
 * written as zeros in the blocked layout.  bf16 inputs use bf16 matrix cores
 * with float32 accumulation; float32 inputs compute in float32. */

/* nabla_attn_fwd that also writes lse[b, h, c, slot] = ln sum_j exp(s_j),
 * s_j = q . k_j * scale over the query's kept valid keys (-inf for pad slots
 * and for rows with no keys).  lse must not be NULL. */
int nabla_attn_fwd_lse(const nabla_geom* geom, const void* q, const void* k,
                       const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                       float scale, void* o, float* lse, void* stream);

/* nabla_attn_fwd_vt with the lse output of nabla_attn_fwd_lse (bf16 only). */
int nabla_attn_fwd_vt_lse(const nabla_geom* geom, const void* q, const void* k,
                          const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                          float scale, void* o, float* lse, void* stream);

/* Transposed mask: bit r of mask_bits_t[b, h, c, :] = bit c of
 * mask_bits[b, h, r, :], i.e. row c lists the query blocks that keep key
 * block c; row_count_t[b, h, c] = its number of set bits.  Shapes as
 * mask_bits / row_count.  nabla_compact on the result gives the key-major
 * lists (col_ptr, row_idx) of nabla_attn_bwd_dkdv.  Bit-exact. */
int nabla_mask_transpose(const nabla_geom* geom, const uint32_t* mask_bits,
                         uint32_t* mask_bits_t, int32_t* row_count_t, void* stream);

/* dq and delta (D) from q, k, v, the forward's o and lse, and dout, over the
 * query-major lists (row_ptr, col_idx) of the forward. */
int nabla_attn_bwd_dq(const nabla_geom* geom, const void* q, const void* k,
                      const void* v, const void* o, const void* dout, const float* lse,
                      const int32_t* row_ptr, const int32_t* col_idx, float scale,
                      void* dq, float* delta, void* stream);

/* dk and dv over the key-major lists (col_ptr [B*heads, nb+1], row_idx
 * [B*heads, nb*nb]) of the transposed mask; delta from nabla_attn_bwd_dq
 * (so this call follows it on the stream). */
int nabla_attn_bwd_dkdv(const nabla_geom* geom, const void* q, const void* k,
                        const void* v, const void* dout, const float* lse,
                        const float* delta, const int32_t* col_ptr, const int32_t* row_idx,
                        float scale, void* dk, void* dv, void* stream);

/* Workspace for nabla_forward and the byte offsets of its parts, in order:
 * offsets[0] qbar, [1] kbar, [2] mask_bits, [3] row_count, [4] row_ptr,
 * [5] col_idx, [6] V^T (bf16 inputs; empty for float32) (see the layouts
 * above); `offsets` (host, 7 entries) may be NULL.  Every part is 256-byte
 * aligned. */
int nabla_forward_workspace_size(const nabla_geom* geom, size_t* bytes, size_t* offsets);

/* One NABLA attention call: nabla_mask_build (pooling, mask, lists) and the
 * attention (bf16: nabla_transpose_v + nabla_attn_fwd_vt; float32:
 * nabla_attn_fwd) in sequence on `stream`, with the intermediates in
 * `workspace` (device memory of at least nabla_forward_workspace_size bytes,
 * caller-owned; its parts can be read back after the call). */
int nabla_forward(const nabla_geom* geom, const void* q, const void* k, const void* v,
                  float thr, const int32_t* sta, float scale, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);

/* nabla_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as nabla_forward, minus the workspace: the call
 * uses a library-owned device array of NABLA_NOALLOC_SCRATCH_BYTES, one copy
 * per GPU, created with the library's code on that GPU and held until the
 * process ends, and allocates nothing.  Heads are processed in passes of as
 * many heads as that array holds (the parts listed for
 * nabla_forward_workspace_size, per pass), so the outputs equal
 * nabla_forward's bit for bit.  Its device address is looked up on the first
 * call on each device.  No part of the array needs to start at zero.
 * Every call on one GPU shares that GPU's array and leaves its contents to
 * the next: calls that overlap on one GPU (other streams, other threads)
 * race, so serialize them.  Returns NABLA_E_WORKSPACE if one head's parts
 * exceed the array (not reached below NABLA_MAX_BLOCKS at head_dim <= 128),
 * other statuses as nabla_forward. */
#define NABLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int nabla_forward_noalloc(const nabla_geom* geom, const void* q, const void* k,
                          const void* v, float thr, const int32_t* sta, float scale,
                          void* o, void* stream);

/* Human-readable text of a status code (static storage). */
const char* nabla_status_string(int status);

/* hipError_t of the last failed launch in this thread (0 if none). */
int nabla_last_hip_error(void);

/* NABLA_ABI_VERSION of the library. */
int nabla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NABLA_H */
