/*
 * lora_mi355x.h -- C ABI of the routed multi-LoRA projection library for
 * AMD MI355X (CDNA4, gfx950).
 *
 * The method (ferrox-core "weight_matrix/lora.rs", module doc):
 *
 *     y_i = W x_i + s_{slot(i)} * B_{slot(i)} (A_{slot(i)} x_i)
 *
 * for a batch of rows, each row naming an adapter slot of a pool through a
 * per-row seq_slot buffer (atlas "spark_model/layers/ops/lora_delta.rs",
 * apply_lora_bgmv doc).  The low-rank term runs as a shrink t = A x
 * (rank-sized) and an expand-and-fold y += s * B t (same page, kernels 1
 * and 2 of apply_lora_bgmv).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Ownership: the caller owns every buffer.  The library never allocates,
 *    frees or synchronises, and never reads device memory on the host, so
 *    every call is a sequence of kernel launches on `stream` (a hipStream_t;
 *    NULL = the default stream) and may be captured into a HIP graph.
 *    Device-pointer arguments are marked [dev], host-pointer ones [host].
 *  - Layout: every matrix is row-major with unit stride along its last
 *    index.  Row strides are in ELEMENTS, not bytes.  W is [n_out][k_in]
 *    (row stride w_row_stride >= k_in); x is [n][x_row_stride >= k_in];
 *    y is [n][y_row_stride >= n_out].  A slot's A is [max_rank][k_in] and
 *    its B is [n_out][max_rank] (row stride max_rank), both zero-padded
 *    from the true rank to the pool's max_rank (atlas LoraPair doc: pad rows
 *    of A and pad columns of B are zero, so running at max_rank equals the
 *    true-rank product).
 *  - dtype: LORA_F32 (W, A, B, x, y all f32) or LORA_BF16 (W, A, B, x, y all
 *    bf16).  The scale table and the rank-sized intermediate t are f32 in
 *    both.  Accumulation is f32; a bf16 y is rounded once, to nearest even.
 *  - LORA_BF16 additionally needs k_in, n_out, every row stride and
 *    max_rank to be multiples of 8 (max_rank a multiple of 16, at most 256)
 *    and every matrix pointer 16-byte aligned (128-bit loads and stores).
 *  - Route resolve (atlas apply_lora_bgmv doc; ferrox add_to): a row whose
 *    slot s is < 0, >= max_loras, whose a_table[s] or b_table[s] is NULL,
 *    or whose scale_table[s] is 0 gets NO delta arithmetic: its y equals
 *    the base W x bit for bit.  Slot values live in device memory and are
 *    never validated on the host; any value is defined by this rule.
 *  - Errors: every call returns LORA_OK (0) or a negative lora_status.
 *    Validation runs before any launch; on error nothing is launched and
 *    lora_last_error() returns a message naming every dimension involved
 *    (ferrox LoraShapeError does the same for a misfit pair).  A failed
 *    launch returns LORA_ERR_LAUNCH with the HIP error text.
 *  - Workspace: the fused entry points take a caller-owned device
 *    workspace of at least lora_workspace_bytes(...) bytes.  It must be
 *    zero-filled before its first use with a given problem shape (op,
 *    n_rows, n_out, k_in, n_groups); every call that returns LORA_OK leaves
 *    the words that must start at zero at zero again, so the same shape can
 *    be called again with no memset (none is recorded into a captured
 *    graph).  Those words sit at offsets that depend on the shape alone, so
 *    routed calls of any rank up to the sized max_rank and base-only calls
 *    of one shape may share a workspace (lora_workspace_bytes covers the
 *    base-only call too).  Reusing one workspace for another shape needs a
 *    new zero fill.  Concurrent calls sharing one workspace race.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1 };

enum lora_status {
  LORA_OK = 0,
  LORA_ERR_SHAPE = -1,       /* a dimension is zero, too large or inconsistent */
  LORA_ERR_NULL_PTR = -2,    /* a required pointer is NULL */
  LORA_ERR_STRIDE = -3,      /* a row stride is smaller than its row */
  LORA_ERR_DTYPE = -4,       /* unknown dtype, or route and call disagree */
  LORA_ERR_UNSUPPORTED = -5, /* shape/alignment outside what the kernels take */
  LORA_ERR_LAUNCH = -6,      /* a HIP launch failed, or the device is not gfx950 */
  LORA_ERR_WORKSPACE = -7    /* workspace missing or smaller than required */
};

enum lora_op {
  LORA_OP_APPLY = 0,
  LORA_OP_SEGMENTED = 1,
  LORA_OP_MOE_GATHER = 2,
  LORA_OP_MOE_GROUPED = 3,
  LORA_OP_STACK = 4
};

/*
 * A module's routing tables (atlas lora_delta.rs LoraRoute): load-time-fixed
 * [dev] arrays of max_loras entries.  a_table[s] -> A_s [max_rank][k_in],
 * b_table[s] -> B_s [n_out][max_rank]; NULL = base-only slot.  For a fused
 * projection split into parts (frink lora_attach.rs module doc: B's rows
 * split in order, one copy of A each) a part's b_table entries point at its
 * block of rows, B_s + row0 * max_rank.  scale_table[s] is read at apply
 * time (ferrox test the_scale_is_read_at_apply_time), so a caller may
 * rewrite it between calls.  The struct itself is [host].
 */
typedef struct lora_route {
  const void *const *a_table;   /* [dev] [max_loras] */
  const void *const *b_table;   /* [dev] [max_loras] */
  const float *scale_table;     /* [dev] [max_loras] */
  uint32_t max_loras;
  uint32_t k_in;
  uint32_t n_out;
  uint32_t max_rank;
  int32_t dtype;
} lora_route;

/*
 * MoE routing tables (atlas lora_delta.rs moe_lora_gather_bgmv field doc:
 * the expert is keyed through the per-slot indices array; the
 * moe_lora_grouped_down field doc: keyed through expert_offsets).  The pair
 * of (adapter a, expert e) sits at table index a * n_experts + e; the scale
 * is the adapter's, scale_table[a].
 */
typedef struct lora_route_moe {
  const void *const *a_table;   /* [dev] [max_loras * n_experts] */
  const void *const *b_table;   /* [dev] [max_loras * n_experts] */
  const float *scale_table;     /* [dev] [max_loras] */
  uint32_t max_loras;
  uint32_t n_experts;
  uint32_t k_in;
  uint32_t n_out;
  uint32_t max_rank;
  int32_t dtype;
} lora_route_moe;

/* ------------------------------------------------------------ host helpers */

/* Last error message of the calling thread ("" when none). */
const char *lora_last_error(void);

/* Library version string. */
const char *lora_version(void);

/*
 * Checks that the current HIP device is a gfx950 and caches its properties.
 * Called implicitly by every launching entry point; returns
 * LORA_ERR_LAUNCH (with the device's name) anywhere else.
 */
int lora_init(void);

/*
 * The LoRA scale (ferrox lora.rs module doc "Scale" and LoraDelta::new;
 * atlas LoraPair doc for rsLoRA): adapter_scale * alpha / rank, or
 * adapter_scale * alpha / sqrt(rank) when rslora != 0, or adapter_scale
 * alone when alpha == 0.  `rank` is the adapter's TRUE rank.  Computed in
 * double.
 */
double lora_scale(double adapter_scale, double alpha, uint32_t rank, int32_t rslora);

/*
 * The [max_loras] f32 scale table (metrale slot_math.rs scale_table_values):
 * entry k is lora_scale(...) of adapter k rounded once to f32, 0.0 for
 * k >= n_adapters.  All arrays [host]; out has max_loras entries.
 * Errors: NULL_PTR, SHAPE (rank 0).
 */
int lora_scale_table(uint32_t n_adapters, const double *adapter_scale, const double *alpha,
                     const uint32_t *rank, const int32_t *rslora, uint32_t max_loras,
                     float *out);

/*
 * The host seq_slot buffer (metrale slot_math.rs build_seq_slot_host): row
 * i < n takes adapter_slots[i] when it is >= 0 and `active` otherwise; rows
 * n..padded_n-1 are padding and take -1.  [host] arrays; out has padded_n
 * entries.  Errors: NULL_PTR, SHAPE (n > padded_n).
 */
int lora_build_seq_slot(const int32_t *adapter_slots, uint32_t n, uint32_t padded_n,
                        int32_t active, int32_t *out);

/*
 * Workspace bytes a fused entry point needs for this problem (0 for
 * LORA_F32, which needs none).  op is a lora_op; n_rows is n (apply,
 * segmented, MoE grouped, stack) or n_tokens * top_k (MoE gather);
 * n_groups is n_experts for the two MoE ops, the number of levels for a
 * stack and 1 otherwise; max_rank is 0 for a base-only call (for a stack,
 * the largest max_rank over its levels).  A stack needs workspace in
 * LORA_F32 too (the further levels' t).
 */
size_t lora_workspace_bytes(int32_t op, int32_t dtype, uint32_t n_rows, uint32_t n_out,
                            uint32_t k_in, uint32_t max_rank, uint32_t n_groups);

/*
 * Measurement aid (atlas lora_delta.rs lora_no_apply doc: apply cost is
 * measured apart from everything else).  With n >= 4 HIP events set, every
 * later fused call on the calling thread (lora_apply, lora_apply_segmented,
 * lora_apply_moe_gather, lora_apply_moe_grouped, lora_apply_stack,
 * lora_embed_rows) records on its stream events[0] before its first kernel, events[1] right before
 * its main kernel (after the route plan and shrink kernel where there is
 * one), events[2] right after the main kernel, and events[3] after its last
 * kernel (the decode epilogue, or a stack's further levels, where there are
 * any).  n == 0 switches it off.  events is [host]; the events themselves
 * are the caller's hipEvent_t.  Returns LORA_ERR_NULL_PTR for 0 < n < 4 or
 * a NULL event.
 */
int lora_set_profile_events(void *const *events, uint32_t n);

/* ------------------------------------------------------------ kernels */

/*
 * Shrink (atlas apply_lora_bgmv kernel 1; ferrox LoraDelta::project):
 *   t[i, 0:max_rank] = A_s x_i,  s = seq_slot[i],  for every row that
 * resolves to a slot.  Rows that skip are NOT written.  t is [dev] f32
 * [n][max_rank].  x [dev] [n][x_row_stride]; seq_slot [dev] int32 [n].
 * n == 0 launches nothing.
 */
int lora_shrink(const lora_route *route, const void *x, uint32_t x_row_stride,
                const int32_t *seq_slot, uint32_t n, float *t, void *stream);

/*
 * Expand and fold (atlas apply_lora_bgmv kernel 2; ferrox
 * LoraDelta::accumulate):  y[i, o] += scale_table[s] * (B_s t_i)[o] in
 * place, for every row that resolves to a slot; other rows are untouched.
 * The sum over the rank runs in f32; a bf16 y is rounded once from
 * f32(y) + s * dot.  t [dev] f32 [n][max_rank]; y [dev] [n][y_row_stride].
 */
int lora_expand_fold(const lora_route *route, const float *t, const int32_t *seq_slot,
                     uint32_t n, void *y, uint32_t y_row_stride, void *stream);

/*
 * Fused decode apply (the whole formula, ferrox lora.rs module doc):
 *   y_i = W x_i + s B_s (A_s x_i)   written (not accumulated), one rounding.
 * route == NULL (or every row skipping) gives the base-only output, bit
 * identical to the skipped rows of a routed call with the same shape.
 * W [dev] [n_out][w_row_stride]; x, seq_slot, y as above (seq_slot may be
 * NULL when route is NULL).  workspace [dev], see the conventions above.
 * Batches up to 64 rows take the one-launch decode kernel, larger ones the
 * tiled GEMM; n is limited to 16384 (LORA_ERR_SHAPE above).  The decode
 * kernel's workgroups wait for each other within the launch; should such a
 * wait ever give up (0.5 s, which only a device that cannot hold the
 * launch's first workgroups at once would reach), the tile's outputs are
 * written as NaN and the workspace must be zero-filled again.
 */
int lora_apply(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W,
               uint32_t w_row_stride, const lora_route *route, const void *x,
               uint32_t x_row_stride, const int32_t *seq_slot, uint32_t n, void *y,
               uint32_t y_row_stride, void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): lora_apply with no
 * workspace argument and the same results bit for bit.  Its intermediate
 * results live in a device array that the library owns, of
 * LORA_NOALLOC_SCRATCH_BYTES per GPU, held on each GPU it runs on until the
 * process ends; the call itself allocates nothing.  A problem that needs
 * more scratch than that (lora_workspace_bytes(LORA_OP_APPLY, ...) plus
 * 1 MiB gives the need) returns LORA_ERR_WORKSPACE and launches nothing.
 * Every call on one GPU uses that GPU's array and leaves what it wrote
 * there: calls that overlap in time on one GPU (other streams, other
 * threads) race; calls ordered on one stream do not.  The first call on a
 * GPU, and every call made while `stream` is being captured, first clears
 * the array's counter words with a small kernel on `stream`.  lora_init
 * looks the array up on the current device ahead of the first call.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)
int lora_apply_noalloc(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W,
                       uint32_t w_row_stride, const lora_route *route, const void *x,
                       uint32_t x_row_stride, const int32_t *seq_slot, uint32_t n, void *y,
                       uint32_t y_row_stride, void *stream);

/*
 * Segmented prefill apply (ferrox add_batch_to; atlas apply_lora_delta for
 * m contiguous rows on one pair): rows seg_indptr[g] .. seg_indptr[g+1]-1
 * use slot seg_slot[g]; otherwise the same definition as lora_apply.
 * seg_indptr [dev] int32 [n_seg+1], non-decreasing, seg_indptr[0] = 0;
 * seg_slot [dev] int32 [n_seg].  Rows outside every segment are not
 * written.  This is the MFMA (dense-contraction) entry point.
 */
int lora_apply_segmented(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W,
                         uint32_t w_row_stride, const lora_route *route, const void *x,
                         uint32_t x_row_stride, const int32_t *seg_indptr,
                         const int32_t *seg_slot, uint32_t n_seg, uint32_t n, void *y,
                         uint32_t y_row_stride, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * MoE expert down_proj with the routed delta, gathered by expert (atlas
 * lora_delta.rs moe_lora_gather_bgmv field doc).  Routing slot j (token
 * j / top_k, slot-major) uses expert e = indices[j] and adapter
 * a = token_slot[j / top_k]:
 *   y[j] = W_e x[j] + scale_table[a] B_{a,e} (A_{a,e} x[j]).
 * W_experts [dev]: expert e's [n_out][w_row_stride] matrix starts
 * e * expert_stride elements in.  x [dev] [n_tokens*top_k][x_row_stride];
 * indices [dev] int32 [n_tokens*top_k]; token_slot [dev] int32 [n_tokens];
 * y [dev] [n_tokens*top_k][y_row_stride].  Rows whose expert id is outside
 * [0, n_experts) are not written.  route may be NULL (base only).
 */
int lora_apply_moe_gather(int32_t dtype, uint32_t n_experts, uint32_t n_out, uint32_t k_in,
                          const void *W_experts, uint64_t expert_stride,
                          uint32_t w_row_stride, const lora_route_moe *route, const void *x,
                          uint32_t x_row_stride, const int32_t *indices, uint32_t top_k,
                          const int32_t *token_slot, uint32_t n_tokens, void *y,
                          uint32_t y_row_stride, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Grouped MoE layout (atlas lora_delta.rs moe_lora_grouped_down field doc:
 * the MoE expert down_proj delta keyed on expert through device
 * expert_offsets; the sorted twin of the gather above).  The n rows come
 * sorted by expert: rows expert_offsets[e] .. expert_offsets[e+1]-1 belong
 * to expert e.  Each sorted row carries its own adapter slot, seq_slot[j]
 * (the slot of the token it was routed from), resolved by the rule of the
 * conventions above with the pair (a = seq_slot[j], e) at table index
 * a * n_experts + e.  expert_offsets [dev] int32 [n_experts+1] must be
 * non-decreasing; it lives in device memory and is not validated on the
 * host.  A row outside [expert_offsets[0], expert_offsets[n_experts]) is
 * not written (and its x row is not read).  With offsets that decrease,
 * every access still stays inside the operands (each row maps to at most
 * one expert by a binary search) but which expert a row gets is
 * unspecified.  seq_slot [dev] int32 [n].
 */

/* Grouped shrink: t[j, 0:max_rank] = A_{a,e} x[j] for rows that resolve;
 * other rows of t are not written.  x [dev] [n][x_row_stride]; t [dev] f32
 * [n][max_rank]. */
int lora_moe_grouped_shrink(const lora_route_moe *route, const void *x, uint32_t x_row_stride,
                            const int32_t *expert_offsets, const int32_t *seq_slot, uint32_t n,
                            float *t, void *stream);

/* Grouped expand and fold: y[j, o] += scale_table[a] * (B_{a,e} t[j])[o] in
 * place for rows that resolve; every other row is untouched.  The rank sum
 * runs in f32; a bf16 y is rounded once.  t [dev] f32 [n][max_rank]; y
 * [dev] [n][y_row_stride]. */
int lora_moe_grouped_expand_fold(const lora_route_moe *route, const float *t,
                                 const int32_t *expert_offsets, const int32_t *seq_slot,
                                 uint32_t n, void *y, uint32_t y_row_stride, void *stream);

/* Fused grouped apply: y[j] = W_e x[j] + scale_table[a] B_{a,e} (A_{a,e} x[j])
 * written with one rounding, e the expert whose range holds j.  W_experts
 * as in lora_apply_moe_gather; x [dev] [n][x_row_stride]; y [dev]
 * [n][y_row_stride]; workspace [dev] (op LORA_OP_MOE_GROUPED, n_rows n,
 * n_groups n_experts).  route may be NULL (base only; seq_slot may then be
 * NULL).  n is limited to 16384 rows. */
int lora_apply_moe_grouped(int32_t dtype, uint32_t n_experts, uint32_t n_out, uint32_t k_in,
                           const void *W_experts, uint64_t expert_stride, uint32_t w_row_stride,
                           const lora_route_moe *route, const void *x, uint32_t x_row_stride,
                           const int32_t *expert_offsets, const int32_t *seq_slot, uint32_t n,
                           void *y, uint32_t y_row_stride, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Token-embedding pair into the one layout (ferrox lora.rs module doc
 * "Layouts": an embedding adapter is stored flipped, because the graph
 * gathers a row per token; frink lora_attach.rs checked_pair, embedding
 * branch).  The file's A_file is [n_vocab][rank] and its B_file
 * [n_embd][rank]; in the one layout B is A_file unchanged and
 * a_out [rank][n_embd] = B_file transposed.  All arrays [host], row-major,
 * dtype elements.  Errors: SHAPE (naming all six dimensions) unless
 * a_rows == n_vocab, b_rows == n_embd and a_cols == b_cols >= 1; NULL_PTR.
 * Pure host code: no HIP call.
 */
int lora_embedding_pair(int32_t dtype, uint32_t n_vocab, uint32_t n_embd, uint32_t a_rows,
                        uint32_t a_cols, const void *a_file, uint32_t b_rows, uint32_t b_cols,
                        const void *b_file, void *a_out);

/*
 * Token-embedding row gather with the routed delta (ferrox lora.rs
 * LoraDelta::add_row_to: the delta of one row of the adapted matrix, which
 * a row gather needs):
 *   y[i, :] = E[t, :] + scale_table[s] * (B_s[t, :] A_s),
 *   t = token_ids[i], s = seq_slot[i],
 * with the route in the one layout: route->k_in = n_embd (A_s is
 * [max_rank][n_embd]), route->n_out = n_vocab (B_s is [n_vocab][max_rank]).
 * A row whose slot skips gets E[t, :] bit for bit; a row whose token lies
 * outside [0, n_vocab) is not written (token values live in device memory
 * and are not validated on the host).  The rank sum runs in f32 and a bf16
 * y is rounded once.  E [dev] [n_vocab][e_row_stride]; token_ids, seq_slot
 * [dev] int32 [n]; y [dev] [n][y_row_stride >= n_embd].  route may be NULL
 * (a plain gather; seq_slot may then be NULL).  No workspace.  bf16 needs
 * n_embd and both strides to be multiples of 8 and 16-byte aligned E and y.
 */
int lora_embed_rows(int32_t dtype, uint32_t n_vocab, uint32_t n_embd, const void *E,
                    uint32_t e_row_stride, const lora_route *route, const int32_t *token_ids,
                    const int32_t *seq_slot, uint32_t n, void *y, uint32_t y_row_stride,
                    void *stream);

/*
 * Adapter stack (ferrox lora.rs LoraStack and module doc: every adapter
 * attached to one base matrix is a term of W x + sum_i s_i B_i (A_i x),
 * applied in order):
 *   y_i = W x_i + sum over levels l = 0 .. n_levels-1 of
 *         scale_l[s] B_{l,s} (A_{l,s} x_i),   s = seq_slots[l][i],
 * each level resolved by the rule of the conventions above (a level whose
 * slot skips adds nothing to the row).  routes is a [host] array of
 * n_levels route descriptors, all of shape [n_out x k_in] and dtype;
 * seq_slots is a [host] array of n_levels [dev] int32 [n] buffers.  At most
 * 8 levels; n_levels == 0 is the base-only output.  Rounding: the first
 * level runs through the fused apply (y rounded once); the further levels'
 * terms are summed in f32 and added to y with one more rounding, so a bf16
 * y is rounded at most twice whatever the depth.  workspace [dev] of at
 * least lora_workspace_bytes(LORA_OP_STACK, dtype, n, n_out, k_in, largest
 * max_rank, n_levels) bytes, zero-filled before its first use with a shape.
 * Decode-shaped batches are the target; n is limited to 16384.
 */
int lora_apply_stack(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W,
                     uint32_t w_row_stride, const lora_route *routes,
                     const int32_t *const *seq_slots, uint32_t n_levels, const void *x,
                     uint32_t x_row_stride, uint32_t n, void *y, uint32_t y_row_stride,
                     void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
