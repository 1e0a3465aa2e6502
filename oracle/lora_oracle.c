/*
 * lora_oracle.c -- plain fp64 CPU oracle for the routed multi-LoRA projection
 *
 *     y_i = W x_i + s_{slot(i)} * B_{slot(i)} (A_{slot(i)} x_i)
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP
 * library: every step below is written out from the pages' definitions.
 *
 * Arithmetic: every stored value (f32, or bf16 bit patterns) is widened
 * exactly to double; products of two widened values are exact in double;
 * every sum runs sequentially in ascending index order.  Build without
 * -ffast-math and with -ffp-contract=off.  OpenMP may split work over rows
 * only; each output element is produced by one thread with one fixed order,
 * so results do not depend on the thread count.
 *
 * Sources (page title, then the item):
 *  - ferrox-core "weight_matrix/lora.rs": module doc (the formula, layouts,
 *    scale, "cost when absent"), LoraDelta::new / effective_scale / project /
 *    accumulate / add_to / add_batch_to / add_row_to (the token-embedding
 *    row gather), LoraStack (adapters applied in order).
 *  - frink-models "lora_attach.rs": module doc (fused-tensor split: one copy
 *    of A per part, B rows split in order).
 *  - atlas "spark_model/layers/ops/lora_delta.rs": LoraRoute, LoraPair
 *    (rank padding, scale alpha/r or alpha/sqrt(r)), apply_lora_bgmv doc
 *    (seq_slot < 0 = base; NULL/0 table entries = base-only slot), the
 *    moe_lora_gather_bgmv field doc (expert keyed through indices), the
 *    moe_lora_grouped_down field doc (expert keyed through expert_offsets).
 *  - metrale "lora/slot_math.rs": build_seq_slot_host, scale_table_values.
 *
 * Readings where the pages leave a step open are listed with each function.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

#ifndef ORC_MUTANT
#define ORC_MUTANT 0 /* planted-mistake builds for the pin-strength tests */
#endif

/* ------------------------------------------------------------------ values */

/* Exact widening of one stored element to double. */
static double widen(const void *base, int dtype, size_t idx) {
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------ scale */

/*
 * ferrox lora.rs module doc "Scale" and LoraDelta::new / effective_scale:
 *   scale = adapter_scale * alpha / rank   if alpha != 0
 *         = adapter_scale                  if alpha == 0
 * atlas lora_delta.rs LoraPair doc and metrale slot_math.rs
 * scale_table_values: alpha / sqrt(r) under rsLoRA.
 * Reading: rsLoRA keeps the adapter_scale factor and the alpha == 0 rule;
 * `rank` is always the TRUE rank, never the pool's padded max_rank.
 */
double orc_scale(double adapter_scale, double alpha, int rank, int rslora) {
#if ORC_MUTANT == 2
  if (alpha == 0.0) return 1.0;
#else
  if (alpha == 0.0) return adapter_scale;
#endif
#if ORC_MUTANT == 1
  if (rslora) return adapter_scale * alpha / (double)rank;
#else
  if (rslora) return adapter_scale * alpha / sqrt((double)rank);
#endif
  return adapter_scale * alpha / (double)rank;
}

/*
 * metrale slot_math.rs scale_table_values: entry k is adapter k's scale,
 * 0.0 for k >= the number of adapters.  Each entry is the fp64 formula
 * rounded once to f32 (the table is f32 device memory in atlas LoraRoute).
 */
void orc_scale_table(int n_adapters, const double *adapter_scale, const double *alpha,
                     const int *rank, const int *rslora, int max_loras, float *out) {
  for (int k = 0; k < max_loras; ++k) {
    if (k < n_adapters)
      out[k] = (float)orc_scale(adapter_scale[k], alpha[k], rank[k], rslora[k]);
    else
#if ORC_MUTANT == 9
      out[k] = 1.0f;
#else
      out[k] = 0.0f;
#endif
  }
}

/*
 * metrale slot_math.rs build_seq_slot_host: row i < n takes adapter_slots[i]
 * when it is >= 0 and `active` otherwise; rows n..padded_n-1 are padding and
 * take -1 ("no delta").
 */
void orc_build_seq_slot(const int32_t *adapter_slots, int n, int padded_n, int active,
                        int32_t *out) {
  for (int i = 0; i < padded_n; ++i) {
    if (i < n) {
#if ORC_MUTANT == 7
      out[i] = adapter_slots[i];
#else
      out[i] = adapter_slots[i] >= 0 ? adapter_slots[i] : active;
#endif
    } else {
#if ORC_MUTANT == 6
      out[i] = active;
#else
      out[i] = -1;
#endif
    }
  }
}

/* ------------------------------------------------------------------ route */

/*
 * atlas lora_delta.rs LoraRoute: [max_loras] tables of A / B pointers (NULL
 * = base-only slot) and a [max_loras] f32 scale table.  Here the tables are
 * host pointers.  For the MoE gather the pair of (adapter a, expert e) sits
 * at table index a * n_experts + e and the scale is the adapter's.
 */
typedef struct {
  const void *const *a;  /* [max_loras * n_experts] -> A [max_rank][k_in] */
  const void *const *b;  /* [max_loras * n_experts] -> B [n_out][max_rank] */
  const float *scale;    /* [max_loras] */
  int max_loras;
  int n_experts;         /* 1 for a dense projection */
  int k_in, n_out, max_rank, dtype;
} orc_route;

/*
 * Step a1, route resolve.  atlas apply_lora_bgmv doc: seq_slot < 0 means
 * base; a NULL table entry or a 0 scale is a base-only slot.  ferrox add_to:
 * a zero scale is skipped before any arithmetic.  Reading: a slot >=
 * max_loras is skipped too.  Returns the table index, or -1 to skip.
 */
static int resolve(const orc_route *r, int slot, int expert) {
  if (r == NULL) return -1;
  if (slot < 0 || slot >= r->max_loras) return -1;
  int idx = slot * r->n_experts + expert;
#if ORC_MUTANT == 10
  if (r->n_experts > 1) idx = expert * r->max_loras + slot;
  if (idx >= r->max_loras * r->n_experts) return -1;
#endif
  if (r->a[idx] == NULL || r->b[idx] == NULL) return -1;
  if (r->scale[slot] == 0.0f) return -1;
  return idx;
}

/* ferrox LoraDelta::project: t[k] = A[k,:] . x for k < max_rank (padded
 * rows of A are zero, atlas LoraPair doc).  c ascending. */
static void shrink_row(const orc_route *r, int idx, const void *x, size_t x_off, double *t) {
  const void *A = r->a[idx];
  for (int k = 0; k < r->max_rank; ++k) {
    double acc = 0.0;
#if ORC_MUTANT == 3
    for (int c = 0; c < r->k_in - 1; ++c)
#else
    for (int c = 0; c < r->k_in; ++c)
#endif
      acc += widen(A, r->dtype, (size_t)k * r->k_in + c) * widen(x, r->dtype, x_off + c);
    t[k] = acc;
  }
}

/* ferrox LoraDelta::accumulate: d[o] = B[o,:] . t, the scale applied after
 * the rank dot.  k ascending. */
static double expand_one(const orc_route *r, int idx, int o, const double *t) {
  const void *B = r->b[idx];
  double acc = 0.0;
  for (int k = 0; k < r->max_rank; ++k) {
#if ORC_MUTANT == 4
    acc += widen(B, r->dtype, (size_t)k * r->n_out + o) * t[k];
#else
    acc += widen(B, r->dtype, (size_t)o * r->max_rank + k) * t[k];
#endif
  }
  return acc;
}

static double delta_sign(void) {
#if ORC_MUTANT == 5
  return -1.0;
#else
  return 1.0;
#endif
}

static size_t xrow(size_t i, int x_stride, int k_in) {
#if ORC_MUTANT == 8
  (void)x_stride;
  return i * (size_t)k_in;
#else
  (void)k_in;
  return i * (size_t)x_stride;
#endif
}

/* base[o] = W[o,:] . x   (ferrox module doc "Layouts": W is [rows][cols]). */
static double base_one(const void *W, size_t w_off, int w_stride, int dtype, int o,
                       const void *x, size_t x_off, int k_in) {
  double acc = 0.0;
#if ORC_MUTANT == 12
  for (int c = 1; c < k_in; ++c)
#else
  for (int c = 0; c < k_in; ++c)
#endif
    acc += widen(W, dtype, w_off + (size_t)o * w_stride + c) * widen(x, dtype, x_off + c);
  return acc;
}

/* ------------------------------------------------------------------ ops */

/*
 * lora_shrink: t[i, 0:max_rank] = A_s x_i for rows that resolve to a slot;
 * rows that skip are left untouched.  atlas apply_lora_bgmv kernel 1.
 */
void orc_shrink(const orc_route *r, const void *x, int x_stride, const int32_t *seq_slot,
                int n, double *t) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    int idx = resolve(r, seq_slot[i], 0);
    if (idx < 0) continue;
    shrink_row(r, idx, x, xrow((size_t)i, x_stride, r->k_in), t + (size_t)i * r->max_rank);
  }
}

/*
 * lora_expand_fold: y_out[i, o] = y_in[i, o] + s * (B_s t_i)[o]; rows that
 * skip copy y_in exactly (no arithmetic).  atlas apply_lora_bgmv kernel 2;
 * t is the f32 intermediate the library's boundary carries.
 */
void orc_expand_fold(const orc_route *r, const float *t, const int32_t *seq_slot, int n,
                     const void *y_in, int y_stride, double *y_out) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    int idx = resolve(r, seq_slot[i], 0);
    double *yo = y_out + (size_t)i * r->n_out;
    if (idx < 0) {
      for (int o = 0; o < r->n_out; ++o)
        yo[o] = widen(y_in, r->dtype, (size_t)i * y_stride + o);
      continue;
    }
    double *tt = (double *)malloc(sizeof(double) * (size_t)r->max_rank);
    for (int k = 0; k < r->max_rank; ++k) tt[k] = (double)t[(size_t)i * r->max_rank + k];
    double s = (double)r->scale[seq_slot[i]];
    for (int o = 0; o < r->n_out; ++o)
      yo[o] = widen(y_in, r->dtype, (size_t)i * y_stride + o) +
              delta_sign() * s * expand_one(r, idx, o, tt);
    free(tt);
  }
}

/* One output row of the fused apply: base, then the delta unless skipped. */
static void apply_row(const void *W, size_t w_off, int w_stride, const orc_route *r,
                      int dtype, int k_in, int n_out, const void *x, size_t x_off, int slot,
                      int expert, double *yo) {
  for (int o = 0; o < n_out; ++o) yo[o] = base_one(W, w_off, w_stride, dtype, o, x, x_off, k_in);
  int idx = resolve(r, slot, expert);
  if (idx < 0) return; /* ferrox add_to: skip before any arithmetic */
  double *t = (double *)malloc(sizeof(double) * (size_t)r->max_rank);
  shrink_row(r, idx, x, x_off, t);
  double s = (double)r->scale[slot];
  for (int o = 0; o < n_out; ++o) yo[o] = yo[o] + delta_sign() * s * expand_one(r, idx, o, t);
  free(t);
}

/*
 * lora_apply: y[i, :] = W x_i (+ s B_s A_s x_i), for every row, in row order
 * (ferrox add_batch_to: each position on its own).  `r` may be NULL (base
 * only).  y is [n][n_out] doubles.
 */
void orc_apply(const void *W, int w_stride, const orc_route *r, int dtype, int k_in,
               int n_out, const void *x, int x_stride, const int32_t *seq_slot, int n,
               double *y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i)
    apply_row(W, 0, w_stride, r, dtype, k_in, n_out, x, xrow((size_t)i, x_stride, k_in),
              seq_slot ? seq_slot[i] : -1, 0, y + (size_t)i * n_out);
}

/* The same for a chosen subset of rows (sampled checks at full size). */
void orc_apply_rows(const void *W, int w_stride, const orc_route *r, int dtype, int k_in,
                    int n_out, const void *x, int x_stride, const int32_t *seq_slot,
                    const int32_t *rows, int n_rows, double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < n_rows; ++j) {
    size_t i = (size_t)rows[j];
#if ORC_MUTANT == 18
    size_t xi = (size_t)j;
#else
    size_t xi = i;
#endif
#if ORC_MUTANT == 19
    size_t si = (size_t)j;
#else
    size_t si = i;
#endif
    apply_row(W, 0, w_stride, r, dtype, k_in, n_out, x, xrow(xi, x_stride, k_in),
              seq_slot ? seq_slot[si] : -1, 0, y + (size_t)j * n_out);
  }
}

/*
 * Segmented prefill: rows seg_indptr[g] .. seg_indptr[g+1]-1 share slot
 * seg_slot[g]; otherwise the same per-row definition.  ferrox add_batch_to
 * (prefill batch), atlas apply_lora_delta (m rows, one pair).  Rows outside
 * every segment are not written.
 */
void orc_apply_segmented(const void *W, int w_stride, const orc_route *r, int dtype,
                         int k_in, int n_out, const void *x, int x_stride,
                         const int32_t *seg_indptr, const int32_t *seg_slot, int n_seg,
                         const int32_t *rows, int n_rows, double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < n_rows; ++j) {
    int i = rows[j];
    int slot = -1, found = 0;
    for (int g = 0; g < n_seg; ++g) {
#if ORC_MUTANT == 11
      if (i >= seg_indptr[g] && i <= seg_indptr[g + 1]) {
#else
      if (i >= seg_indptr[g] && i < seg_indptr[g + 1]) {
#endif
        slot = seg_slot[g];
        found = 1;
        break;
      }
    }
    if (!found) continue;
#if ORC_MUTANT == 20
    size_t xi = (size_t)j;
#else
    size_t xi = (size_t)i;
#endif
    apply_row(W, 0, w_stride, r, dtype, k_in, n_out, x, xrow(xi, x_stride, k_in), slot,
              0, y + (size_t)j * n_out);
  }
}

/*
 * MoE down_proj gather (atlas lora_delta.rs, moe_lora_gather_bgmv field doc:
 * keyed on expert through the per-slot indices array, slot-major).  Routing
 * slot j belongs to token j / top_k and expert e = indices[j]:
 *   y[j] = W_e x[j] + s_a B_{a,e} (A_{a,e} x[j]),  a = token_slot[j / top_k].
 * Rows whose expert id is outside [0, n_experts) are not written.
 */
void orc_apply_moe_gather(const void *W, long long expert_stride, int w_stride,
                          const orc_route *r, int dtype, int k_in, int n_out, int n_experts,
                          const void *x, int x_stride, const int32_t *indices, int top_k,
                          const int32_t *token_slot, const int32_t *rows, int n_rows,
                          double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int jj = 0; jj < n_rows; ++jj) {
    int j = rows[jj];
    int e = indices[j];
    if (e < 0 || e >= n_experts) continue;
#if ORC_MUTANT == 21
    int a = token_slot[jj / top_k];
#else
    int a = token_slot[j / top_k];
#endif
    apply_row(W, (size_t)e * (size_t)expert_stride, w_stride, r, dtype, k_in, n_out, x,
              xrow((size_t)j, x_stride, k_in), a, e, y + (size_t)jj * n_out);
  }
}

/*
 * MoE grouped layout (atlas lora_delta.rs, the moe_lora_grouped_down field
 * doc: the expert down_proj delta keyed on expert through device
 * expert_offsets, the sorted twin of the gather above).  The rows come
 * sorted by expert: rows expert_offsets[e] .. expert_offsets[e+1]-1 belong
 * to expert e.  Readings: offsets are non-decreasing, so at most one range
 * holds a row; a row outside every range is not written; each sorted row
 * carries its own adapter slot (seq_slot[j], the slot of the token it came
 * from), resolved by the same rule as the dense path with the pair of
 * (adapter a, expert e) at table index a * n_experts + e.
 * Returns the expert of row j, or -1.
 */
static int expert_of(const int32_t *offsets, int n_experts, int j) {
  for (int e = 0; e < n_experts; ++e) {
#if ORC_MUTANT == 13
    if (j >= offsets[e] && j <= offsets[e + 1]) return e;
#else
    if (j >= offsets[e] && j < offsets[e + 1]) return e;
#endif
  }
  return -1;
}

/* The slot a grouped row carries. */
static int grouped_slot(const int32_t *seq_slot, const int32_t *offsets, int e, int j) {
#if ORC_MUTANT == 14
  return seq_slot[j - offsets[e]];
#else
  (void)offsets;
  (void)e;
  return seq_slot[j];
#endif
}

/*
 * Fused grouped apply: y[j] = W_e x[j] + s_a B_{a,e} (A_{a,e} x[j]) for row
 * j of expert e's range, a = seq_slot[j]; only the listed rows, in order.
 * Rows outside every range are left untouched.  `r` may be NULL (base only).
 */
void orc_apply_moe_grouped(const void *W, long long expert_stride, int w_stride,
                           const orc_route *r, int dtype, int k_in, int n_out, int n_experts,
                           const void *x, int x_stride, const int32_t *expert_offsets,
                           const int32_t *seq_slot, const int32_t *rows, int n_rows,
                           double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int jj = 0; jj < n_rows; ++jj) {
    int j = rows[jj];
#if ORC_MUTANT == 22
    int e = expert_of(expert_offsets, n_experts, jj);
#else
    int e = expert_of(expert_offsets, n_experts, j);
#endif
    if (e < 0) continue;
    int a = seq_slot ? grouped_slot(seq_slot, expert_offsets, e, j) : -1;
    apply_row(W, (size_t)e * (size_t)expert_stride, w_stride, r, dtype, k_in, n_out, x,
              xrow((size_t)j, x_stride, k_in), a, e, y + (size_t)jj * n_out);
  }
}

/* The grouped shrink: t[j] = A_{a,e} x[j] for rows that resolve; others untouched. */
void orc_moe_grouped_shrink(const orc_route *r, const void *x, int x_stride,
                            const int32_t *expert_offsets, const int32_t *seq_slot, int n,
                            double *t) {
#pragma omp parallel for schedule(static)
  for (int j = 0; j < n; ++j) {
    int e = expert_of(expert_offsets, r->n_experts, j);
    if (e < 0) continue;
    int idx = resolve(r, grouped_slot(seq_slot, expert_offsets, e, j), e);
    if (idx < 0) continue;
    shrink_row(r, idx, x, xrow((size_t)j, x_stride, r->k_in), t + (size_t)j * r->max_rank);
  }
}

/*
 * The grouped expand-and-fold: y_out[j] = y_in[j] + s_a B_{a,e} t[j] for rows
 * that resolve; every other row (skipped, or outside every range) copies
 * y_in exactly.
 */
void orc_moe_grouped_expand_fold(const orc_route *r, const float *t,
                                 const int32_t *expert_offsets, const int32_t *seq_slot, int n,
                                 const void *y_in, int y_stride, double *y_out) {
#pragma omp parallel for schedule(static)
  for (int j = 0; j < n; ++j) {
    double *yo = y_out + (size_t)j * r->n_out;
    for (int o = 0; o < r->n_out; ++o) yo[o] = widen(y_in, r->dtype, (size_t)j * y_stride + o);
    int e = expert_of(expert_offsets, r->n_experts, j);
    if (e < 0) continue;
    int a = grouped_slot(seq_slot, expert_offsets, e, j);
    int idx = resolve(r, a, e);
    if (idx < 0) continue;
    double *tt = (double *)malloc(sizeof(double) * (size_t)r->max_rank);
    for (int k = 0; k < r->max_rank; ++k) tt[k] = (double)t[(size_t)j * r->max_rank + k];
    double s = (double)r->scale[a];
    for (int o = 0; o < r->n_out; ++o) yo[o] = yo[o] + delta_sign() * s * expand_one(r, idx, o, tt);
    free(tt);
  }
}

/*
 * Adapter stack (ferrox lora.rs LoraStack: every adapter attached to one
 * base matrix, applied in order, each a term of the sum W x + sum_i s_i
 * B_i (A_i x)).  Level l has its own route and per-row slot buffer;
 * y[i] = W x_i + sum over levels, in level order, of the level's delta
 * (each level skips by the usual rule).  Only the listed rows.
 */
void orc_apply_stack(const void *W, int w_stride, const orc_route *const *routes,
                     const int32_t *const *seq_slots, int n_levels, int dtype, int k_in,
                     int n_out, const void *x, int x_stride, const int32_t *rows, int n_rows,
                     double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int jj = 0; jj < n_rows; ++jj) {
    size_t i = (size_t)rows[jj];
    size_t x_off = xrow(i, x_stride, k_in);
    double *yo = y + (size_t)jj * n_out;
    for (int o = 0; o < n_out; ++o) yo[o] = base_one(W, 0, w_stride, dtype, o, x, x_off, k_in);
#if ORC_MUTANT == 15
    for (int l = 0; l < n_levels && l < 1; ++l) {
#else
    for (int l = 0; l < n_levels; ++l) {
#endif
      const orc_route *r = routes[l];
#if ORC_MUTANT == 23
      int slot = seq_slots[l][jj];
#else
      int slot = seq_slots[l][i];
#endif
      int idx = resolve(r, slot, 0);
      if (idx < 0) continue; /* this level adds nothing to the row */
      double *t = (double *)malloc(sizeof(double) * (size_t)r->max_rank);
      shrink_row(r, idx, x, x_off, t);
      double s = (double)r->scale[slot];
      for (int o = 0; o < n_out; ++o) yo[o] = yo[o] + delta_sign() * s * expand_one(r, idx, o, t);
      free(t);
    }
  }
}

/*
 * Token-embedding row gather (ferrox lora.rs LoraDelta::add_row_to: the delta
 * of ONE row of the adapted matrix, s * (B[r] A), which a row gather needs;
 * module doc "Layouts": the embedding pair is brought into the one layout,
 * A [rank][n_embd], B [n_vocab][rank]).  The route's k_in is n_embd (A's
 * columns) and its n_out is n_vocab (B's rows).  Row i takes token
 * t = token_ids[i]:
 *   y[i, c] = E[t, c] + s * sum_k B[t, k] A[k, c]     (k ascending)
 * for rows whose slot resolves; E[t, :] alone otherwise.  Reading: a token
 * outside [0, n_vocab) leaves the row unwritten.  Only the listed rows.
 */
void orc_embed_rows(const void *E, int e_stride, const orc_route *r, int dtype, int n_vocab,
                    int n_embd, const int32_t *token_ids, const int32_t *seq_slot,
                    const int32_t *rows, int n_rows, double *y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int jj = 0; jj < n_rows; ++jj) {
    int i = rows[jj];
    int tok = token_ids[i];
    if (tok < 0 || tok >= n_vocab) continue;
    double *yo = y + (size_t)jj * n_embd;
    for (int c = 0; c < n_embd; ++c) yo[c] = widen(E, dtype, (size_t)tok * e_stride + c);
#if ORC_MUTANT == 24
    int slot = seq_slot ? seq_slot[jj] : -1;
#else
    int slot = seq_slot ? seq_slot[i] : -1;
#endif
    int idx = resolve(r, slot, 0);
    if (idx < 0) continue;
    double s = (double)r->scale[slot];
    for (int c = 0; c < n_embd; ++c) {
      double acc = 0.0;
      for (int k = 0; k < r->max_rank; ++k) {
#if ORC_MUTANT == 16
        double b = widen(r->b[idx], dtype, (size_t)k * n_vocab + tok);
#else
        double b = widen(r->b[idx], dtype, (size_t)tok * r->max_rank + k);
#endif
        acc += b * widen(r->a[idx], dtype, (size_t)k * n_embd + c);
      }
      yo[c] = yo[c] + delta_sign() * s * acc;
    }
  }
}

/*
 * The token-embedding pair brought into the one layout (ferrox lora.rs
 * module doc "Layouts"; frink lora_attach.rs checked_pair, embedding
 * branch): the file stores A_file [n_vocab][rank] and B_file [n_embd][rank];
 * in the one layout B is A_file as it is and A [rank][n_embd] is B_file
 * transposed, A[k][e] = B_file[e][k].  Copies elements of the storage type.
 */
void orc_embedding_pair(const void *b_file, int dtype, int n_embd, int rank, void *a_out) {
  size_t esz = dtype == ORC_F32 ? 4 : 2;
  for (int k = 0; k < rank; ++k)
    for (int e = 0; e < n_embd; ++e) {
#if ORC_MUTANT == 17
      size_t src = (size_t)k * n_embd + e;
#else
      size_t src = (size_t)e * rank + k;
#endif
      memcpy((char *)a_out + ((size_t)k * n_embd + e) * esz, (const char *)b_file + src * esz, esz);
    }
}

int orc_mutant(void) { return ORC_MUTANT; }

/* Threads an OpenMP loop here uses (1 without OpenMP). */
int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the loops over rows from now on (timing only; the results do
   not depend on it: every row is computed by one thread in a fixed order). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
