// launch.hpp -- internal launchers the C ABI (lora_host.cpp) calls.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace lora {

// Plan written by the prep kernel for the main kernel: row order grouped by
// (W group, pair), and the main kernel's row tiles.
struct PlanDev {
  int *pos_row;   // [n] original row at sorted position
  int *pos_pair;  // [n] table index, kSkip, at sorted position
  int4 *tiles;    // [max_mtiles] {group, start, count, 0}
  int *n_tiles;   // [1]
};

struct PrepArgs {
  RouteDev rd;
  Routing rt;
  bool has_lora;
  const u16 *x;
  int x_stride;
  int k_in;
  int n;
  float *t;        // [k_splits][n][R] partial shrink sums (k_splits > 1)
  float *t_final;  // [n][R] the shrink's output
  u16 *tt;         // [n][2R] or null: s_pair * t as bf16, high parts then remainders, for the GEMM
  unsigned *counters;  // [n_units] arrival counters (k_splits > 1), zero between calls
  int k_splits;    // k chunks per shrink unit
  int n_pairs;    // table entries = max_loras * n_experts
  int do_plan;    // a workgroup writes the plan: workgroup plan_at of the grid
  int plan_at;
  int seg_units;  // segmented, no route kernel: units take their rows from the segments
  int reg_units;  // the shrink units load their operands into registers (k_prep.hip)
  PlanDev plan;
  int tile_rows;  // main kernel rows per tile
  int n_units;    // shrink units (grid = do_plan + n_units * k_splits)
  int *routes;    // [n] every row's packed route (the route kernel writes it)
  // With routes: the route kernel also counts the rows of every pair and
  // gives each row its rank among them (in no particular order), so that a
  // shrink unit finds its rows without sorting; the last prep workgroup to
  // finish zeroes the counts again.
  int *ranks;              // [n] the row's rank within its pair, or -1
  unsigned *pair_cnt;      // [n_pairs] rows per pair, zero between calls
  unsigned *prep_done;     // [1] prep workgroups finished, zero between calls
  // With ranks: pair q's rows of rank below kShrinkRows at
  // bucket[q kShrinkRows + rank], for q < bucket_pairs (or null), so that a
  // unit of a pair with at most kShrinkRows rows takes them without a scan.
  int *bucket;
  int bucket_pairs;
};

struct GemmArgs {
  const u16 *W;
  long long w_group_stride;
  int w_row_stride;
  const u16 *x;
  int x_row_stride;
  u16 *y;
  int y_row_stride;
  int n_out, k_in;
  PlanDev plan;
  int max_mtiles, n_ntiles;
  int has_lora;
  const void *const *b_table;
  const float *scale_table;
  int n_experts;
  const u16 *tt;   // [n][2R] the shrink's output scaled by the pair's scale, bf16 high parts
                   // (columns 0..R-1) and what they leave over (R..2R-1)
  int R;
  int splits;      // split-K: k ranges per tile, the same ranges for every tile
  float *partials; // [tiles * splits][BO*BR] partial tiles
  unsigned *counters;  // [tiles] arrival counters, zero between calls
};

// The decode-shaped apply (k_decode.hip), n <= 64 rows, in one launch (after
// a prep launch for the shrink when the pool is too large for the launch's
// carrier waves).  Workgroup (g, z) = tile g of tile_out outputs x
// k range z of kDecodeKR columns; its f32 partial of each 16-output slice
// goes to `partials`, and contributor z finalizes slices z, z + S, ... of its
// tile.
struct DecodeArgs {
  const u16 *W;
  int w_row_stride;
  const u16 *x;
  int x_row_stride;
  u16 *y;
  int y_row_stride;
  int n_out, k_in, n;
  RouteDev rd;
  const int32_t *seq_slot;
  int has_lora;
  int R;                // max_rank (0: base only)
  int S;                // k ranges
  int n_tiles;          // ceil(n_out / tile_out)
  int tile_out;         // outputs per tile: 16 x the waves (128 or 64)
  float *partials;      // [n_tiles][S][kDecodeSlices][kDecodeSliceFloats]
  // The shrink: with unit_tiles > 0 it rides this launch (one unit, on wave
  // 0 of each workgroup of the first unit_tiles tiles, see k_decode.hip) and
  // leaves range pieces [S][max_loras][n][R] in t_part, written for the rows
  // on each slot (max_loras x R <= kDecodeUnitRanks); otherwise a prep
  // launch wrote t [n][R].
  int unit_tiles;
  float *t_part;
  const float *t;
  // words that are zero between calls, a cache line each (kDecodeCtrStride
  // words apart): tile g's at tile_cnt + g kDecodeCtrStride, [0]
  // contributors that stored their partials plus k ranges whose units are
  // all done, [1] finalization items past the wait for them; then range z's
  // unit count at tile_cnt + (n_tiles + z) kDecodeCtrStride
  unsigned *tile_cnt;
  // 1: tile g's S contributors are the workgroups 8 (S (g / 8) + z) + g % 8,
  // which the chip's round-robin hand-out of workgroups to its 8 XCDs puts
  // on one XCD, and their partials pass through that XCD's L2; 0: tile g's
  // contributors are workgroups S g .. S g + S - 1 and their partials pass
  // through the memory side
  int xcd_local;
};

// Largest batch the decode kernel takes; columns per k range; the largest
// k split (so k_in <= 512 x 16 = 8192 on this path); slices (16 outputs)
// per tile at most; floats of one slice partial (64 rows x 16 outputs).
constexpr int kDecodeMaxRows = 64;
constexpr int kDecodeKR = 512;
constexpr int kDecodeMaxSplit = 16;
constexpr int kDecodeSlices = 8;
constexpr int kDecodeSliceFloats = 64 * 16;
constexpr int kDecodeCtrStride = 32;  // words: 128 bytes
// The most pool ranks (slots x max_rank) the shrink takes inside the decode
// launch: 16 units of 16 ranks.
constexpr int kDecodeUnitRanks = 256;
constexpr int kDecodeTileOut = 128;
// Projections up to this many outputs take tiles of kDecodeTileOutSmall
// outputs, so that their launch still spreads over the chip.
constexpr int kDecodeTileOutSmall = 64;
constexpr int kDecodeSmallTileMaxOut = 2048;
// Workgroups of a decode launch that may carry the shrink's units (one
// each); the host also keeps them to half the device's compute units.
constexpr int kDecodeMaxCarrierWgs = 128;

// Rows per shrink unit; its 64-column stages in LDS at a time (16 KB each);
// with register loads, the 32-column steps whose loads a wave has in flight
// together, and the LDS where its four waves' sums meet (12 blocks (wave,
// rank block) of another wave's rank block x 4 row groups x 64 lanes x 16
// bytes); the LDS either way.
constexpr int kShrinkRows = 64;
constexpr int kShrinkStages = 3;
constexpr int kShrinkSteps = 4;
constexpr int kShrinkRedBytes = 12 * (kShrinkRows / 16) * 64 * 16;
constexpr int kShrinkLdsBytes =
    kShrinkStages * 128 * 128 > kShrinkRedBytes ? kShrinkStages * 128 * 128 : kShrinkRedBytes;
// Largest k split of the shrink units.
constexpr int kMaxShrinkSplits = 8;
// Largest key space the one-workgroup plan handles (LDS histogram).
constexpr int kMaxKeys = 4096;

// The extra levels of an adapter stack (every level but the first, which the
// fused apply takes): each level's route tables, per-row slots and shrink
// output t [n][R].
constexpr int kMaxStackLevels = 8;
struct StackLevel {
  const void *const *a_table;
  const void *const *b_table;
  const float *scale_table;
  const int32_t *seq_slot;
  const float *t;
  int max_loras;
  int R;
};
struct StackFold {
  StackLevel lv[kMaxStackLevels];
  int n_levels;
};

// The token-embedding row gather (k_embed.hip).
struct EmbedArgs {
  const void *E;        // [n_vocab][e_row_stride]
  int e_row_stride;
  int n_vocab, n_embd, n;
  RouteDev rd;          // A [R][n_embd], B [n_vocab][R]
  int has_lora;
  const int32_t *token_ids;  // [n]
  const int32_t *seq_slot;   // [n]
  void *y;              // [n][y_row_stride]
  int y_row_stride;
};

// The shrinks of a stack's further levels in one launch: level l takes
// blocks [l * blocks_per_level, (l + 1) * blocks_per_level), each level's
// arguments those of a standalone shrink (no plan, no routes).
struct ShrinkLevels {
  PrepArgs lv[kMaxStackLevels];
  int n_levels;
  int blocks_per_level;
};

size_t prep_lds_bytes(const PrepArgs &a);
hipError_t launch_shrink_levels(const ShrinkLevels &s, hipStream_t st);

// The standalone shrink and expand-fold by pool slot (k_bgmv.hip), bf16,
// for batches of at most kBgmvMaxRows rows; x, t and y 16-byte aligned.
constexpr int kBgmvMaxRows = 1024;
hipError_t launch_bgmv_shrink(const RouteDev &rd, const int32_t *seq_slot, int n, const u16 *x, int x_stride,
                              int k_in, float *t, hipStream_t st);
hipError_t launch_bgmv_expand(const RouteDev &rd, const int32_t *seq_slot, int n, const float *t, u16 *y,
                              int y_stride, int n_out, hipStream_t st);
// The same shrink for an adapter stack's further levels, in one launch:
// level l writes t[l] [n][R_l] for its rows that resolve.
struct BgmvLevels {
  RouteDev rd[kMaxStackLevels];
  const int32_t *seq_slot[kMaxStackLevels];
  float *t[kMaxStackLevels];
  int n_levels;
  int blocks_per_level;  // the largest max_loras x R over the levels
};
hipError_t launch_bgmv_shrink_levels(const BgmvLevels &L, const u16 *x, int x_stride, int k_in, int n,
                                     hipStream_t st);

hipError_t launch_shrink_f32(const RouteDev &rd, const Routing &rt, const float *x, int x_stride,
                             int k_in, int n, float *t, hipStream_t st);
hipError_t launch_apply_f32(const RouteDev &rd, const Routing &rt, bool has_lora, const float *W,
                            long long w_group_stride, int w_stride, const float *x, int x_stride,
                            int k_in, int n_out, int n, float *y, int y_stride, hipStream_t st);
hipError_t launch_expand_fold(const RouteDev &rd, int dtype, const Routing &rt, const float *t,
                              void *y, int y_stride, int n_out, int n, hipStream_t st);
hipError_t launch_expand_fold_stack(const StackFold &f, int dtype, void *y, int y_stride, int n_out, int n,
                                    hipStream_t st);
hipError_t launch_embed_rows(const EmbedArgs &a, int dtype, hipStream_t st);
hipError_t launch_prep(const PrepArgs &a, hipStream_t st);
hipError_t launch_gemm(const GemmArgs &a, int to, int tr, hipStream_t st);
// `stack` (or null): an adapter stack's further levels, folded into the same rounding.
hipError_t launch_decode(const DecodeArgs &a, const StackFold *stack, hipStream_t st);

}  // namespace lora
