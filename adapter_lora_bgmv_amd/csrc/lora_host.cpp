// lora_host.cpp -- the C ABI declared in include/lora_mi355x.h.
//
// Host side only: argument validation (before any launch), the scale and
// seq_slot helpers, the launch geometry and the workspace layout.  Nothing
// here allocates, frees, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/lora_mi355x.h"
#include "launch.hpp"

using namespace lora;

// The array itself (see ScratchDev below).
static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];
thread_local hipEvent_t g_prof[4];
thread_local bool g_prof_on = false;

void prof_record(int i, hipStream_t st) {
  if (g_prof_on) (void)hipEventRecord(g_prof[i], st);
}

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_err() { g_err[0] = 0; }

int launch_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(LORA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return LORA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------ device check
int g_dev_ok[64];   // 0 unknown, 1 gfx950, -1 other
int g_dev_cus[64];  // compute units, once known

int check_device(const char *what) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(LORA_ERR_LAUNCH, "%s: no HIP device is current", what);
  if (dev < 0 || dev >= 64) return fail(LORA_ERR_LAUNCH, "%s: device index %d out of range", what, dev);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(LORA_ERR_LAUNCH, "%s: cannot query device %d", what, dev);
    g_dev_cus[dev] = prop.multiProcessorCount;
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (g_dev_ok[dev] < 0)
      return fail(LORA_ERR_LAUNCH, "%s: device %d is %s, the kernels are built for gfx950 only",
                  what, dev, prop.gcnArchName);
  }
  if (g_dev_ok[dev] < 0) return fail(LORA_ERR_LAUNCH, "%s: device %d is not a gfx950", what, dev);
  return LORA_OK;
}

// The current device's compute units (0 if it was never checked).
int current_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  return g_dev_cus[dev];
}

// ------------------------------------------------------------ scratch for callers that cannot allocate
// lora_apply_noalloc's workspace: one array per device, held until the
// process ends.  The words that must be zero between calls of any shape lie
// in its first kScratchZeroBytes; everything else lies above them.  Host
// code uses the address hipGetSymbolAddress gives on each device, never the
// array's name.
constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchZeroBytes = 1u << 20;
static_assert(kScratchZeroBytes % 16 == 0 && kScratchZeroBytes < kScratchBytes, "zero region");

struct ScratchDev {
  void *ptr;    // the array's address on this device
  bool zeroed;  // its zero region has been cleared by a call made outside stream capture
};
std::mutex g_scratch_mu;
ScratchDev g_scratch[64];

__global__ void zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------ tiling
struct Cfg {
  int to, tr, splits, k_per_split, max_mtiles, n_ntiles;
  int partial_slots;  // partial tiles the GEMM's split-K may store
  bool decode;   // the one-launch decode kernel (k_decode.hip)
  int units;     // upper bound of shrink units
  int t_splits;     // k chunks of the shrink; the consumer sums the partials
  int t_splits_ws;  // the most k chunks any routing of this shape may take (workspace sizing)
  long long zero_tiles;  // tile counters any tiling of this shape may use (64 x 64 tiles are the smallest)
  int zero_units;        // shrink arrival counters any routing of this shape may use
};

constexpr int kNarrowTileMaxRows = 256;  // 256 x 128 GEMM tiles up to this many rows

int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Tile shape and split factor.  The split factor is a function of the
// operation, the batch size and k_in, never of n_out, the rank or the
// routing; every output element's reduction order follows from the split
// factor and k_in alone (not from the tile shape), so it is the same whether
// a fused projection is applied whole or part by part, and a skipped row's
// is the base-only call's.
Cfg choose_cfg(int op, int n, int n_out, int k_in, int groups, int R, int n_pairs) {
  Cfg c{};
  const bool moe = op == LORA_OP_MOE_GATHER || op == LORA_OP_MOE_GROUPED;
  c.decode = op == LORA_OP_APPLY && n <= kDecodeMaxRows && k_in <= kDecodeKR * kDecodeMaxSplit;
  c.units = R > 0 ? (n + kShrinkRows - 1) / kShrinkRows + std::min(n, n_pairs) : 0;
  // Shrink k chunks: enough workgroups to cover the chip for small batches,
  // chunks of at least 256 columns.  A function of (n, k_in) only, so the
  // workspace size does not depend on the routing.
  // about 512 shrink workgroups: the units are row blocks of 64 for few
  // pairs, and about one per pair when many pairs share the rows (MoE);
  // the workspace holds partials for the most chunks the shape allows
  const int ks_max = std::min(kMaxShrinkSplits, std::max(1, k_in / 256));
  const int units_est = std::max((n + kShrinkRows - 1) / kShrinkRows, std::min(n, n_pairs));
  c.t_splits = R > 0 ? clampi(512 / std::max(1, units_est), 1, ks_max) : 1;
  c.t_splits_ws = R > 0 ? ks_max : 1;
  if (c.decode) {
    // k ranges of kDecodeKR columns; a small projection takes 64-output tiles
    // (more workgroups; every output is reduced in the same order either way)
    c.to = n_out <= kDecodeSmallTileMaxOut ? kDecodeTileOutSmall : kDecodeTileOut;
    c.tr = kDecodeMaxRows;
    c.splits = (k_in + kDecodeKR - 1) / kDecodeKR;
  } else if (moe) {
    // one row tile per expert where the batch allows: an expert's W slab is
    // read once per row tile (128-row tiles from ~96 rows per expert on,
    // 256-row tiles from ~160 when the rank fits the LDS LoRA path)
    const int per = n / std::max(1, groups);
    const bool lds_rank = R == 0 || (R <= 64 && 64 % R == 0);
    c.to = 256; c.tr = per >= 160 && lds_rank ? 256 : (per >= 96 ? 128 : 64); c.splits = 1;
    // 64-row tiles 512 outputs wide when one row tile per expert makes one
    // round of workgroups on the device (256 wide would take two)
    if (c.tr == 64 && lds_rank && n_out >= 512 && groups * ((n_out + 511) / 512) <= current_cus()) c.to = 512;
  } else if (n <= 64) {
    c.to = 64; c.tr = 64; c.splits = clampi(k_in / 1024, 1, 8);
  } else if (n <= 128) {
    c.to = 128; c.tr = 128; c.splits = clampi(k_in / 1024, 1, 4);
  } else {
    // up to kNarrowTileMaxRows rows W is the stream to keep moving: 256 x 128
    // tiles leave LDS for three 48 KB stages (two in flight) where 256 x 256
    // tiles fit two 64 KB ones; the row tiles of one W tile run on
    // neighbouring workgroups, so W still comes from HBM about once.  One k
    // range per tile: on the fused gate/up shape (256 rows, 22016 x 4096) two
    // or four ranges were slower (their partial tiles cost more than the
    // extra workgroups gain).  The 256 x 256 tiles stage the LoRA term
    // through LDS, which takes ranks dividing 64; other ranks keep 256 x 128
    // tiles (the tile shape does not change any element's reduction order).
    const bool lds_rank = R == 0 || (R <= 64 && 64 % R == 0);
    c.to = 256; c.tr = n <= kNarrowTileMaxRows || !lds_rank ? 128 : 256;
    c.splits = 1;
    // 128-row tiles 192 outputs wide when they still make one round of
    // workgroups on the device: a stage's fragment reads and MFMAs, not its
    // DMA, bound these tiles, so more busy CUs finish sooner (the fused
    // gate/up shape: 172 workgroups of 256 x 128, or 230 of 192 x 128)
    const int mt = (n + 127) / 128, cus = current_cus();
    if (c.tr == 128 && (n_out + 191) / 192 * mt <= cus) c.to = 192;
  }
  if (c.decode) {
    c.k_per_split = kDecodeKR;
  } else {
    const int kslabs = (k_in + 63) / 64;
    c.k_per_split = ((kslabs + c.splits - 1) / c.splits) * 64;
  }
  c.max_mtiles = (n + c.tr - 1) / c.tr + (moe ? groups : 0);
  c.zero_tiles = (long long)((n + 63) / 64 + (moe ? groups : 0)) * ((n_out + 63) / 64);
  c.zero_units = (n + kShrinkRows - 1) / kShrinkRows + n;
  c.n_ntiles = (n_out + c.to - 1) / c.to;
  const long long tiles = (long long)c.max_mtiles * c.n_ntiles;
  c.partial_slots = c.splits > 1 ? (int)(tiles * c.splits) : 0;
  return c;
}

struct WsLayout {
  size_t counters, shrink_counters, pos_row, pos_pair, routes, ranks, bucket, pair_cnt, tiles, n_tiles, t, t_final, tt,
      partials, total;
  // the decode kernel's zero-between-calls words
  size_t tile_cnt;
  size_t zero_end;  // the words that must be zero between calls lie below this offset
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// `data_base`: the first byte past the words that must be zero between
// calls may not lie below it (0: packed); a shared scratch buffer keeps
// every shape's zero words below one fixed offset that way.
WsLayout ws_layout(const Cfg &c, int n, int R, int k_in, size_t data_base = 0) {
  WsLayout w{};
  size_t off = 0;
  if (c.decode) {
    // the tiles' arrival counters (zero between calls; their offsets depend
    // on n_out alone), the prep shrink's arrival counters, the slice
    // partials, the shrink's partials, then t
    const size_t tiles = (size_t)c.n_ntiles;
    w.tile_cnt = off; off = up256(off + (tiles + c.splits) * kDecodeCtrStride * 4);
    w.shrink_counters = off; off = up256(off + (size_t)c.zero_units * 4);
    w.zero_end = off; off = std::max(off, data_base);
    w.partials = off;
    off = up256(off + tiles * c.splits * kDecodeSlices * kDecodeSliceFloats * 4);
    // the shrink's partials: the prep launch's k chunks, or this launch's
    // range pieces, whichever is larger
    const size_t prep_parts = (size_t)(c.t_splits_ws > 1 ? c.t_splits_ws : 0) * n * R;
    const size_t pieces = (size_t)c.splits * kDecodeUnitRanks * n;
    w.t = off; off = up256(off + (R > 0 ? std::max(prep_parts, pieces) * 4 : 0));
    w.t_final = off; off = up256(off + (size_t)n * R * 4);
    w.total = off;
    return w;
  }
  // The words that must be zero between calls come first, sized for any
  // tiling and routing of the shape, so that every call of the shape --
  // routed with any rank, or base only -- finds them at the same offsets.
  w.counters = off; off = up256(off + (size_t)c.zero_tiles * 4);
  w.shrink_counters = off; off = up256(off + (size_t)c.zero_units * 4);
  w.pair_cnt = off; off = up256(off + (size_t)(kMaxKeys + 1) * 4);  // any table size, then the arrival count
  w.zero_end = off; off = std::max(off, data_base);
  w.pos_row = off; off = up256(off + (size_t)n * 4);
  w.pos_pair = off; off = up256(off + (size_t)n * 4);
  w.routes = off; off = up256(off + (size_t)n * 4);
  w.ranks = off; off = up256(off + (size_t)n * 4);
  w.bucket = off; off = up256(off + (R > 0 ? (size_t)std::min(n, kMaxKeys) * kShrinkRows * 4 : 0));
  w.tiles = off; off = up256(off + (size_t)c.max_mtiles * 16);
  w.n_tiles = off; off = up256(off + 16);
  w.t = off; off = up256(off + (c.t_splits_ws > 1 ? (size_t)c.t_splits_ws * n * R * 4 : 0));
  w.t_final = off; off = up256(off + (size_t)n * R * 4);
  w.tt = off; off = up256(off + (size_t)n * R * 4);  // [n][2R] bf16
  w.partials = off;
  off = up256(off + (size_t)c.partial_slots * c.to * c.tr * 4);
  w.total = off;
  return w;
}

constexpr uint32_t kMaxRows = 16384;
constexpr uint32_t kMaxRank = 256;

// ------------------------------------------------------------ validation
int check_dtype(int32_t dtype, const char *what) {
  if (dtype != LORA_F32 && dtype != LORA_BF16)
    return fail(LORA_ERR_DTYPE, "%s: dtype %d is neither LORA_F32 (0) nor LORA_BF16 (1)", what, dtype);
  return LORA_OK;
}

// Checks shared by every call on a [n_out x k_in] projection.
int check_proj(const char *what, int32_t dtype, uint32_t n_out, uint32_t k_in, uint32_t n,
               uint32_t x_row_stride, uint32_t y_row_stride, uint32_t w_row_stride) {
  if (int e = check_dtype(dtype, what)) return e;
  if (n_out == 0 || k_in == 0)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: both dimensions must be >= 1", what, n_out, k_in);
  if (n > kMaxRows)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: n %u rows exceeds the limit %u", what, n_out,
                k_in, n, kMaxRows);
  if (x_row_stride < k_in)
    return fail(LORA_ERR_STRIDE, "%s: [n_out %u x k_in %u]: x_row_stride %u < k_in %u", what, n_out, k_in,
                x_row_stride, k_in);
  if (y_row_stride < n_out)
    return fail(LORA_ERR_STRIDE, "%s: [n_out %u x k_in %u]: y_row_stride %u < n_out %u", what, n_out, k_in,
                y_row_stride, n_out);
  if (w_row_stride < k_in)
    return fail(LORA_ERR_STRIDE, "%s: [n_out %u x k_in %u]: w_row_stride %u < k_in %u", what, n_out, k_in,
                w_row_stride, k_in);
  if (dtype == LORA_BF16) {
    if (k_in % 8 || n_out % 8)
      return fail(LORA_ERR_UNSUPPORTED,
                  "%s: [n_out %u x k_in %u]: bf16 needs n_out and k_in to be multiples of 8", what, n_out,
                  k_in);
    if (x_row_stride % 8 || y_row_stride % 8 || w_row_stride % 8)
      return fail(LORA_ERR_UNSUPPORTED,
                  "%s: [n_out %u x k_in %u]: bf16 needs row strides that are multiples of 8 "
                  "(x_row_stride %u, y_row_stride %u, w_row_stride %u)",
                  what, n_out, k_in, x_row_stride, y_row_stride, w_row_stride);
  }
  return LORA_OK;
}

int check_rank(const char *what, int32_t dtype, uint32_t n_out, uint32_t k_in, uint32_t R) {
  if (R == 0 || R > kMaxRank)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u] at max_rank %u: max_rank must be in 1..%u", what,
                n_out, k_in, R, kMaxRank);
  if (dtype == LORA_BF16 && R % 16)
    return fail(LORA_ERR_UNSUPPORTED,
                "%s: [n_out %u x k_in %u] at max_rank %u: bf16 pools must pad max_rank to a multiple of 16",
                what, n_out, k_in, R);
  return LORA_OK;
}

int check_route(const char *what, const lora_route *r, int32_t dtype, uint32_t n_out, uint32_t k_in) {
  if (!r->a_table || !r->b_table || !r->scale_table)
    return fail(LORA_ERR_NULL_PTR, "%s: route tables must be non-NULL (a_table %p, b_table %p, scale_table %p)",
                what, (const void *)r->a_table, (const void *)r->b_table, (const void *)r->scale_table);
  if (r->dtype != dtype)
    return fail(LORA_ERR_DTYPE, "%s: route dtype %d differs from the call's dtype %d", what, r->dtype, dtype);
  if (r->k_in != k_in || r->n_out != n_out)
    return fail(LORA_ERR_SHAPE, "%s: route is [n_out %u x k_in %u] but the projection is [n_out %u x k_in %u]",
                what, r->n_out, r->k_in, n_out, k_in);
  if (r->max_loras == 0 || r->max_loras + 1 > (uint32_t)kMaxKeys)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: max_loras %u must be in 1..%d", what, n_out, k_in,
                r->max_loras, kMaxKeys - 1);
  return check_rank(what, dtype, n_out, k_in, r->max_rank);
}

RouteDev route_dev(const lora_route *r) {
  RouteDev d{};
  if (r) {
    d.a_table = r->a_table;
    d.b_table = r->b_table;
    d.scale_table = r->scale_table;
    d.max_loras = (int)r->max_loras;
    d.n_experts = 1;
    d.R = (int)r->max_rank;
  }
  return d;
}

// A MoE route against the call's shape; fills *rd (all zero for a NULL
// route, a base-only call).
int check_route_moe(const char *what, const lora_route_moe *route, int32_t dtype, uint32_t n_experts,
                    uint32_t n_out, uint32_t k_in, RouteDev *rd) {
  *rd = RouteDev{};
  if (!route) return LORA_OK;
  if (!route->a_table || !route->b_table || !route->scale_table)
    return fail(LORA_ERR_NULL_PTR, "%s: route tables must be non-NULL (a_table %p, b_table %p, scale_table %p)",
                what, (const void *)route->a_table, (const void *)route->b_table,
                (const void *)route->scale_table);
  if (route->dtype != dtype)
    return fail(LORA_ERR_DTYPE, "%s: route dtype %d differs from the call's dtype %d", what, route->dtype, dtype);
  if (route->k_in != k_in || route->n_out != n_out || route->n_experts != n_experts)
    return fail(LORA_ERR_SHAPE,
                "%s: route is [n_out %u x k_in %u] over %u experts but the call is [n_out %u x k_in %u] over %u",
                what, route->n_out, route->k_in, route->n_experts, n_out, k_in, n_experts);
  if (n_experts == 0 || route->max_loras == 0 || (uint64_t)n_experts * (route->max_loras + 1) > (uint64_t)kMaxKeys)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: n_experts %u x (max_loras %u + 1) must be in 1..%d", what,
                n_out, k_in, n_experts, route->max_loras, kMaxKeys);
  if (int e = check_rank(what, dtype, n_out, k_in, route->max_rank)) return e;
  rd->a_table = route->a_table;
  rd->b_table = route->b_table;
  rd->scale_table = route->scale_table;
  rd->max_loras = (int)route->max_loras;
  rd->n_experts = (int)n_experts;
  rd->R = (int)route->max_rank;
  return LORA_OK;
}

// Checks of a W_experts operand: expert_stride covers one expert's matrix.
int check_experts(const char *what, int32_t dtype, uint32_t n_experts, uint32_t n_out, uint32_t k_in,
                  uint64_t expert_stride, uint32_t w_row_stride) {
  if (n_experts == 0 || (uint64_t)n_experts > (uint64_t)kMaxKeys)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: n_experts %u must be in 1..%d", what, n_out, k_in,
                n_experts, kMaxKeys);
  if (expert_stride < (uint64_t)(n_out - 1) * w_row_stride + k_in && n_experts > 1)
    return fail(LORA_ERR_STRIDE, "%s: [n_out %u x k_in %u]: expert_stride %llu is smaller than one expert", what,
                n_out, k_in, (unsigned long long)expert_stride);
  if (dtype == LORA_BF16 && expert_stride % 8)
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs expert_stride %llu to be a multiple of 8", what,
                (unsigned long long)expert_stride);
  return LORA_OK;
}

// Shared by the grouped shrink and expand-fold: the route, the row count
// and the pointers (the input rows `in`, the output `out`).
int check_grouped_call(const char *what, const lora_route_moe *route, uint32_t n, const void *in,
                       const int32_t *expert_offsets, const int32_t *seq_slot, const void *out,
                       uint32_t x_row_stride, uint32_t y_row_stride, bool shrink, RouteDev *rd) {
  if (!route) return fail(LORA_ERR_NULL_PTR, "%s: route is NULL", what);
  const uint32_t k_in = route->k_in, n_out = route->n_out;
  if (int e = check_proj(what, route->dtype, n_out, k_in, n, shrink ? x_row_stride : k_in,
                         shrink ? n_out : y_row_stride, k_in))
    return e;
  if (route->n_experts == 0)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: route n_experts must be >= 1", what, n_out, k_in);
  if (int e = check_route_moe(what, route, route->dtype, route->n_experts, n_out, k_in, rd)) return e;
  if (n == 0) return LORA_OK;
  if (!in || !expert_offsets || !seq_slot || !out)
    return fail(LORA_ERR_NULL_PTR,
                "%s: [n_out %u x k_in %u]: %s %p, expert_offsets %p, seq_slot %p, %s %p must be non-NULL", what,
                n_out, k_in, shrink ? "x" : "t", in, (const void *)expert_offsets, (const void *)seq_slot,
                shrink ? "t" : "y", out);
  return LORA_OK;
}

Routing routing_grouped(const int32_t *expert_offsets, const int32_t *seq_slot, uint32_t n_experts) {
  Routing rt{};
  rt.mode = kModeMoeGrouped;
  rt.expert_offsets = expert_offsets;
  rt.seq_slot = seq_slot;
  rt.n_experts = (int)n_experts;
  rt.top_k = 1;
  return rt;
}

// A further stack level's shrink: k split like the fused paths' shrink (a
// function of n and k_in only), its partials summed by the last arrival.
int stack_shrink_splits(int n, int k_in) {
  return clampi(512 / ((n + kShrinkRows - 1) / kShrinkRows), 1, std::min(kMaxShrinkSplits, std::max(1, k_in / 256)));
}

// Workspace of one further stack level: arrival counters (zero between
// calls), k-split partials, and t [n][R].  Sized for any pool of up to n
// slots, so the offsets depend on (n, R, k_in) only.
struct StackLevelLayout {
  size_t counters, partials, t, total;
};
StackLevelLayout stack_level_layout(int32_t dtype, int n, int R, int k_in) {
  StackLevelLayout w{};
  size_t off = 0;
  const int ks = dtype == LORA_BF16 ? stack_shrink_splits(n, k_in) : 1;
  w.counters = off; off = up256(off + (ks > 1 ? (size_t)((n + kShrinkRows - 1) / kShrinkRows + n) * 4 : 0));
  w.partials = off; off = up256(off + (ks > 1 ? (size_t)ks * n * R * 4 : 0));
  w.t = off; off = up256(off + (size_t)n * R * 4);
  w.total = off;
  return w;
}

// The workspace the first level of a stack takes: the fused apply's, for any
// first-level rank up to max_rank (bf16 ranks are multiples of 16).
size_t stack_apply_bytes(int32_t dtype, int n, int n_out, int k_in, int max_rank) {
  if (dtype != LORA_BF16) return 0;
  size_t most = 0;
  for (int R = 0; R <= max_rank; R += 16) {
    const Cfg c = choose_cfg(LORA_OP_APPLY, n, n_out, k_in, 1, R, R ? n : 0);
    most = std::max(most, ws_layout(c, n, R, k_in).total);
  }
  return up256(most);
}

Routing routing_decode(const int32_t *seq_slot) {
  Routing rt{};
  rt.mode = kModeDecode;
  rt.seq_slot = seq_slot;
  rt.n_experts = 1;
  rt.top_k = 1;
  return rt;
}

// The f32 path is one kernel; it records the profile events as an empty prep
// followed by the kernel, like the fused path.
template <typename F>
int run_f32_timed(const char *what, F launch, hipStream_t st) {
  prof_record(0, st);
  prof_record(1, st);
  const int e = launch_status(launch(), what);
  prof_record(2, st);
  prof_record(3, st);
  return e;
}

// The bf16 fused path shared by the three apply entry points.
// `stack` (or null): an adapter stack's further levels, whose t are ready;
// on the decode path the epilogue folds them in and *stack_folded is set.
int run_fused(const char *what, int op, const Routing &rt, const RouteDev &rd, bool has_lora,
              uint32_t n_out, uint32_t k_in, const void *W, long long w_group_stride,
              uint32_t w_row_stride, const void *x, uint32_t x_row_stride, uint32_t n, void *y,
              uint32_t y_row_stride, void *workspace, size_t workspace_bytes, int groups,
              hipStream_t st, const StackFold *stack = nullptr, bool *stack_folded = nullptr,
              size_t data_base = 0) {
  const int R = has_lora ? rd.R : 0;
  const int n_pairs = has_lora ? rd.max_loras * rd.n_experts : 0;
  const Cfg c = choose_cfg(op, (int)n, (int)n_out, (int)k_in, groups, R, n_pairs);
  const WsLayout L = ws_layout(c, (int)n, R, (int)k_in, data_base);
  if (!workspace || workspace_bytes < L.total || (data_base && L.zero_end > data_base))
    return fail(LORA_ERR_WORKSPACE,
                "%s: [n_out %u x k_in %u] at max_rank %d, n %u: workspace %p of %zu bytes, %zu needed%s", what,
                n_out, k_in, R, n, workspace, workspace_bytes, L.total,
                data_base && L.zero_end > data_base ? " (its counter words exceed the shared scratch's zero region)"
                                                    : "");
  if (!aligned16(workspace))
    return fail(LORA_ERR_UNSUPPORTED, "%s: workspace %p is not 16-byte aligned", what, workspace);
  char *ws = (char *)workspace;
  if (c.decode) {
    DecodeArgs da{};
    da.W = (const u16 *)W;
    da.w_row_stride = (int)w_row_stride;
    da.x = (const u16 *)x;
    da.x_row_stride = (int)x_row_stride;
    da.y = (u16 *)y;
    da.y_row_stride = (int)y_row_stride;
    da.n_out = (int)n_out;
    da.k_in = (int)k_in;
    da.n = (int)n;
    da.rd = rd;
    da.seq_slot = rt.seq_slot;
    da.has_lora = has_lora;
    da.R = R;
    da.S = c.splits;
    da.n_tiles = c.n_ntiles;
    da.tile_out = c.to;
    da.partials = (float *)(ws + L.partials);
    da.t = (const float *)(ws + L.t_final);
    da.t_part = (float *)(ws + L.t);
    da.tile_cnt = (unsigned *)(ws + L.tile_cnt);
    // The shrink rides the decode launch when its units (pool slots x
    // 16-rank blocks, one per carrier workgroup) fit on a few tiles: those
    // workgroups, the first ones of the launch, never wait before they
    // count themselves in, and every other workgroup waits for them, so
    // they must all be resident at once: at most kDecodeMaxCarrierWgs of
    // them, and at most half the device's compute units (a workgroup of
    // this kernel takes a whole CU).  Otherwise a prep launch computes t
    // first.
    //
    // A tile's contributors share their partials through one XCD's L2 when
    // the chip's round-robin hand-out of workgroups to its 8 XCDs puts them
    // on one XCD (DecodeArgs::xcd_local): tiles in multiples of 8, and the
    // whole launch resident at once (a workgroup per CU), so that every
    // contributor of a tile runs alongside the others whatever their places
    // in the launch.  Each XCD then fetches every k range of x instead of
    // one; measured, that costs more than the L2 saves once the launch
    // fills the chip (64 x 4096 x 4096: 16.0 -> 17.4 us a step), and less on
    // launches of at most half the CUs (36 x 4096 x 1024: 11.6 -> 11.1 us),
    // which alone take it.  Carriers are then the first 8 S
    // ceil(unit_tiles / 8) workgroups.
    const int cus = current_cus();
    da.xcd_local = c.n_ntiles % 8 == 0 && 2 * c.n_ntiles * c.splits <= cus ? 1 : 0;
    const int units = R > 0 ? rd.max_loras * (R / 16) : 0;
    const int ut = units;
    const int carrier_wgs = (da.xcd_local ? (ut + 7) / 8 * 8 : ut) * c.splits;
    const int carrier_cap = std::min(kDecodeMaxCarrierWgs, cus / 2);
    da.unit_tiles = R > 0 && R <= 64 && rd.max_loras * R <= kDecodeUnitRanks && ut <= c.n_ntiles &&
                            carrier_wgs <= carrier_cap
                        ? ut
                        : 0;
    const bool fold = stack && stack->n_levels > 0 && has_lora;
    prof_record(0, st);
    if (has_lora && da.unit_tiles == 0) {  // the shrink: t [n][R] for the rows that resolve
      PrepArgs pa{};
      pa.rd = rd;
      pa.rt = rt;
      pa.has_lora = true;
      pa.x = (const u16 *)x;
      pa.x_stride = (int)x_row_stride;
      pa.k_in = (int)k_in;
      pa.n = (int)n;
      pa.k_splits = c.t_splits;
      pa.t = (float *)(ws + L.t);
      pa.t_final = (float *)(ws + L.t_final);
      pa.counters = (unsigned *)(ws + L.shrink_counters);
      pa.n_pairs = n_pairs;
      pa.do_plan = 0;
      pa.n_units = c.units;
      if (int e = launch_status(launch_prep(pa, st), what)) return e;
    }
    prof_record(1, st);
    const int e = launch_status(launch_decode(da, fold ? stack : nullptr, st), what);
    if (stack_folded) *stack_folded = fold && e == LORA_OK;
    prof_record(2, st);
    prof_record(3, st);
    return e;
  }
  PlanDev plan{(int *)(ws + L.pos_row), (int *)(ws + L.pos_pair), (int4 *)(ws + L.tiles),
               (int *)(ws + L.n_tiles)};

  PrepArgs pa{};
  pa.rd = rd;
  pa.rt = rt;
  pa.has_lora = has_lora;
  pa.x = (const u16 *)x;
  pa.x_stride = (int)x_row_stride;
  pa.k_in = (int)k_in;
  pa.n = (int)n;
  pa.t = (float *)(ws + L.t);
  pa.t_final = (float *)(ws + L.t_final);
  pa.tt = R > 0 ? (u16 *)(ws + L.tt) : nullptr;
  // a segmented call over at most 64 segments needs no per-row routes: the
  // plan and the shrink units work from the segments (up to 4096 rows, where
  // a unit's fallback for bounds that decrease, which routes every row into
  // LDS, still leaves two units per CU)
  const bool seg_direct = rt.mode == kModeSegmented && rt.n_seg <= 64 && n <= 4096;
  pa.seg_units = seg_direct ? 1 : 0;
  pa.routes = seg_direct ? nullptr : (int *)(ws + L.routes);
  if (R > 0 && !seg_direct) {
    pa.ranks = (int *)(ws + L.ranks);
    // the pairs' row buckets spare a unit its scan of the whole batch:
    // worth it on large batches routed by row (measured: the MoE gather's
    // 3072 rows, step 121.9 -> 118.7 us); a segmented or grouped call scans
    // only its segment or expert range (and the grouped MoE ran 3 us slower
    // with the buckets)
    const bool whole_scan = rt.mode != kModeSegmented && rt.mode != kModeMoeGrouped;
    pa.bucket = whole_scan && n >= 1024 ? (int *)(ws + L.bucket) : nullptr;
    pa.bucket_pairs = std::min((int)n, kMaxKeys);
    pa.pair_cnt = (unsigned *)(ws + L.pair_cnt);
    pa.prep_done = pa.pair_cnt + kMaxKeys;  // past every pair count, at a fixed word
  }
  pa.counters = (unsigned *)(ws + L.shrink_counters);
  pa.k_splits = c.t_splits;
  pa.n_pairs = n_pairs;
  pa.do_plan = 1;
  // The shrink units' register loads and the plan behind the units (the last
  // workgroup when they all fit one round)
  // (measured against the LDS-DMA units and the plan first, steps: segmented
  // prefill 186.5 -> 174.4 us, fused gate/up ~109 -> 105.3 us) suit every
  // call but the MoE ones, whose many small units run better three to a CU
  // with the plan beside them (gather 120.8 against 127.7 us, grouped 180
  // against 199.5 us).
  const bool moe_op = op == LORA_OP_MOE_GATHER || op == LORA_OP_MOE_GROUPED;
  pa.reg_units = moe_op ? 0 : 1;
  pa.plan = plan;
  pa.tile_rows = c.tr;
  pa.n_units = c.units;
  // the plan right after the units of the first round (two per CU), before
  // the unit slots the batch may not need
  pa.plan_at = moe_op ? 0 : std::min(pa.n_units * pa.k_splits, 2 * current_cus());
  prof_record(0, st);
  if (int e = launch_status(launch_prep(pa, st), what)) return e;
  prof_record(1, st);

  GemmArgs ga{};
  ga.W = (const u16 *)W;
  ga.w_group_stride = w_group_stride;
  ga.w_row_stride = (int)w_row_stride;
  ga.x = (const u16 *)x;
  ga.x_row_stride = (int)x_row_stride;
  ga.y = (u16 *)y;
  ga.y_row_stride = (int)y_row_stride;
  ga.n_out = (int)n_out;
  ga.k_in = (int)k_in;
  ga.plan = plan;
  ga.max_mtiles = c.max_mtiles;
  ga.n_ntiles = c.n_ntiles;
  ga.has_lora = has_lora;
  ga.b_table = rd.b_table;
  ga.scale_table = rd.scale_table;
  ga.n_experts = rd.n_experts > 0 ? rd.n_experts : 1;
  ga.tt = pa.tt;
  ga.R = R;
  ga.splits = c.splits;
  ga.partials = (float *)(ws + L.partials);
  ga.counters = (unsigned *)(ws + L.counters);
  const int e = launch_status(launch_gemm(ga, c.to, c.tr, st), what);
  prof_record(2, st);
  prof_record(3, st);
  return e;
}

// The current device's scratch entry: the array's address is looked up once
// per device, with that device current.
int scratch_dev(const char *what, ScratchDev **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LORA_ERR_LAUNCH, "%s: no HIP device is current", what);
  if (dev < 0 || dev >= 64) return fail(LORA_ERR_LAUNCH, "%s: device index %d out of range", what, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDev &d = g_scratch[dev];
  if (!d.ptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LORA_ERR_LAUNCH, "%s: hipGetSymbolAddress of the scratch array on device %d failed: %s", what,
                  dev, hipGetErrorString(e));
    d.ptr = p;
  }
  *out = &d;
  return LORA_OK;
}

}  // namespace

extern "C" {

const char *lora_last_error(void) { return g_err; }

int lora_set_profile_events(void *const *events, uint32_t n) {
  clear_err();
  if (n == 0) {
    g_prof_on = false;
    return LORA_OK;
  }
  if (n < 4 || !events || !events[0] || !events[1] || !events[2] || !events[3])
    return fail(LORA_ERR_NULL_PTR, "lora_set_profile_events: need 4 non-NULL events, got %u", n);
  for (int i = 0; i < 4; ++i) g_prof[i] = (hipEvent_t)events[i];
  g_prof_on = true;
  return LORA_OK;
}

const char *lora_version(void) { return "lora_mi355x 0.1 (gfx950)"; }

int lora_init(void) {
  clear_err();
  if (int e = check_device("lora_init")) return e;
  ScratchDev *d = nullptr;
  return scratch_dev("lora_init", &d);
}

double lora_scale(double adapter_scale, double alpha, uint32_t rank, int32_t rslora) {
  if (alpha == 0.0) return adapter_scale;
  if (rank == 0) return 0.0;
  return rslora ? adapter_scale * alpha / std::sqrt((double)rank) : adapter_scale * alpha / (double)rank;
}

int lora_scale_table(uint32_t n_adapters, const double *adapter_scale, const double *alpha,
                     const uint32_t *rank, const int32_t *rslora, uint32_t max_loras, float *out) {
  clear_err();
  if (!out || (n_adapters && (!adapter_scale || !alpha || !rank || !rslora)))
    return fail(LORA_ERR_NULL_PTR, "lora_scale_table: NULL array for %u adapters", n_adapters);
  for (uint32_t k = 0; k < n_adapters && k < max_loras; ++k)
    if (rank[k] == 0) return fail(LORA_ERR_SHAPE, "lora_scale_table: adapter %u has rank 0", k);
  for (uint32_t k = 0; k < max_loras; ++k)
    out[k] = k < n_adapters ? (float)lora_scale(adapter_scale[k], alpha[k], rank[k], rslora[k]) : 0.0f;
  return LORA_OK;
}

int lora_build_seq_slot(const int32_t *adapter_slots, uint32_t n, uint32_t padded_n, int32_t active,
                        int32_t *out) {
  clear_err();
  if ((n && !adapter_slots) || (padded_n && !out))
    return fail(LORA_ERR_NULL_PTR, "lora_build_seq_slot: NULL array (n %u, padded_n %u)", n, padded_n);
  if (n > padded_n)
    return fail(LORA_ERR_SHAPE, "lora_build_seq_slot: n %u real rows exceed padded_n %u", n, padded_n);
  for (uint32_t i = 0; i < padded_n; ++i) out[i] = i < n ? (adapter_slots[i] >= 0 ? adapter_slots[i] : active) : -1;
  return LORA_OK;
}

size_t lora_workspace_bytes(int32_t op, int32_t dtype, uint32_t n_rows, uint32_t n_out, uint32_t k_in,
                            uint32_t max_rank, uint32_t n_groups) {
  if (op == LORA_OP_STACK) {
    if (n_rows == 0) return 0;
    const size_t levels = n_groups ? n_groups : 1;
    return stack_apply_bytes(dtype, (int)n_rows, (int)n_out, (int)k_in, (int)max_rank) +
           (levels - 1) * stack_level_layout(dtype, (int)n_rows, (int)max_rank, (int)k_in).total;
  }
  if (dtype != LORA_BF16 || n_rows == 0) return 0;
  // pairs are counted generously (any table size the call may use), and the
  // base-only call of the same shape fits too
  const int groups = (int)(n_groups ? n_groups : 1);
  const Cfg c = choose_cfg(op, (int)n_rows, (int)n_out, (int)k_in, groups, (int)max_rank,
                           max_rank ? (int)n_rows : 0);
  const Cfg c0 = choose_cfg(op, (int)n_rows, (int)n_out, (int)k_in, groups, 0, 0);
  return std::max(ws_layout(c, (int)n_rows, (int)max_rank, (int)k_in).total,
                  ws_layout(c0, (int)n_rows, 0, (int)k_in).total);
}

int lora_shrink(const lora_route *route, const void *x, uint32_t x_row_stride, const int32_t *seq_slot,
                uint32_t n, float *t, void *stream) {
  clear_err();
  const char *what = "lora_shrink";
  if (!route) return fail(LORA_ERR_NULL_PTR, "%s: route is NULL", what);
  if (int e = check_proj(what, route->dtype, route->n_out, route->k_in, n, x_row_stride, route->n_out,
                         route->k_in))
    return e;
  if (int e = check_route(what, route, route->dtype, route->n_out, route->k_in)) return e;
  if (n == 0) return LORA_OK;
  if (!x || !seq_slot || !t)
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: x %p, seq_slot %p, t %p must be non-NULL", what,
                route->n_out, route->k_in, x, (const void *)seq_slot, (void *)t);
  if (route->dtype == LORA_BF16 && (!aligned16(x) || !aligned16(t)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned x %p and t %p", what, x, (void *)t);
  if (int e = check_device(what)) return e;
  const RouteDev rd = route_dev(route);
  const Routing rt = routing_decode(seq_slot);
  hipStream_t st = (hipStream_t)stream;
  if (route->dtype == LORA_F32)
    return launch_status(launch_shrink_f32(rd, rt, (const float *)x, (int)x_row_stride, (int)route->k_in, (int)n,
                                           t, st),
                         what);
  if (n <= (uint32_t)kBgmvMaxRows)  // decode-sized: by pool slot, each A read once
    return launch_status(launch_bgmv_shrink(rd, seq_slot, (int)n, (const u16 *)x, (int)x_row_stride,
                                            (int)route->k_in, t, st),
                         what);
  PrepArgs pa{};
  pa.rd = rd;
  pa.rt = rt;
  pa.has_lora = true;
  pa.x = (const u16 *)x;
  pa.x_stride = (int)x_row_stride;
  pa.k_in = (int)route->k_in;
  pa.n = (int)n;
  pa.t = t;
  pa.t_final = t;
  pa.k_splits = 1;  // t is the caller's [n][max_rank] output: whole k per unit
  pa.n_pairs = (int)route->max_loras;
  pa.do_plan = 0;
  pa.n_units = (int)((n + kShrinkRows - 1) / kShrinkRows) + (int)std::min<uint32_t>(n, route->max_loras);
  return launch_status(launch_prep(pa, st), what);
}

int lora_expand_fold(const lora_route *route, const float *t, const int32_t *seq_slot, uint32_t n, void *y,
                     uint32_t y_row_stride, void *stream) {
  clear_err();
  const char *what = "lora_expand_fold";
  if (!route) return fail(LORA_ERR_NULL_PTR, "%s: route is NULL", what);
  if (int e = check_proj(what, route->dtype, route->n_out, route->k_in, n, route->k_in, y_row_stride,
                         route->k_in))
    return e;
  if (int e = check_route(what, route, route->dtype, route->n_out, route->k_in)) return e;
  if (n == 0) return LORA_OK;
  if (!t || !seq_slot || !y)
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: t %p, seq_slot %p, y %p must be non-NULL", what,
                route->n_out, route->k_in, (const void *)t, (const void *)seq_slot, y);
  if (int e = check_device(what)) return e;
  // decode-sized bf16 batches: by pool slot, each B read once, 16-byte y
  // pieces (which need 16-byte aligned rows)
  if (route->dtype == LORA_BF16 && n <= (uint32_t)kBgmvMaxRows && aligned16(y) && aligned16(t))
    return launch_status(launch_bgmv_expand(route_dev(route), seq_slot, (int)n, t, (u16 *)y, (int)y_row_stride,
                                            (int)route->n_out, (hipStream_t)stream),
                         what);
  return launch_status(launch_expand_fold(route_dev(route), route->dtype, routing_decode(seq_slot), t, y,
                                          (int)y_row_stride, (int)route->n_out, (int)n, (hipStream_t)stream),
                       what);
}

int lora_apply(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W, uint32_t w_row_stride,
               const lora_route *route, const void *x, uint32_t x_row_stride, const int32_t *seq_slot,
               uint32_t n, void *y, uint32_t y_row_stride, void *workspace, size_t workspace_bytes,
               void *stream) {
  clear_err();
  const char *what = "lora_apply";
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (route) {
    if (int e = check_route(what, route, dtype, n_out, k_in)) return e;
  }
  if (n == 0) return LORA_OK;
  if (!W || !x || !y || (route && !seq_slot))
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: W %p, x %p, y %p%s must be non-NULL", what, n_out,
                k_in, W, x, y, route ? " and seq_slot" : "");
  if (dtype == LORA_BF16 && (!aligned16(W) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W %p, x %p, y %p", what, W, x, y);
  if (int e = check_device(what)) return e;
  const RouteDev rd = route_dev(route);
  const Routing rt = routing_decode(route ? seq_slot : nullptr);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LORA_F32)
    return run_f32_timed(what, [&] { return launch_apply_f32(rd, rt, route != nullptr, (const float *)W, 0, (int)w_row_stride,
                                          (const float *)x, (int)x_row_stride, (int)k_in, (int)n_out, (int)n,
                                          (float *)y, (int)y_row_stride, st); }, st);
  return run_fused(what, LORA_OP_APPLY, rt, rd, route != nullptr, n_out, k_in, W, 0, w_row_stride, x,
                   x_row_stride, n, y, y_row_stride, workspace, workspace_bytes, 1, st);
}

int lora_apply_noalloc(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W, uint32_t w_row_stride,
                       const lora_route *route, const void *x, uint32_t x_row_stride, const int32_t *seq_slot,
                       uint32_t n, void *y, uint32_t y_row_stride, void *stream) {
  clear_err();
  const char *what = "lora_apply_noalloc";
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (route) {
    if (int e = check_route(what, route, dtype, n_out, k_in)) return e;
  }
  if (n == 0) return LORA_OK;
  if (!W || !x || !y || (route && !seq_slot))
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: W %p, x %p, y %p%s must be non-NULL", what, n_out,
                k_in, W, x, y, route ? " and seq_slot" : "");
  if (dtype == LORA_BF16 && (!aligned16(W) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W %p, x %p, y %p", what, W, x, y);
  const RouteDev rd = route_dev(route);
  if (dtype == LORA_BF16) {  // the size check, before any HIP call
    const int R = route ? rd.R : 0;
    const Cfg c = choose_cfg(LORA_OP_APPLY, (int)n, (int)n_out, (int)k_in, 1, R,
                             route ? rd.max_loras * rd.n_experts : 0);
    const WsLayout L = ws_layout(c, (int)n, R, (int)k_in, kScratchZeroBytes);
    if (L.total > kScratchBytes || L.zero_end > kScratchZeroBytes)
      return fail(LORA_ERR_WORKSPACE,
                  "%s: [n_out %u x k_in %u] at max_rank %d, n %u needs %zu bytes of scratch; the limit is %zu", what,
                  n_out, k_in, R, n, L.total, kScratchBytes);
  }
  if (int e = check_device(what)) return e;
  const Routing rt = routing_decode(route ? seq_slot : nullptr);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LORA_F32)  // (this path uses no workspace)
    return run_f32_timed(what, [&] { return launch_apply_f32(rd, rt, route != nullptr, (const float *)W, 0, (int)w_row_stride,
                                          (const float *)x, (int)x_row_stride, (int)k_in, (int)n_out, (int)n,
                                          (float *)y, (int)y_row_stride, st); }, st);
  ScratchDev *d = nullptr;
  if (int e = scratch_dev(what, &d)) return e;
  // The zero region is cleared by the first call on the device, and by every
  // call made under stream capture (a graph then carries its own clear).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess)
    return fail(LORA_ERR_LAUNCH, "%s: cannot query the stream's capture status", what);
  const bool capturing = cap != hipStreamCaptureStatusNone;
  bool clear = capturing;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!d->zeroed) {
      clear = true;
      if (!capturing) d->zeroed = true;
    }
  }
  if (clear) {
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, st, (uint4 *)d->ptr, kScratchZeroBytes / 16);
    if (int e = launch_status(hipGetLastError(), what)) return e;
  }
  return run_fused(what, LORA_OP_APPLY, rt, rd, route != nullptr, n_out, k_in, W, 0, w_row_stride, x,
                   x_row_stride, n, y, y_row_stride, d->ptr, kScratchBytes, 1, st, nullptr, nullptr,
                   kScratchZeroBytes);
}

int lora_apply_segmented(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W, uint32_t w_row_stride,
                         const lora_route *route, const void *x, uint32_t x_row_stride,
                         const int32_t *seg_indptr, const int32_t *seg_slot, uint32_t n_seg, uint32_t n, void *y,
                         uint32_t y_row_stride, void *workspace, size_t workspace_bytes, void *stream) {
  clear_err();
  const char *what = "lora_apply_segmented";
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (route) {
    if (int e = check_route(what, route, dtype, n_out, k_in)) return e;
  }
  if (n == 0) return LORA_OK;
  if (!W || !x || !y || !seg_indptr || (n_seg && !seg_slot))
    return fail(LORA_ERR_NULL_PTR,
                "%s: [n_out %u x k_in %u]: W %p, x %p, y %p, seg_indptr %p, seg_slot %p must be non-NULL", what,
                n_out, k_in, W, x, y, (const void *)seg_indptr, (const void *)seg_slot);
  if (dtype == LORA_BF16 && (!aligned16(W) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W %p, x %p, y %p", what, W, x, y);
  if (int e = check_device(what)) return e;
  const RouteDev rd = route_dev(route);
  Routing rt{};
  rt.mode = kModeSegmented;
  rt.seg_indptr = seg_indptr;
  rt.seg_slot = seg_slot;
  rt.n_seg = (int)n_seg;
  rt.n_experts = 1;
  rt.top_k = 1;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LORA_F32)
    return run_f32_timed(what, [&] { return launch_apply_f32(rd, rt, route != nullptr, (const float *)W, 0, (int)w_row_stride,
                                          (const float *)x, (int)x_row_stride, (int)k_in, (int)n_out, (int)n,
                                          (float *)y, (int)y_row_stride, st); }, st);
  return run_fused(what, LORA_OP_SEGMENTED, rt, rd, route != nullptr, n_out, k_in, W, 0, w_row_stride, x,
                   x_row_stride, n, y, y_row_stride, workspace, workspace_bytes, 1, st);
}

int lora_apply_moe_gather(int32_t dtype, uint32_t n_experts, uint32_t n_out, uint32_t k_in,
                          const void *W_experts, uint64_t expert_stride, uint32_t w_row_stride,
                          const lora_route_moe *route, const void *x, uint32_t x_row_stride,
                          const int32_t *indices, uint32_t top_k, const int32_t *token_slot, uint32_t n_tokens,
                          void *y, uint32_t y_row_stride, void *workspace, size_t workspace_bytes,
                          void *stream) {
  clear_err();
  const char *what = "lora_apply_moe_gather";
  if (top_k == 0 || n_experts == 0)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: n_experts %u and top_k %u must be >= 1", what, n_out,
                k_in, n_experts, top_k);
  const uint64_t rows64 = (uint64_t)n_tokens * top_k;
  if (rows64 > kMaxRows)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: n_tokens %u x top_k %u rows exceed the limit %u", what,
                n_out, k_in, n_tokens, top_k, kMaxRows);
  const uint32_t n = (uint32_t)rows64;
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (int e = check_experts(what, dtype, n_experts, n_out, k_in, expert_stride, w_row_stride)) return e;
  RouteDev rd{};
  if (int e = check_route_moe(what, route, dtype, n_experts, n_out, k_in, &rd)) return e;
  if (n == 0) return LORA_OK;
  if (!W_experts || !x || !y || !indices || (route && !token_slot))
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: W_experts, x, y, indices%s must be non-NULL", what,
                n_out, k_in, route ? ", token_slot" : "");
  if (dtype == LORA_BF16 && (!aligned16(W_experts) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W_experts %p, x %p, y %p", what, W_experts,
                x, y);
  if (int e = check_device(what)) return e;
  Routing rt{};
  rt.mode = kModeMoe;
  rt.indices = indices;
  rt.token_slot = token_slot;
  rt.top_k = (int)top_k;
  rt.n_experts = (int)n_experts;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LORA_F32)
    return run_f32_timed(what, [&] { return launch_apply_f32(rd, rt, route != nullptr, (const float *)W_experts,
                                          (long long)expert_stride, (int)w_row_stride, (const float *)x,
                                          (int)x_row_stride, (int)k_in, (int)n_out, (int)n, (float *)y,
                                          (int)y_row_stride, st); }, st);
  return run_fused(what, LORA_OP_MOE_GATHER, rt, rd, route != nullptr, n_out, k_in, W_experts,
                   (long long)expert_stride, w_row_stride, x, x_row_stride, n, y, y_row_stride, workspace,
                   workspace_bytes, (int)n_experts, st);
}

int lora_moe_grouped_shrink(const lora_route_moe *route, const void *x, uint32_t x_row_stride,
                            const int32_t *expert_offsets, const int32_t *seq_slot, uint32_t n, float *t,
                            void *stream) {
  clear_err();
  const char *what = "lora_moe_grouped_shrink";
  RouteDev rd{};
  if (int e = check_grouped_call(what, route, n, x, expert_offsets, seq_slot, t, x_row_stride, 0, true, &rd))
    return e;
  if (n == 0) return LORA_OK;
  if (route->dtype == LORA_BF16 && (!aligned16(x) || !aligned16(t)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned x %p and t %p", what, x, (void *)t);
  if (int e = check_device(what)) return e;
  const Routing rt = routing_grouped(expert_offsets, seq_slot, route->n_experts);
  hipStream_t st = (hipStream_t)stream;
  if (route->dtype == LORA_F32)
    return launch_status(launch_shrink_f32(rd, rt, (const float *)x, (int)x_row_stride, (int)route->k_in, (int)n,
                                           t, st),
                         what);
  const int n_pairs = rd.max_loras * rd.n_experts;
  PrepArgs pa{};
  pa.rd = rd;
  pa.rt = rt;
  pa.has_lora = true;
  pa.x = (const u16 *)x;
  pa.x_stride = (int)x_row_stride;
  pa.k_in = (int)route->k_in;
  pa.n = (int)n;
  pa.t = t;
  pa.t_final = t;
  pa.k_splits = 1;  // t is the caller's [n][max_rank] output: whole k per unit
  pa.n_pairs = n_pairs;
  pa.do_plan = 0;
  pa.n_units = (int)((n + kShrinkRows - 1) / kShrinkRows) + (int)std::min<uint32_t>(n, (uint32_t)n_pairs);
  return launch_status(launch_prep(pa, st), what);
}

int lora_moe_grouped_expand_fold(const lora_route_moe *route, const float *t, const int32_t *expert_offsets,
                                 const int32_t *seq_slot, uint32_t n, void *y, uint32_t y_row_stride,
                                 void *stream) {
  clear_err();
  const char *what = "lora_moe_grouped_expand_fold";
  RouteDev rd{};
  if (int e = check_grouped_call(what, route, n, t, expert_offsets, seq_slot, y, 0, y_row_stride, false, &rd))
    return e;
  if (n == 0) return LORA_OK;
  if (int e = check_device(what)) return e;
  return launch_status(launch_expand_fold(rd, route->dtype, routing_grouped(expert_offsets, seq_slot, route->n_experts),
                                          t, y, (int)y_row_stride, (int)route->n_out, (int)n, (hipStream_t)stream),
                       what);
}

int lora_apply_moe_grouped(int32_t dtype, uint32_t n_experts, uint32_t n_out, uint32_t k_in,
                           const void *W_experts, uint64_t expert_stride, uint32_t w_row_stride,
                           const lora_route_moe *route, const void *x, uint32_t x_row_stride,
                           const int32_t *expert_offsets, const int32_t *seq_slot, uint32_t n, void *y,
                           uint32_t y_row_stride, void *workspace, size_t workspace_bytes, void *stream) {
  clear_err();
  const char *what = "lora_apply_moe_grouped";
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (int e = check_experts(what, dtype, n_experts, n_out, k_in, expert_stride, w_row_stride)) return e;
  RouteDev rd{};
  if (int e = check_route_moe(what, route, dtype, n_experts, n_out, k_in, &rd)) return e;
  if (n == 0) return LORA_OK;
  if (!W_experts || !x || !y || !expert_offsets || (route && !seq_slot))
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: W_experts, x, y, expert_offsets%s must be non-NULL",
                what, n_out, k_in, route ? ", seq_slot" : "");
  if (dtype == LORA_BF16 && (!aligned16(W_experts) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W_experts %p, x %p, y %p", what, W_experts,
                x, y);
  if (int e = check_device(what)) return e;
  const Routing rt = routing_grouped(expert_offsets, route ? seq_slot : nullptr, n_experts);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == LORA_F32)
    return run_f32_timed(what, [&] { return launch_apply_f32(rd, rt, route != nullptr, (const float *)W_experts,
                                          (long long)expert_stride, (int)w_row_stride, (const float *)x,
                                          (int)x_row_stride, (int)k_in, (int)n_out, (int)n, (float *)y,
                                          (int)y_row_stride, st); }, st);
  return run_fused(what, LORA_OP_MOE_GROUPED, rt, rd, route != nullptr, n_out, k_in, W_experts,
                   (long long)expert_stride, w_row_stride, x, x_row_stride, n, y, y_row_stride, workspace,
                   workspace_bytes, (int)n_experts, st);
}

int lora_embedding_pair(int32_t dtype, uint32_t n_vocab, uint32_t n_embd, uint32_t a_rows, uint32_t a_cols,
                        const void *a_file, uint32_t b_rows, uint32_t b_cols, const void *b_file, void *a_out) {
  clear_err();
  const char *what = "lora_embedding_pair";
  if (int e = check_dtype(dtype, what)) return e;
  if (n_vocab != a_rows || n_embd != b_rows || a_cols != b_cols || a_cols == 0)
    return fail(LORA_ERR_SHAPE,
                "%s: embedding [n_vocab %u x n_embd %u]: A_file is [%u x %u] and B_file [%u x %u]; they must be "
                "[n_vocab x rank] and [n_embd x rank] with one rank >= 1",
                what, n_vocab, n_embd, a_rows, a_cols, b_rows, b_cols);
  if (!a_file || !b_file || !a_out)
    return fail(LORA_ERR_NULL_PTR, "%s: a_file %p, b_file %p, a_out %p must be non-NULL", what, a_file, b_file,
                a_out);
  const size_t esz = dtype == LORA_F32 ? 4 : 2;
  const uint32_t rank = a_cols;
  for (uint32_t k = 0; k < rank; ++k)
    for (uint32_t e = 0; e < n_embd; ++e)
      std::memcpy((char *)a_out + ((size_t)k * n_embd + e) * esz, (const char *)b_file + ((size_t)e * rank + k) * esz,
                  esz);
  return LORA_OK;
}

int lora_embed_rows(int32_t dtype, uint32_t n_vocab, uint32_t n_embd, const void *E, uint32_t e_row_stride,
                    const lora_route *route, const int32_t *token_ids, const int32_t *seq_slot, uint32_t n, void *y,
                    uint32_t y_row_stride, void *stream) {
  clear_err();
  const char *what = "lora_embed_rows";
  // a row gather of a [n_vocab x n_embd] matrix: every output row is n_embd long
  if (int e = check_dtype(dtype, what)) return e;
  if (n_vocab == 0 || n_embd == 0)
    return fail(LORA_ERR_SHAPE, "%s: embedding [n_vocab %u x n_embd %u]: both dimensions must be >= 1", what,
                n_vocab, n_embd);
  if (n > kMaxRows)
    return fail(LORA_ERR_SHAPE, "%s: embedding [n_vocab %u x n_embd %u]: n %u rows exceeds the limit %u", what,
                n_vocab, n_embd, n, kMaxRows);
  if (e_row_stride < n_embd || y_row_stride < n_embd)
    return fail(LORA_ERR_STRIDE, "%s: embedding [n_vocab %u x n_embd %u]: e_row_stride %u and y_row_stride %u "
                "must be >= n_embd %u", what, n_vocab, n_embd, e_row_stride, y_row_stride, n_embd);
  if (dtype == LORA_BF16 && (n_embd % 8 || e_row_stride % 8 || y_row_stride % 8))
    return fail(LORA_ERR_UNSUPPORTED, "%s: embedding [n_vocab %u x n_embd %u]: bf16 needs n_embd, e_row_stride %u "
                "and y_row_stride %u to be multiples of 8", what, n_vocab, n_embd, e_row_stride, y_row_stride);
  if (route) {
    if (int e = check_route(what, route, dtype, n_vocab, n_embd)) return e;
  }
  if (n == 0) return LORA_OK;
  if (!E || !token_ids || !y || (route && !seq_slot))
    return fail(LORA_ERR_NULL_PTR, "%s: embedding [n_vocab %u x n_embd %u]: E, token_ids, y%s must be non-NULL",
                what, n_vocab, n_embd, route ? ", seq_slot" : "");
  if (dtype == LORA_BF16 && (!aligned16(E) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned E %p and y %p", what, E, y);
  if (int e = check_device(what)) return e;
  EmbedArgs a{};
  a.E = E;
  a.e_row_stride = (int)e_row_stride;
  a.n_vocab = (int)n_vocab;
  a.n_embd = (int)n_embd;
  a.n = (int)n;
  a.rd = route_dev(route);
  a.has_lora = route != nullptr;
  a.token_ids = token_ids;
  a.seq_slot = seq_slot;
  a.y = y;
  a.y_row_stride = (int)y_row_stride;
  hipStream_t st = (hipStream_t)stream;
  prof_record(0, st);
  prof_record(1, st);
  const int e = launch_status(launch_embed_rows(a, dtype, st), what);
  prof_record(2, st);
  prof_record(3, st);
  return e;
}

int lora_apply_stack(int32_t dtype, uint32_t n_out, uint32_t k_in, const void *W, uint32_t w_row_stride,
                     const lora_route *routes, const int32_t *const *seq_slots, uint32_t n_levels,
                     const void *x, uint32_t x_row_stride, uint32_t n, void *y, uint32_t y_row_stride,
                     void *workspace, size_t workspace_bytes, void *stream) {
  clear_err();
  const char *what = "lora_apply_stack";
  if (int e = check_proj(what, dtype, n_out, k_in, n, x_row_stride, y_row_stride, w_row_stride)) return e;
  if (n_levels > (uint32_t)kMaxStackLevels)
    return fail(LORA_ERR_SHAPE, "%s: [n_out %u x k_in %u]: %u levels exceed the limit %d", what, n_out, k_in,
                n_levels, kMaxStackLevels);
  if (n_levels && (!routes || !seq_slots))
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: routes %p and seq_slots %p must be non-NULL for %u levels",
                what, n_out, k_in, (const void *)routes, (const void *)seq_slots, n_levels);
  int r_max = 0;
  for (uint32_t l = 0; l < n_levels; ++l) {
    if (int e = check_route(what, &routes[l], dtype, n_out, k_in)) return e;
    r_max = std::max(r_max, (int)routes[l].max_rank);
  }
  if (n == 0) return LORA_OK;
  if (!W || !x || !y)
    return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: W %p, x %p, y %p must be non-NULL", what, n_out, k_in,
                W, x, y);
  for (uint32_t l = 0; l < n_levels; ++l)
    if (!seq_slots[l])
      return fail(LORA_ERR_NULL_PTR, "%s: [n_out %u x k_in %u]: seq_slots[%u] is NULL", what, n_out, k_in, l);
  if (dtype == LORA_BF16 && (!aligned16(W) || !aligned16(x) || !aligned16(y)))
    return fail(LORA_ERR_UNSUPPORTED, "%s: bf16 needs 16-byte aligned W %p, x %p, y %p", what, W, x, y);
  // layout: the first level's fused-apply workspace, then t [n][R_l] of every further level
  const size_t apply_bytes = stack_apply_bytes(dtype, (int)n, (int)n_out, (int)k_in, r_max);
  size_t need = apply_bytes;
  for (uint32_t l = 1; l < n_levels; ++l)
    need += stack_level_layout(dtype, (int)n, (int)routes[l].max_rank, (int)k_in).total;
  if ((need && !workspace) || workspace_bytes < need)
    return fail(LORA_ERR_WORKSPACE, "%s: [n_out %u x k_in %u] with %u levels up to max_rank %d, n %u: workspace %p of %zu bytes, %zu needed",
                what, n_out, k_in, n_levels, r_max, n, workspace, workspace_bytes, need);
  if (workspace && !aligned16(workspace))
    return fail(LORA_ERR_UNSUPPORTED, "%s: workspace %p is not 16-byte aligned", what, workspace);
  if (int e = check_device(what)) return e;
  hipStream_t st = (hipStream_t)stream;
  const lora_route *r0 = n_levels ? &routes[0] : nullptr;
  const RouteDev rd0 = route_dev(r0);
  const Routing rt0 = routing_decode(r0 ? seq_slots[0] : nullptr);
  int e = LORA_OK;
  // every further level's shrink into its own t first (the bf16 shrinks of
  // all levels in one launch); then the first level's apply, whose decode
  // epilogue folds the further levels in the same rounding, or else one
  // fold of all of them after it
  StackFold f{};
  f.n_levels = n_levels > 1 ? (int)n_levels - 1 : 0;
  ShrinkLevels sl{};
  // decode-sized bf16 stacks: the further levels' shrinks by pool slot, each
  // level's t written whole (no k-split partials); larger batches take the
  // k-split shrink units
  const bool by_slot = dtype == LORA_BF16 && n <= (uint32_t)kBgmvMaxRows;
  BgmvLevels bl{};
  bl.n_levels = by_slot ? f.n_levels : 0;
  sl.n_levels = dtype == LORA_BF16 && !by_slot ? f.n_levels : 0;
  char *tp = (char *)workspace + apply_bytes;
  for (uint32_t l = 1; l < n_levels; ++l) {
    const RouteDev rd = route_dev(&routes[l]);
    const Routing rt = routing_decode(seq_slots[l]);
    const StackLevelLayout lay = stack_level_layout(dtype, (int)n, (int)routes[l].max_rank, (int)k_in);
    float *t = (float *)(tp + lay.t);
    if (dtype == LORA_F32) {
      e = launch_status(launch_shrink_f32(rd, rt, (const float *)x, (int)x_row_stride, (int)k_in, (int)n, t, st),
                        what);
      if (e) return e;
    } else if (by_slot) {
      bl.rd[l - 1] = rd;
      bl.seq_slot[l - 1] = seq_slots[l];
      bl.t[l - 1] = t;
      bl.blocks_per_level = std::max(bl.blocks_per_level, rd.max_loras * rd.R);
    } else {
      PrepArgs &pa = sl.lv[l - 1];
      pa.rd = rd;
      pa.rt = rt;
      pa.has_lora = true;
      pa.x = (const u16 *)x;
      pa.x_stride = (int)x_row_stride;
      pa.k_in = (int)k_in;
      pa.n = (int)n;
      pa.k_splits = stack_shrink_splits((int)n, (int)k_in);
      pa.t = pa.k_splits > 1 ? (float *)(tp + lay.partials) : t;
      pa.t_final = t;
      pa.counters = (unsigned *)(tp + lay.counters);
      pa.n_pairs = (int)routes[l].max_loras;
      pa.do_plan = 0;
      pa.n_units = (int)((n + kShrinkRows - 1) / kShrinkRows) + (int)std::min<uint32_t>(n, routes[l].max_loras);
      sl.blocks_per_level = std::max(sl.blocks_per_level, pa.n_units * pa.k_splits);
    }
    tp += lay.total;
    f.lv[l - 1] = StackLevel{rd.a_table, rd.b_table, rd.scale_table, seq_slots[l], t, rd.max_loras, rd.R};
  }
  if (sl.n_levels) {
    e = launch_status(launch_shrink_levels(sl, st), what);
    if (e) return e;
  }
  if (bl.n_levels) {
    e = launch_status(launch_bgmv_shrink_levels(bl, (const u16 *)x, (int)x_row_stride, (int)k_in, (int)n, st), what);
    if (e) return e;
  }
  bool folded = false;
  if (dtype == LORA_F32)
    e = run_f32_timed(what, [&] { return launch_apply_f32(rd0, rt0, r0 != nullptr, (const float *)W, 0,
                                                          (int)w_row_stride, (const float *)x, (int)x_row_stride,
                                                          (int)k_in, (int)n_out, (int)n, (float *)y,
                                                          (int)y_row_stride, st); }, st);
  else
    e = run_fused(what, LORA_OP_APPLY, rt0, rd0, r0 != nullptr, n_out, k_in, W, 0, w_row_stride, x, x_row_stride,
                  n, y, y_row_stride, workspace, apply_bytes, 1, st, &f, &folded);
  if (e || f.n_levels == 0 || folded) return e;
  e = launch_status(launch_expand_fold_stack(f, dtype, y, (int)y_row_stride, (int)n_out, (int)n, st), what);
  prof_record(3, st);
  return e;
}

}  // extern "C"
