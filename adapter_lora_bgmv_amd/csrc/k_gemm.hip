// k_gemm.hip -- the fused apply: y = W x + s B (A x), bf16 MFMA, f32 accumulate.
//
// A workgroup owns an output tile of BO output features x BR rows (rows in
// the plan's grouped order, gathered from x and scattered to y).  The
// contraction over k_in runs on v_mfma_f32_16x16x32_bf16 with W as the A
// operand and the gathered x rows as the B operand.
//
// Staging: both operands go to LDS by LDS-DMA (global_load_lds_dwordx4),
// which takes in as much per CU as loads into registers do and holds no
// registers while in flight.  A stage is 64 k columns of every row of the
// tile (W rows, then the gathered x rows), row-major at 128 bytes a row,
// each row's eight 16-byte chunks stored XOR-swizzled by row; one DMA
// instruction moves eight whole 128-byte row segments (full cache lines),
// and the MFMA fragments are read from the swizzled slots with ds_read_b128
// on distinct banks.  NS stages form a ring with NS-1 stages in flight.  The
// waits are explicit (s_waitcnt vmcnt + s_barrier): a stage is consumed only
// after every wave's DMA for it has landed.
//
// Ragged tiles: rows past the tile's end (x) or past n_out (W) load a valid
// row instead; they only feed output rows and columns that are never stored.
// A k tail that does not fill a stage is zeroed in LDS once it has landed.
//
// The low-rank term rides the same accumulators as a k-extension that runs
// after the base contraction (ferrox lora.rs "expand + fold"; atlas
// lora_delta.rs dense_gemm_tc_scaled_acc folds the scaled expand into the
// output the same way):
//     acc[o, i] += sum_kappa B_q[o, kappa] * T[i, kappa]
// where T holds s_q * t_i split into a bf16 high and low part (so the f32
// intermediate t is carried at ~16 significant bits; the shrink writes it),
// and rows of another pair, or skipped rows, contribute exact zeros.  A
// base-only accumulator that starts at +0 is never -0 afterwards, so adding
// those zeros leaves a skipped row bit-identical to the base-only launch.
//
// Split-K: the `splits` workgroups of a tile each take one of the same k
// ranges, whatever the tile (the range bounds are a function of k_in and
// the split count, which the host picks from the batch size and k_in
// alone); the last to arrive (a device-scope counter) sums the partial tiles
// in k order and writes y, so results do not depend on arrival order.  A
// row's LoRA term goes into the partial of contributor q mod splits (q its
// pair), whichever tile holds the row.  So an output element's sum is the
// same whatever tile its row lands in, whatever the other rows' routing, and
// whatever the output count: a skipped row equals the base-only call's, and
// a projection cut into blocks of output features equals the whole one.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lora {

// MODE: kOneTile (a workgroup per tile), kSplitK (the tile's k ranges on
// `splits` workgroups).
enum { kOneTile = 0, kSplitK = 1 };

template <int BO, int BR, int WGO, int WGR, int NS, int MODE>
__global__ __launch_bounds__(WGO *WGR * 64) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NW = WGO * WGR;
  constexpr int WO = BO / WGO, WR = BR / WGR;  // wave tile
  constexpr int NBO = WO / 16, NBR = WR / 16;  // fragment blocks per wave
  constexpr int RS = BO + BR;                  // rows of a stage: W rows, then x rows
  constexpr int SI = RS / 8;                   // DMA instructions per stage (8 rows x 128 B each)
  constexpr int LPW = SI / NW;                 // DMA instructions per wave per stage
  static_assert(SI % NW == 0, "stage rows must split evenly over the waves");
  static_assert(NS >= 2 && (NS - 2) * LPW < 64, "ring depth / vmcnt range");
  // A stage is 64 k columns of every row of the tile, row-major, 128 B per
  // row, its eight 16-byte chunks stored XOR-swizzled by row (chunk c of row
  // r at slot c ^ ((r >> 1) & 7)) so that the MFMA fragment reads below hit
  // distinct banks.
  __shared__ __attribute__((aligned(16))) uint4 ring[NS][RS * 8];
  __shared__ int s_row[BR], s_pair[BR];
  __shared__ const u16 *s_bq[BR];  // the row's B_pair, or null
  __shared__ int s_last;
  __shared__ int s_run[BR], s_rend[BR], s_nrun;  // runs of equal pairs: [start, end)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave % WGO, wr = wave / WGO;
  // Work partition: workgroup w takes tile w / splits, k range w mod splits.
  const int mtiles = *p.plan.n_tiles;
  const int G = mtiles * p.n_ntiles * p.splits;
  const int nst = (p.k_in + 63) / 64;
  const int b = blockIdx.x;
  if (b >= G) return;
  // The chip hands workgroups to its 8 XCDs in turn, each XCD with its own
  // L2: the workgroups of one XCD get a contiguous range of w, so they work
  // on neighbouring tiles, which its L2 then serves.
  const int xq = G / 8, xr = G % 8, xcd = b % 8;
  const int w = xcd * xq + min(xcd, xr) + b / 8;

  // Tile t, its stages [sb, se); wf..wl are the tile's contributors.
  auto segment = [&](int t, int sb, int se, int wf, int wl) {
  // Tile order: groups of up to 8 row tiles, rows fastest, so consecutive
  // tiles share W tiles and x tiles.
  const int gm0 = t / (8 * p.n_ntiles) * 8;  // first row tile of the group
  const int gsz = min(8, mtiles - gm0);
  const int tg = t - gm0 * p.n_ntiles;  // place within the group
  const int mt = gm0 + tg % gsz;
  const int nt = tg / gsz;
  const int4 tile = p.plan.tiles[mt];
  const int o0 = nt * BO;
  for (int i = tid; i < BR; i += NW * 64) {
    const bool in = i < tile.z;
    const int q = in ? p.plan.pos_pair[tile.y + i] : kSkip;
    s_row[i] = in ? p.plan.pos_row[tile.y + i] : -1;
    s_pair[i] = q;
    s_bq[i] = (p.has_lora && q >= 0) ? (const u16 *)p.b_table[q] : nullptr;
  }
  __syncthreads();

  f32x4 acc[NBO][NBR];
#pragma unroll
  for (int a = 0; a < NBO; ++a)
#pragma unroll
    for (int b = 0; b < NBR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------- base contraction
  const int kb = sb * 64;
  const int ke = min(se * 64, p.k_in);
  const int nstage = se - sb;
  const u16 *Wg = p.W + (size_t)tile.x * (size_t)p.w_group_stride;
  // Each DMA instruction moves 8 whole 128-byte row segments (full cache
  // lines): lane l takes row 8i + l/8 of the stage and the chunk that belongs
  // at slot l%8 of that row.  This lane's rows are the same in every stage:
  // instructions j < JW carry W rows, the rest x rows.  The slot of a chunk
  // depends on (row >> 1) & 7, which is the same for every j (the rows of
  // instruction j are NW * 8 j apart, a multiple of 16).
  constexpr int JW = BO / (8 * NW);
  static_assert(JW * 8 * NW == BO, "a DMA instruction carries W rows or x rows, not both");
  int rowid[LPW];  // the W row (output feature) or the x row of each instruction
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rr = (wave + NW * j) * 8 + (lane >> 3);  // row of the stage
    if (j < JW) {
      rowid[j] = min(o0 + rr, p.n_out - 1);
    } else {
      int r = s_row[rr - BO];
      if (r < 0) r = s_row[0];
      rowid[j] = r;
    }
  }
  const int sch = ((lane & 7) ^ (((wave * 8 + (lane >> 3)) >> 1) & 7)) * 8;  // this lane's chunk
  // Every wave issues exactly LPW DMA instructions per stage, so the vmcnt
  // waits count stages exactly.  Lanes whose chunk lies past the k range read
  // column 0 of their row instead and zero their landed chunk afterwards.
  auto issue = [&](int st) {
    const int k0 = kb + st * 64;
    const int kk = k0 + sch < ke ? k0 + sch : 0;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const u16 *g = j < JW ? Wg + (size_t)rowid[j] * p.w_row_stride + kk
                            : p.x + (size_t)rowid[j] * p.x_row_stride + kk;
      dma16(g, lds_addr(&ring[st % NS][(wave + NW * j) * 64]));
    }
  };
  for (int st = 0; st < NS - 1 && st < nstage; ++st) issue(st);

  // Stage st is in LDS for every wave: wait for this wave's DMAs (at most
  // `younger` stages issued after it may stay in flight), zero the chunks
  // this wave fetched past the k range, then the barrier.
  auto landed = [&](int st, int younger) {
    wait_stages<LPW, (NS > 2 ? NS - 2 : 0)>(younger);
    const int k0 = kb + st * 64;
    if (k0 + 64 > ke) {
#pragma unroll
      for (int j = 0; j < LPW; ++j)
        if (k0 + sch >= ke) ring[st % NS][(wave + NW * j) * 64 + lane] = z4();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
    block_barrier();
  };
  // MFMA fragments of one 32-wide half h of a stage: lane l reads row l%16
  // of the block, chunk 4h + l/16, at its swizzled slot.
  uint4 af[2][NBO], bf[2][NBR];
  auto fetch = [&](int st, auto hc) {
    constexpr int h = decltype(hc)::value;
    const uint4 *sl = ring[st % NS];
    const int c = 4 * h + (lane >> 4);
#pragma unroll
    for (int bo = 0; bo < NBO; ++bo) {
      const int r = (wo * NBO + bo) * 16 + (lane & 15);
      af[h][bo] = sl[r * 8 + (c ^ ((r >> 1) & 7))];
    }
#pragma unroll
    for (int b = 0; b < NBR; ++b) {
      const int r = BO + (wr * NBR + b) * 16 + (lane & 15);
      bf[h][b] = sl[r * 8 + (c ^ ((r >> 1) & 7))];
    }
  };
  auto mma = [&](auto hc) {
    constexpr int h = decltype(hc)::value;
#pragma unroll
    for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
      for (int b = 0; b < NBR; ++b) acc[bo][b] = mfma16(af[h][bo], bf[h][b], acc[bo][b]);
  };
  for (int st = 0; st < nstage; ++st) {
    landed(st, min(NS - 2, nstage - 1 - st));
    // every wave is done with stage st - 1: its ring slot takes stage st + NS - 1
    if (st + NS - 1 < nstage) issue(st + NS - 1);
    fetch(st, std::integral_constant<int, 0>{});
    fetch(st, std::integral_constant<int, 1>{});  // read while the first half's MFMAs run
    mma(std::integral_constant<int, 0>{});
    mma(std::integral_constant<int, 1>{});
  }

  // ---------------------------------------------------------- LoRA term
  // acc[o, i] += sum_kappa B_q[o, kappa mod R] T[i, kappa] over kappa < 2R,
  // where row i of T holds s_q t_i as bf16 high parts (kappa < R) and the
  // bf16 roundings of what they leave over (kappa >= R), and rows of another
  // pair, or skipped rows, contribute exact zeros.  It runs after the base
  // contraction: an accumulator that started at +0 is never -0 there, so the
  // zeros leave a skipped row bit-identical to the base-only launch.
  //
  // The tile's rows are sorted by pair, so a pair is one run of rows.  With
  // R dividing 64, T's rows go to LDS once (one or two 64-column chunks) and
  // each run's B slice (BO rows x R, repeated to 64 columns) streams through
  // an LDS-DMA ring, so every byte is fetched once per workgroup; only the
  // waves whose rows meet the run do its MFMAs.  The tile's C contributors
  // share the runs out by pair: contributor j takes the pairs q with
  // q mod C = j.
  if (p.has_lora && p.R <= 64 && 64 % p.R == 0) {
    constexpr int LPB = BO / 8 / NW;  // DMA instructions per wave per B stage
    constexpr int LPT = BR / 8 / NW;  // per 64-column chunk of T
    constexpr int kRing = NS * RS * 128, kT = 2 * BR * 128;
    constexpr int EB = (kRing - kT) / (BO * 128) > 4 ? 4 : (kRing - kT) / (BO * 128);
    static_assert(LPB * NW * 8 == BO && LPT * NW * 8 == BR, "rows must split evenly over the waves");
    static_assert(EB >= 2, "the ring must hold T and two B stages");
    const int R = p.R, nck = (2 * R + 63) / 64;
    uint4 *const tlds = &ring[0][0];
    uint4 *const blds = tlds + 2 * BR * 8;
    const int C = wl - wf + 1, jc = w - wf;
    block_barrier();  // every wave is done with the ring
    if (wave == 0) {
      const uint64_t below = (1ull << lane) - 1ull;
      int ns = 0, ne = 0;
      for (int i = lane; i < BR; i += 64) {
        const int q = s_pair[i];
        const bool mine = q >= 0 && q % C == jc;
        const bool st = mine && (i == 0 || s_pair[i - 1] != q);
        const bool en = mine && (i + 1 == BR || s_pair[i + 1] != q);
        const uint64_t ms = __ballot(st), me = __ballot(en);
        if (st) s_run[ns + (int)__popcll(ms & below)] = i;
        if (en) s_rend[ne + (int)__popcll(me & below)] = i + 1;
        ns += (int)__popcll(ms);
        ne += (int)__popcll(me);
      }
      if (lane == 0) s_nrun = ns;
    }
    block_barrier();
    const int nmine = s_nrun;
    if (nmine > 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c >= nck) break;
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int rr = (wave + NW * j) * 8 + (lane >> 3);
          int r = s_row[rr];
          if (r < 0) r = s_row[0];
          const int kap = 64 * c + ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
          dma16(p.tt + (size_t)r * 2 * R + (kap < 2 * R ? kap : 0),
                lds_addr(tlds + c * BR * 8 + (wave + NW * j) * 64));
        }
      }
      auto issue_b = [&](int s) {
        const u16 *Bq = s_bq[s_run[s]];
#pragma unroll
        for (int j = 0; j < LPB; ++j) {
          const int rr = (wave + NW * j) * 8 + (lane >> 3);
          const int o = min(o0 + rr, p.n_out - 1);
          const int col = (((lane & 7) ^ ((rr >> 1) & 7)) * 8) & (R - 1);
          dma16(Bq + (size_t)o * R + col, lds_addr(blds + (s % EB) * BO * 8 + (wave + NW * j) * 64));
        }
      };
      for (int s = 0; s < EB - 1 && s < nmine; ++s) issue_b(s);
      for (int s = 0; s < nmine; ++s) {
        wait_stages<LPB, EB - 2>(min(EB - 2, nmine - 1 - s));  // T went out first
        if (s == 0 && 2 * R < 64) {  // zero the columns past 2R
#pragma unroll
          for (int j = 0; j < LPT; ++j) {
            const int rr = (wave + NW * j) * 8 + (lane >> 3);
            if (((lane & 7) ^ ((rr >> 1) & 7)) * 8 >= 2 * R) tlds[(wave + NW * j) * 64 + lane] = z4();
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        }
        block_barrier();
        if (s + EB - 1 < nmine) issue_b(s + EB - 1);
        const int i0 = s_run[s], i1 = s_rend[s];
        if (i0 >= (wr + 1) * WR || i1 <= wr * WR) continue;  // none of this wave's rows
        const uint4 *bs = blds + (s % EB) * BO * 8;
        // one 32-column half of the B slice, and at most four of its output
        // blocks, at a time (few registers beside the accumulators): its
        // fragments serve every row block and T chunk
        constexpr int OB = NBO < 4 ? NBO : 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c8 = 4 * h + (lane >> 4);
#pragma unroll
          for (int ob = 0; ob < NBO; ob += OB) {
#pragma unroll
            for (int bo = 0; bo < OB; ++bo) {
              const int r = (wo * NBO + ob + bo) * 16 + (lane & 15);
              af[0][bo] = bs[r * 8 + (c8 ^ ((r >> 1) & 7))];
            }
#pragma unroll
            for (int b = 0; b < NBR; ++b) {
              const int rb0 = wr * WR + b * 16;
              if (i0 >= rb0 + 16 || i1 <= rb0) continue;
              const int r = rb0 + (lane & 15);
              const bool in = r >= i0 && r < i1;
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                if (c >= nck) break;
                const uint4 tv = tlds[c * BR * 8 + r * 8 + (c8 ^ ((r >> 1) & 7))];
                const uint4 tf = in ? tv : z4();
#pragma unroll
                for (int bo = 0; bo < OB; ++bo) acc[ob + bo][b] = mfma16(af[0][bo], tf, acc[ob + bo][b]);
              }
            }
          }
        }
      }
    }
  } else if constexpr (BO * BR < 256 * 256) {  // (256 x 256 launches take R dividing 64 only)
  if (p.has_lora && w == wl) {
  // Other ranks: the tile's last contributor loads the operands into
  // registers.  Items are (run of equal pairs within a 16-row block, 32-wide
  // kappa step); the loads of up to G items are issued together before their
  // MFMAs.  When every row of the wave's range that has a pair has the same
  // one, the B fragments of a kappa step serve all NBR row blocks.
  int upair = kSkip;
  bool uniform = true;
  if (uniform) {
    for (int i = 0; i < WR; ++i) {  // LDS broadcast reads, the same for every lane
      const int q = s_pair[wr * WR + i];
      if (q < 0) continue;
      if (upair < 0) upair = q;
      else if (q != upair) { uniform = false; break; }
    }
    uniform = uniform && upair >= 0;
  }
  if (uniform) {
    const int R = p.R, nks = 2 * R / 32;
    const int l0 = wr * WR;
    const u16 *Bq = nullptr;
    for (int i = 0; i < WR; ++i)
      if (s_pair[l0 + i] == upair) { Bq = s_bq[l0 + i]; break; }
    const u16 *trow[NBR];  // the row's s * t (high parts, then remainders), or null
#pragma unroll
    for (int b = 0; b < NBR; ++b) {
      const int li = l0 + b * 16 + (lane & 15);
      trow[b] = s_pair[li] == upair ? p.tt + (size_t)s_row[li] * 2 * R : nullptr;
    }
    // kappa steps per round: two, or one where the accumulators leave no room
    constexpr int ES = NBO >= 8 ? 1 : 2;
    for (int ks0 = 0; ks0 < nks; ks0 += ES) {
      uint4 bv[ES][NBO], tv[ES][NBR];
#pragma unroll
      for (int s = 0; s < ES; ++s) {
        const int kap = (ks0 + s) * 32 + (lane >> 4) * 8;
        const int r0 = kap >= R ? kap - R : kap;
        const bool in = ks0 + s < nks;
#pragma unroll
        for (int bo = 0; bo < NBO; ++bo) {
          const int o = min(o0 + wo * WO + bo * 16 + (lane & 15), p.n_out - 1);
          bv[s][bo] = in ? ldg16(Bq + (size_t)o * R + r0) : z4();
        }
#pragma unroll
        for (int b = 0; b < NBR; ++b) tv[s][b] = in && trow[b] ? ldg16(trow[b] + kap) : z4();
      }
#pragma unroll
      for (int s = 0; s < ES; ++s) {
        if (ks0 + s >= nks) break;
#pragma unroll
        for (int b = 0; b < NBR; ++b)
#pragma unroll
          for (int bo = 0; bo < NBO; ++bo) acc[bo][b] = mfma16(bv[s][bo], tv[s][b], acc[bo][b]);
      }
    }
  } else {
    const int R = p.R, nks = 2 * R / 32;
    constexpr int G = NBO <= 2 ? 8 : (NBO <= 4 ? 4 : 1);
    const int myr = lane & 15;
    int br = 0, i = 0, ks = 0;  // iterator: next item to load
    auto run_end = [&](int b, int i0) {
      const int l0 = wr * WR + b * 16, q = s_pair[l0 + i0];
      int j = i0 + 1;
      while (j < 16 && s_pair[l0 + j] == q) ++j;
      return j;
    };
    // skip to the first run that has a pair
    auto settle = [&]() {
      while (br < NBR) {
        if (i >= 16) { ++br; i = 0; continue; }
        if (s_pair[wr * WR + br * 16 + i] >= 0) return;
        i = run_end(br, i);
      }
    };
    settle();
    while (br < NBR) {
      uint4 bv[G][NBO], tv[G];
      int ibr[G], ns = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ibr[g] = -1;
        if (br >= NBR) continue;
        const int l0 = wr * WR + br * 16;
        const int j = run_end(br, i);
        const u16 *Bq = s_bq[l0 + i];
        const int kap = ks * 32 + (lane >> 4) * 8;
        const int r0 = kap >= R ? kap - R : kap;
#pragma unroll
        for (int bo = 0; bo < NBO; ++bo) {
          const int o = min(o0 + wo * WO + bo * 16 + (lane & 15), p.n_out - 1);
          bv[g][bo] = ldg16(Bq + (size_t)o * R + r0);
        }
        const int grow = s_row[l0 + myr];
        tv[g] = myr >= i && myr < j && grow >= 0 ? ldg16(p.tt + (size_t)grow * 2 * R + kap) : z4();
        ibr[g] = br;
        ++ns;
        if (++ks == nks) {  // next run
          ks = 0;
          i = j;
          settle();
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= ns) break;
#pragma unroll
        for (int b = 0; b < NBR; ++b)
          if (ibr[g] == b)
#pragma unroll
            for (int bo = 0; bo < NBO; ++bo) acc[bo][b] = mfma16(bv[g][bo], tv[g], acc[bo][b]);
      }
    }
  }

  }
  }

  // ---------------------------------------------------------- split-K fixup
  if (MODE != kOneTile && wf != wl) {
    // Every contributor stores its partial tile, then moves the tile's
    // arrival counter; the last to arrive sums the partials in k order (so
    // the result does not depend on arrival order) and writes y.  A
    // contributor's partial of its first tile sits in slot w, of its last
    // tile in slot G + w.
    constexpr int TT = BO * BR;
    // fragment (bo, br) of wave v sits at byte ((v NBO + bo) NBR + br) KB, lane l at +16 l
    const int wbase = __builtin_amdgcn_readfirstlane(wave) * NBO * NBR * 1024;
    const auto slot_rsrc = [&](int cw) {
      // the same for every lane: keeps the resource in scalar registers
      const int slot = __builtin_amdgcn_readfirstlane(cw);
      return coherent_rsrc(p.partials + (size_t)slot * TT, TT * 4);
    };
    {
      const auto rs = slot_rsrc(w);
#pragma unroll
      for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
        for (int br = 0; br < NBR; ++br)
          st16_coherent(rs, lane * 16, wbase + (bo * NBR + br) * 1024, acc[bo][br]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&p.counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (unsigned)(wl - wf);
    __syncthreads();
    if (!s_last) return;
    // FB output blocks at a time: their loads for one contributor are in
    // flight together, few enough to leave the accumulators in registers
    constexpr int FB = NBO >= 4 ? 4 : NBO;
#pragma unroll
    for (int b0 = 0; b0 < NBO; b0 += FB)
      for (int cw = wf; cw <= wl; ++cw) {
        const auto rs = slot_rsrc(cw);
#pragma unroll
        for (int bo = b0; bo < b0 + FB; ++bo)
#pragma unroll
          for (int br = 0; br < NBR; ++br) {
            const f32x4 v = ld16_coherent(rs, lane * 16, wbase + (bo * NBR + br) * 1024);
            acc[bo][br] = cw == wf ? v : acc[bo][br] + v;
          }
      }
    if (tid == 0) __hip_atomic_store(&p.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---------------------------------------------------------- epilogue
  // The tile goes through LDS as bf16 (16-byte chunk c of tile row r at slot
  // c ^ (r % CPR), or within its group of 8 chunks c ^ (r % 8) when CPR is
  // not a power of two, so the fragment-ordered writes spread over the
  // banks) and leaves in whole 16-byte pieces, each tile row's by
  // consecutive lanes.
  constexpr int CPR = BO / 8;  // 16-byte chunks per tile row
  static_assert(BR * CPR <= NS * RS * 8, "the bf16 tile fits the ring");
  static_assert((CPR & (CPR - 1)) == 0 || CPR % 8 == 0, "chunk swizzle");
  auto yslot = [](int r, int c) {
    if constexpr ((CPR & (CPR - 1)) == 0) return r * CPR + (c ^ (r & (CPR - 1)));
    else return r * CPR + ((c & ~7) | ((c ^ r) & 7));
  };
  uint4 *const ylds = &ring[0][0];
  __syncthreads();  // every wave is done with the ring
#pragma unroll
  for (int bo = 0; bo < NBO; ++bo) {
    const int oc = wo * WO + bo * 16 + (lane >> 4) * 4;  // four outputs of the tile
#pragma unroll
    for (int br = 0; br < NBR; ++br) {
      const int lr = wr * WR + br * 16 + (lane & 15);  // tile row
      const f32x4 v = acc[bo][br];
      const uint2 pk = make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
      uint2 *dst = (uint2 *)&ylds[yslot(lr, oc >> 3)];
      dst[(oc >> 2) & 1] = pk;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < BR * CPR; idx += NW * 64) {
    const int r = idx / CPR, c = idx % CPR;
    const int grow = s_row[r], o = o0 + c * 8;
    if (grow >= 0 && o < p.n_out)
      *(uint4 *)(p.y + (size_t)grow * p.y_row_stride + o) = ylds[yslot(r, c)];
  }
  };  // segment

  const int t = w / p.splits;
  const int j = w - t * p.splits;
  segment(t, j * nst / p.splits, (j + 1) * nst / p.splits, t * p.splits, t * p.splits + p.splits - 1);
}

hipError_t launch_gemm(const GemmArgs &a, int to, int tr, hipStream_t st) {
  const int grid = a.max_mtiles * a.n_ntiles * a.splits;
  if (grid == 0) return hipSuccess;
  // ring depth: as many 64-column stages as fit in about 128 KB of LDS
#define LORA_GEMM(BO, BR, WGO, WGR, NS, MODE) \
  hipLaunchKernelGGL((gemm_bf16_kernel<BO, BR, WGO, WGR, NS, MODE>), dim3(grid), dim3(WGO * WGR * 64), 0, st, a)
  const int mode = a.splits > 1 ? kSplitK : kOneTile;
  // the 256 x 256 tiles stage the LoRA term through LDS only
  if (to == 256 && tr == 256 && a.has_lora && (a.R > 64 || 64 % a.R != 0)) return hipErrorInvalidValue;
  if (to == 64 && tr == 64 && mode == kOneTile) LORA_GEMM(64, 64, 2, 2, 8, kOneTile);
  else if (to == 64 && tr == 64 && mode == kSplitK) LORA_GEMM(64, 64, 2, 2, 8, kSplitK);
  else if (to == 128 && tr == 128 && mode == kOneTile) LORA_GEMM(128, 128, 2, 2, 4, kOneTile);
  else if (to == 128 && tr == 128 && mode == kSplitK) LORA_GEMM(128, 128, 2, 2, 4, kSplitK);
  else if (to == 256 && tr == 64 && mode == kOneTile) LORA_GEMM(256, 64, 4, 1, 3, kOneTile);
  else if (to == 512 && tr == 64 && mode == kOneTile) LORA_GEMM(512, 64, 8, 1, 2, kOneTile);
  else if (to == 256 && tr == 128 && mode == kOneTile) LORA_GEMM(256, 128, 4, 4, 3, kOneTile);  // 16 waves of 64 x 32
  else if (to == 192 && tr == 128 && mode == kOneTile) LORA_GEMM(192, 128, 4, 2, 3, kOneTile);
  else if (to == 256 && tr == 256 && mode == kOneTile) LORA_GEMM(256, 256, 4, 4, 2, kOneTile);  // 16 waves of 64 x 64
  else
    return hipErrorInvalidValue;
#undef LORA_GEMM
  return hipGetLastError();
}

}  // namespace lora
