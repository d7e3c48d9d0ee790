// Grouped GEMM with wide tiles: 384 rows x 256 B-columns per work group (bf16, gfx950).
//
// Same contract as the 128-row kernels in moe_gemm.hip (one launch over the block
// table [expert, m_start, valid_m] plus an optional dense segment; TileLang chapter
// "MoE, MLA and sparse-attention operators", section 2.4 (a); dropless notes sections
// 3, 5 and 7), for routing where experts own many 128-row blocks.
//
// Why wider tiles.  On gfx950 the global->LDS copies through each CU's vector-memory
// path, not the MFMAs, bound the 128 x 512 tile: per 32-deep K slice it moves 40 KB
// for 2 M multiply-adds.  A 384 x 256 tile moves the same 40 KB (24 KB of A, 16 KB of
// B) for 3 M multiply-adds, a third fewer bytes per FLOP; its 98,304 fp32
// accumulators fill three quarters of the CU's register file.
//
//   * A work item is (group, column tile).  A group is up to three consecutive table
//     blocks of one expert whose rows are contiguous (every block but the last full),
//     so all its rows read the same weight panel.  Each work group builds the group
//     list of the launch from the device-side table, in the LDS ring before its first
//     item: runs of such blocks, cut into threes from the start of each run.  The
//     dense segment's groups are 384-row spans of its rows.
//   * NW waves (4: one per SIMD, 384 accumulator registers each; 8: two per SIMD, 192
//     each).  Wave w owns column half w % 2 of 32-row subtiles interleaved across the
//     NW / 2 wave pairs: subtile i of pair p = w / 2 is tile rows (i NW/2 + p) 32 ..
//     +31.  So a group of b blocks (rows below 128 b) leaves every wave about b live
//     subtiles, and a wave multiplies only its live ones (the forward loop is
//     specialised on their number, decided once per item), which balances the SIMDs
//     on groups of one or two blocks.  GATEUP: 64 act columns, i.e. the matching 64
//     gate (W1) and 64 up (W3) columns, so SiLU*mul stays in registers; DOWN: 128
//     columns.
//   * Operands move HBM -> LDS with 16-byte global_load_lds copies into a 4-slot ring of
//     32-deep K slices (40 KB each, the whole LDS).  A is [384 rows][64 B] with the chunk swizzle
//     c ^ ((row >> 2) & 3); B keeps its [k][n] layout (GATEUP: W1 and W3 regions of
//     [32][128 columns]; DOWN: one [32][256 columns] region) with the swizzle
//     c ^ 4 * (k & 3), and is read with ds_read_b64_tr_b16.  Both swizzles were
//     measured conflict-free on gfx950.
//   * Every lane issues the same copies every slice (rows past the group's valid rows
//     copy row 0, columns past N copy column 0; those results are never stored), so
//     the vmcnt waits are constants.
#include <algorithm>
#include <cstdlib>

#include "moe_gemm_common.h"

namespace moe {

static constexpr int kWRows = 384;                    // rows per tile
static constexpr int kWideLagFrom = 4;                 // waves >= this run half a step late
static constexpr int kWBK = 32;                       // K per ring slot
static constexpr int kWABytes = kWRows * kWBK * 2;    // 24 KB
static constexpr int kWBBytes = kWBK * 256 * 2;       // 16 KB
static constexpr int kWStage = kWABytes + kWBBytes;   // 40 KB
static constexpr int kWStages = 4;
static constexpr int kWACopies = kWRows / 16;         // 1 KB copies per slice: A
static constexpr int kWBCopies = kWBBytes / 1024;     //                        B
static constexpr int kWMaxBlocks = 8192;              // block-table limit (see below)

// Block table limit of the wide kernel: the staged table (3 ints per block), the group
// list (one int per block at most) and its length must fit the ring while it is idle.
int wide_max_blocks() {
  static_assert(kWMaxBlocks * 16 + 16 <= kWStages * kWStage, "group list fits the ring");
  return kWMaxBlocks;
}

// Work order.  Items (row group g, column tile t) are numbered in supertiles of
// Gs x Ts = 32 items (Ts = min(n_tiles, 8) consecutive tiles of Gs consecutive groups,
// group-major inside), supertiles row by row; the slot j * grid + q of a persistent
// grid's iteration j goes to work group (q % (grid / 8)) * 8 + q / (grid / 8).  Work
// groups are dealt to the 8 XCDs in turn, so each XCD runs 32 consecutive items - one
// supertile: a few A panels and B panels shared through that XCD's L2, instead of up to
// 32 of each.
__device__ __forceinline__ void wide_item_st(int slot, int ngt, int n_tiles, int& g, int& t) {
  const int Ts = min(n_tiles, 8);
  const int Gs = 32 / Ts;
  const int row_items = Gs * n_tiles;
  const int sr = slot / row_items, rem = slot - sr * row_items;
  const int gr = min(Gs, ngt - sr * Gs);
  const int sc = rem / (gr * Ts), within = rem - sc * gr * Ts;
  const int tc = min(Ts, n_tiles - sc * Ts);
  g = sr * Gs + within / tc;
  t = sc * Ts + within % tc;
}
// The item order with a split last round: the first ngt - nsingle groups in supertiles,
// then the nsingle single-block groups split off the list's end, group by group (their
// items take the last round; consecutive items stay on one XCD, so a split group's three
// singles share its weight panel there).
__device__ __forceinline__ void wide_item(int slot, int ngt, int nsingle, int n_tiles, int& g,
                                          int& t) {
  const int main_items = (ngt - nsingle) * n_tiles;
  if (slot < main_items) {
    wide_item_st(slot, ngt - nsingle, n_tiles, g, t);
  } else {
    const int r = slot - main_items;
    g = ngt - nsingle + r / n_tiles;
    t = r - (r / n_tiles) * n_tiles;
  }
}

// f(std::integral_constant<int, clamp(n, 1, N)>): one instance per count, so that code
// specialised on the count runs without branches inside it.  The full count is the
// expected one and comes first (measured: without the hint the full-tile items of
// ep-share's gate/up ran 1 % slower; without the zero-count instance a wave with no live
// subtile multiplies one, whose rows are never stored).
template <int N, class F>
__device__ __forceinline__ void dispatch_live(int n, F&& f) {
  if constexpr (N == 1) {
    f(std::integral_constant<int, 1>{});
  } else {
    if (__builtin_expect(n >= N, 1)) f(std::integral_constant<int, N>{});
    else dispatch_live<N - 1>(n, f);
  }
}

template <int OP, int NW, bool FP8>
__global__ void __launch_bounds__(NW * 64, 1)
k_gg_wide(GGOperands routed, GGOperands dense, int K, int N,
          const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
          int max_blocks, int E, int64_t max_rows, int dense_rows, int n_tiles) {
  constexpr bool GU = OP == MOE_OP_GATEUP_SWIGLU || OP == kOpGateUpBwd;
  constexpr bool BWD = OP == kOpGateUpBwd;
  static_assert(!(FP8 && BWD), "fp8 weights: forward ops only");
  constexpr int NT = NW * 64;
  constexpr int WR = kWRows * 2 / NW;     // rows per wave
  constexpr int MI = WR / 32;             // 32-row subtiles per wave
  // fp8 weights: a slice's B is half the bytes (8 KB), so a slot is 32 KB and five fit
  constexpr int kBBytes = FP8 ? kWBBytes / 2 : kWBBytes;
  constexpr int kStage = kWABytes + kBBytes;
  constexpr int kStages = FP8 ? 5 : kWStages;
  constexpr int CPA = kWACopies / NW;     // copies per wave per slice
  constexpr int CPB = kBBytes / 1024 / NW;
  constexpr int CPW = CPA + CPB;
  constexpr int kOutCols = GU ? 128 : 256;
  // bytes per staged B row (per matrix region for gate/up)
  constexpr int kBPitch = (GU ? 128 : 256) * (FP8 ? 1 : 2);
  constexpr int kEB = FP8 ? 1 : 2;        // bytes per weight
  static_assert(kWACopies % NW == 0 && (kBBytes / 1024) % NW == 0 && WR % 32 == 0, "tile split");
  static_assert(kStages * kStage <= kWStages * kWStage, "ring fits the LDS array");

  __shared__ __align__(1024) unsigned char lds[kWStages * kWStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = max_blocks > 0 ? clamp_block_count(num_blocks_ptr, max_blocks) : 0;

  // ---- group list ----------------------------------------------------------------
  // Built in the ring while it is idle: the table is staged at s_meta, then wave 0 forms
  // the groups into s_groups (lane l walks blocks [l*per, (l+1)*per); the run start that
  // governs its first block and its first output slot come from two wave-wide scans)
  // and their number into s_ngroups[0] (s_ngroups[1]: how many single-block groups the
  // last-round split appended).  Every wave then keeps the entries of its next 64
  // work items in one register (lane j: item j), so the whole LDS holds the ring.
  const int ng_dense = (dense_rows + kWRows - 1) / kWRows;
  int32_t* s_meta = reinterpret_cast<int32_t*>(lds);
  int32_t* s_groups = s_meta + 3 * nb;
  int32_t* s_ngroups = s_groups + nb;
  auto build_groups = [&]() {
    for (int i = tid; i < 3 * nb; i += NT) s_meta[i] = meta[i];
    __syncthreads();
    if (wave == 0) {
      auto ok = [&](int b) {
        const int e = s_meta[3 * b], m = s_meta[3 * b + 1], v = s_meta[3 * b + 2];
        return e >= 0 && e < E && m >= 0 && v >= 1 && v <= 128 && (int64_t)m + v <= max_rows;
      };
      // block b (valid) continues the run of block b-1: same expert, and its rows start
      // where b-1's end (padded layout: b-1 is full; unpadded: b-1 may be the expert's
      // partial first entry)
      auto joins = [&](int b) {
        return b > 0 && ok(b - 1) && s_meta[3 * b] == s_meta[3 * b - 3] &&
               s_meta[3 * b + 1] == s_meta[3 * b - 2] + s_meta[3 * b - 1];
      };
      const int per = (nb + 63) / 64;
      const int lo = min(lane * per, nb), hi = min(lo + per, nb);
      int last_rs = -1;
      for (int b = lo; b < hi; ++b) {
        if (!ok(b)) MOE_DEBUG_REPORT(MOE_DBG_BLOCK_TABLE);
        if (ok(b) && !joins(b)) last_rs = b;
      }
      int incl = last_rs;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl = max(incl, o);
      }
      int in_rs = __shfl_up(incl, 1, 64);
      if (lane == 0) in_rs = -1;
      int cnt = 0, rs = in_rs;
      for (int b = lo; b < hi; ++b) {
        if (!ok(b)) continue;
        if (!joins(b)) rs = b;
        if ((b - rs) % 3 == 0) ++cnt;
      }
      int inc = cnt;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
      }
      int idx = inc - cnt;
      rs = in_rs;
      for (int b = lo; b < hi; ++b) {
        if (!ok(b)) continue;
        if (!joins(b)) rs = b;
        if ((b - rs) % 3 == 0) {
          int n = 1;
          while (n < 3 && b + n < nb && ok(b + n) && joins(b + n)) ++n;
          s_groups[idx++] = (b << 2) | n;
        }
      }
      if (lane == 63) {
        // The last round of the persistent grid.  Items (group, column tile) cost about
        // the same, so total items on G work groups take ceil(total / G) rounds and a
        // short last round leaves most work groups idle.  Trailing three-block groups
        // are split into single blocks (2 n_tiles more items each) when that adds no
        // round and the last round then holds only single-block items (wide_item numbers
        // the singles' items last), which multiply a third of the rows.  Each output
        // row's sum is unchanged.
        int ng = inc, nsingle = 0;
        const int G = (int)gridDim.x;
        const int total = (ng_dense + ng) * n_tiles;
        const int F = total / G;
        // (not in the SwiGLU-backward op: there the extra registers put a spill reload
        // and a full wait into each item's first half-slice)
        if (!BWD && total - F * G > 0) {
          const int smax = ((F + 1) * G - total) / (2 * n_tiles);
          int sp = 0;
          while (sp < smax && sp < ng && (s_groups[ng - 1 - sp] & 3) == 3) ++sp;
          if (sp > 0 && 3 * sp * n_tiles >= total + 2 * sp * n_tiles - F * G) {
            for (int i = sp - 1; i >= 0; --i) {   // backwards: no entry overwritten unread
              const int b = s_groups[ng - sp + i] >> 2;
              for (int j2 = 2; j2 >= 0; --j2) s_groups[ng - sp + 3 * i + j2] = ((b + j2) << 2) | 1;
            }
            ng += 2 * sp;
            nsingle = 3 * sp;
          }
        }
        s_ngroups[0] = ng;
        s_ngroups[1] = nsingle;
      }
    }
    __syncthreads();
  };
  build_groups();
  const int ngroups = __builtin_amdgcn_readfirstlane(s_ngroups[0]);
  const int nsingle = __builtin_amdgcn_readfirstlane(s_ngroups[1]);

  const int total = (ng_dense + ngroups) * n_tiles;
  const int nk = K / kWBK;

  // Fixed per-lane parts of the fragment addresses, so that inside the loop an address
  // is slot base + one of these + an immediate.
  //   A (ds_read_b128): row rsub(i) + (l & 31), logical chunk 2kk + (l >> 5); the
  //   swizzle c ^ ((row >> 2) & 3) sees the row only through (l >> 2) & 7, so subtile i
  //   is the immediate 2048 NP i and kk selects one of two lane offsets.
  //   B (ds_read_b64_tr_b16): 16-lane group g, row r = (l & 15) >> 2, column quad
  //   c4 = l & 3; slice row k = 16kk + 8(g >> 1) + 4hh + r and column
  //   n = 32j' + 16(g & 1) + 4c4 of the wave's columns, at chunk (n >> 3) ^ 4r (k & 3 is r).
  //   Subtile j's first chunk cj is a multiple of 4, so its swizzled chunk is
  //   (cj ^ 4r) | (2(g & 1) + (c4 >> 1)): kk and hh are immediates (16 and 4 rows); the
  //   lane offset depends on j (GATEUP: on j & 1, the W1/W3 region being an immediate).
  const int g = lane >> 4, tr_r = (lane & 15) >> 2, tr_c4 = lane & 3;
  const int ch = wave & 1;                 // column half
  constexpr int NP = NW / 2;               // wave pairs
  const int rpair = wave >> 1;
  // first tile row of the wave's subtile i
  auto rsub = [&](int i) { return (i * NP + rpair) * 32; };
  constexpr int NBL = GU ? 2 : 4;          // distinct B lane offsets
  uint32_t a_lane[2], b_lane[NBL];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int row = rpair * 32 + (lane & 31);
    a_lane[kk] = (uint32_t)(row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16);
  }
#pragma unroll
  for (int jb = 0; jb < NBL; ++jb) {
    if constexpr (FP8) {
      // ds_read_b64_tr_b8: in 16-lane group g, lane gi points at row gi / 2 of an 8-row
      // block, bytes 8 (gi % 2) .. +7 of a 16-byte (16-column) chunk, and receives that
      // chunk's column gi for the 8 rows: rows 8 (g >> 1) + .. (the k group of the
      // 32x32x16 operand) and the chunk of columns 16 (g & 1) of the 32-column subtile.
      // The fp8 chunk swizzle is c ^ (k & 7) (gate/up, 8 chunks per row) or c ^ (k & 15)
      // (down, 16 chunks per row).
      const int gi = lane & 15;
      const int k = 8 * (g >> 1) + (gi >> 1);
      const int col0 = GU ? ch * 64 + jb * 32 : ch * 128 + jb * 32;
      const int chunk = col0 / 16 + (g & 1);
      const int pc = chunk ^ (k & (GU ? 7 : 15));
      b_lane[jb] = (uint32_t)(k * kBPitch + pc * 16 + (gi & 1) * 8);
    } else {
      const int cj = (GU ? ch * 64 + jb * 32 : ch * 128 + jb * 32) >> 3;
      const int chunk = (cj ^ (4 * tr_r)) | (2 * (g & 1) + (tr_c4 >> 1));
      b_lane[jb] = (uint32_t)(((g >> 1) * 8 + tr_r) * kBPitch + chunk * 16 + (tr_c4 & 1) * 8);
    }
  }

  const int ngt = ng_dense + ngroups;
  const int per_xcd = gridDim.x / 8;
  const int q = (gridDim.x % 8 == 0) ? (blockIdx.x % 8) * per_xcd + blockIdx.x / 8 : blockIdx.x;
  int my_groups = 0;  // lane j: the group-list entry of this work group's item (batch + j)
  for (int j = 0;; ++j) {
    const int w = q + j * gridDim.x;
    if (w >= total) break;
    if (j % 64 == 0) {
      if (j > 0) build_groups();   // the ring is idle between items
      const int wl = q + (j + lane) * gridDim.x;
      int gl_g = 0, gl_t = 0;
      if (wl < total) wide_item(wl, ngt, nsingle, n_tiles, gl_g, gl_t);
      const int gl = gl_g - ng_dense;
      my_groups = (wl < total && gl >= 0) ? s_groups[gl] : 0;
      __syncthreads();             // every wave has its entries before the ring refills
    }
    int gidx, nt;
    wide_item(w, ngt, nsingle, n_tiles, gidx, nt);
    const bool in_dense = gidx < ng_dense;
    int e, m0, valid;
    if (in_dense) {
      e = 0;
      m0 = gidx * kWRows;
      valid = min(kWRows, dense_rows - m0);
    } else {
      const int it = __builtin_amdgcn_readlane(my_groups, j % 64);
      const int b = it >> 2, n = it & 3;
      e = meta[3 * b];
      m0 = meta[3 * b + 1];
      valid = meta[3 * (b + n - 1) + 1] + meta[3 * (b + n - 1) + 2] - m0;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    valid = __builtin_amdgcn_readfirstlane(valid);
    const GGOperands& ops = in_dense ? dense : routed;
    bf16_t* const C = ops.C;
    const int n0 = nt * kOutCols;
    const bf16_t* asrc = ops.A + (size_t)m0 * K;
    const unsigned char* b0e = reinterpret_cast<const unsigned char*>(ops.B0) + (size_t)e * K * N * kEB;
    const unsigned char* b1e =
        GU ? reinterpret_cast<const unsigned char*>(ops.B1) + (size_t)e * K * N * kEB : b0e;

    // Copies go out in two groups per slice, each behind one M0 load: the wave's A
    // windows, then its B rows.  Copy i of a group carries the immediate offset 1 KB * i,
    // which moves its LDS destination; its global source is corrected through the lane
    // offset, against a base lowered by the group's largest immediate so that every
    // lane offset stays non-negative.
    //
    // A: window t = wave*CPA + i covers tile rows 16t .. 16t+15, four lanes per row;
    // the logical chunk of lane l is (l & 3) ^ ((l >> 4) & 3) for every window (the
    // swizzle is an involution and depends on the row only through row >> 2).
    // With a gather the source row is the token behind the permuted row, addressed from
    // the start of A (rows of A * K * 2 bytes fit 32 bits; the host checks).
    const int32_t* gat = ops.gather;
    uint32_t a_voff[CPA];
#pragma unroll
    for (int i = 0; i < CPA; ++i) {
      const int row = (wave * CPA + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((lane >> 4) & 3);
      const int rr = row < valid ? row : 0;
      const int src = gat ? gather_row(ops, m0 + rr) : rr;
      a_voff[i] = (uint32_t)(src * K + c * 8) * 2u + (uint32_t)(CPA - 1 - i) * 1024u;
    }
    const unsigned char* a_gbase =
        reinterpret_cast<const unsigned char*>(gat ? ops.A : asrc) - (CPA - 1) * 1024;
    const int a_ldst = wave * CPA * 1024;
    // B: copy u = wave*CPB + p.  GATEUP: u < 8 moves W1 rows 4u'..4u'+3 (u' = u % 8;
    // u >= 8: the same rows of W3), 16 lanes per 256-byte row, and the logical chunk of
    // lane l is (l & 15) ^ 4 * ((l >> 4) & 3) for every u.  DOWN: copy u moves rows 2u,
    // 2u+1, 32 lanes per 512-byte row; the chunk depends on u through its parity, which
    // is p's parity (CPB is even).
    const int u0 = wave * CPB;
    uint32_t b_voff[CPB];
    const unsigned char* b_gbase;
    int b_ldst;
    if constexpr (FP8) {
      // fp8 B: one copy per wave and slice.  GATEUP: copy u < 4 moves W1 rows 8u..8u+7
      // (u >= 4: the same rows of W3), 8 lanes per 128-byte row; DOWN: copy u moves rows
      // 4u..4u+3, 16 lanes per 256-byte row.  Lane l's logical chunk is its position
      // XOR the row's swizzle (k & 7, or k & 15).
      const int rows_per = GU ? 8 : 4;
      const int uu = GU ? (u0 & 3) : u0;
      const int kl = GU ? (lane >> 3) : (lane >> 4);
      const int k = rows_per * uu + kl;
      const int cpos = GU ? (lane & 7) : (lane & 15);
      int col = n0 + (cpos ^ (k & (GU ? 7 : 15))) * 16;   // past N -> column 0
      if (col >= N) col = 0;
      b_voff[0] = (uint32_t)(kl * N + col);
      b_gbase = (GU ? (u0 < 4 ? b0e : b1e) : b0e) + (size_t)rows_per * uu * N;
      b_ldst = kWABytes + (GU ? (u0 >> 2) * (kBBytes / 2) + uu * 1024 : u0 * 1024);
    } else {
#pragma unroll
      for (int p = 0; p < CPB; ++p) {
        const int kl = GU ? (lane >> 4) : (lane >> 5);
        const int k = GU ? kl : 2 * (p & 1) + kl;           // row within the slice, mod 4
        const int cpos = GU ? (lane & 15) : (lane & 31);
        int col = n0 + swz_b(k, cpos) * 8;                  // past N -> column 0
        if (col >= N) col = 0;
        const int rows_before = (GU ? 4 : 2) * p;           // slice rows of earlier copies
        b_voff[p] = (uint32_t)((rows_before + kl) * N + col) * 2u + (uint32_t)(CPB - 1 - p) * 1024u;
      }
      if (GU) {
        b_gbase = (u0 < 8 ? b0e : b1e) + (size_t)4 * (u0 & 7) * N * 2;
        b_ldst = kWABytes + (u0 >> 3) * (kWBBytes / 2) + (u0 & 7) * 1024;
      } else {
        b_gbase = b0e + (size_t)2 * u0 * N * 2;
        b_ldst = kWABytes + u0 * 1024;
      }
      b_gbase -= (CPB - 1) * 1024;
    }
    // fp8: the scales of this item's columns, one per 128-deep k-block (wave-uniform:
    // gate/up's 64 act columns of a wave lie in one 128-column block of W1 and of W3,
    // down's 128 columns in one block)
    const int KBq = (K + 127) / 128, NBq = (N + 127) / 128;
    // (read through the constant address space: wave-uniform scalar loads into SGPRs,
    // which the copies' vmcnt waits do not count)
    typedef const __attribute__((address_space(4))) float* cfloat_p;
    cfloat_p sc0 = nullptr;
    cfloat_p sc1 = nullptr;
    if constexpr (FP8) {
      const int nb = GU ? (n0 >> 7) : ((n0 + ch * 128) >> 7);
      sc0 = (cfloat_p)uniform_ptr(ops.S0 + (size_t)e * KBq * NBq + nb);
      sc1 = GU ? (cfloat_p)uniform_ptr(ops.S1 + (size_t)e * KBq * NBq + nb) : sc0;
    }
    // copy i of slice ks's A group (i == 0 loads M0 first) into ring slot `slot`
    auto issue_a = [&](int ks, int slot, int i) {
      if (i == 0) set_lds_dma_base(lds + slot * kStage + a_ldst);
      copy16_to_lds_nth(i, a_gbase + (size_t)ks * (kWBK * 2), a_voff[i]);
    };
    auto issue_b = [&](int ks, int slot, int p) {
      if (p == 0) set_lds_dma_base(lds + slot * kStage + b_ldst);
      copy16_to_lds_nth(p, b_gbase + (size_t)ks * kWBK * N * kEB, b_voff[p]);
    };
    auto issue = [&](int ks) {
#pragma unroll
      for (int i = 0; i < CPA; ++i) issue_a(ks, ks % kStages, i);
#pragma unroll
      for (int p = 0; p < CPB; ++p) issue_b(ks, ks % kStages, p);
    };

    f32x16_t acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // One set of fragment registers (192 accumulators leave no room for two): the
    // other wave on the SIMD covers each wave's LDS read latency.
    bf16x8_t af[MI], bf[4];
    // fp8: the memory phase only reads the codes (8 per lane and fragment) and the
    // block scales; the MFMA phase dequantises fragment j (code * scale, rounded to
    // nearest even: the values moe_dequantize_fp8 writes) while the MFMAs of fragment
    // j-1 run, so the conversion overlaps the matrix pipe and no more registers are live
    // than with bf16 fragments.
    typedef int v2i __attribute__((ext_vector_type(2)));
    v2i braw[FP8 ? 4 : 1];
    float s_g = 0.f, s_u = 0.f;
    auto dequant = [&](int j) {
      const float sc = (GU && j >= 2) ? s_u : s_g;
      bf16x8_t o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(braw[j][h], false);   // bytes 0, 1
        const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(braw[j][h], true);    // bytes 2, 3
        o[4 * h + 0] = static_cast<__bf16>(f0[0] * sc);
        o[4 * h + 1] = static_cast<__bf16>(f0[1] * sc);
        o[4 * h + 2] = static_cast<__bf16>(f1[0] * sc);
        o[4 * h + 3] = static_cast<__bf16>(f1[1] * sc);
      }
      return o;
    };
    // the fragments and MFMAs of the wave's first NL subtiles (its live ones)
    auto read_frags = [&](int ks, int kk, auto nl_c) {
      constexpr int NL = decltype(nl_c)::value;
      if constexpr (NL == 0) return;
      const unsigned char* sa = lds + (ks % kStages) * kStage;
      const unsigned char* sb = sa + kWABytes;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + a_lane[kk] + i * NP * 2048);
      if constexpr (FP8) {
        const int kb = (ks * kWBK) >> 7;
        s_g = sc0[(size_t)kb * NBq];
        s_u = GU ? sc1[(size_t)kb * NBq] : s_g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned char* hb = sb + (GU ? (j >> 1) * (kBBytes / 2) + b_lane[j & 1] : b_lane[j]) +
                                    kk * 16 * kBPitch;
          braw[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MOE_LDS v2i*)hb);
        }
        bf[0] = dequant(0);   // ready when this wave's MFMA phase starts
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned char* hb = sb + (GU ? (j >> 1) * (kWBBytes / 2) + b_lane[j & 1] : b_lane[j]) +
                                    kk * 16 * kBPitch;
          i16x4_t hv[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(hb + hh * 4 * kBPitch));
          bf[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto mfma_block = [&](auto nl_c) {
      constexpr int NL = decltype(nl_c)::value;
      if constexpr (NL == 0) return;
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t b = j == 0 ? bf[0] : dequant(j);
#pragma unroll
          for (int i = 0; i < NL; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], b, acc[i][j], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    };
    using AllSub = std::integral_constant<int, MI>;

    // Prologue: every slot in flight (slices past the end re-copy the last slice into a
    // slot that is never read again, so every slice issues the same number of copies
    // and the waits are constants), then wait for slice 0.
#pragma unroll
    for (int p = 0; p < kStages; ++p) issue(min(p, nk - 1));
    MOE_WAIT_VMCNT((kStages - 1) * CPW);
    __syncthreads();

    // Ping-pong over half-slices t = 2 ks + kk: every wave runs MEM(t), barrier,
    // MFMA(t), barrier.  Waves 4-7 (the second wave on each SIMD) start one barrier
    // late and waves 0-3 end one barrier late, so on every SIMD one wave issues its
    // MFMAs while the other reads its fragments (and issues copies): the LDS reads of
    // half the waves overlap the other half's MFMAs instead of all waves reading at
    // once after a shared barrier.  Every wave executes 4 nk + 1 barriers.
    //   MEM(2 ks), ks >= 1: slice ks+1 has landed for this wave (then, before any wave
    //   reads it, at least two barriers pass); every wave has read slice ks-1 (its
    //   reads completed before the barriers since), so its slot takes slice ks-1+S
    //   (the A copies; the B copies in MEM(2 ks + 1)).  The wait counts whole slices:
    //   at MEM(2 ks) every slice up to ks-2+S has been issued in full.
    // The loop is instantiated per number of live subtiles (1 .. MI); every instance
    // issues the same copies and barriers.
    const int live = __builtin_amdgcn_readfirstlane(
        [&] { int n = 0; for (int i = 0; i < MI; ++i) n += rsub(i) < valid; return n; }());
    const bool lag = wave >= kWideLagFrom;
    if (lag) __syncthreads();
    // One half-slice: MEM(2 ks + KK), barrier, MFMA(2 ks + KK), barrier.  KK and the
    // first slice are compile-time, so the steady state branches only on the lag and at
    // the end of each slice.
    auto half = [&](int ks, auto kk_c, auto first_c, auto nl_c) {
      constexpr int KK = decltype(kk_c)::value;
      // first_c: std::true_type / std::false_type, or a bool decided at run time
      bool first;
      if constexpr (std::is_same_v<decltype(first_c), bool>) first = first_c;
      else first = decltype(first_c)::value;
      // the refill of slice ks-1's slot (after every wave's last read of slice ks-1):
      // the A copies in the first half's memory phase, the B copies in the second
      // half's (measured faster for both ops than all copies in the first half, for
      // gate/up once its barriers stopped waiting for the fragment reads)
      const int ksrc = min(ks - 1 + kStages, nk - 1);
      const int slot = (ks + kStages - 1) % kStages;
      if constexpr (KK == 0) {
        if (first) {
          MOE_WAIT_VMCNT((kStages - 2) * CPW);   // slice 1 has landed
        } else {
          MOE_WAIT_VMCNT((kStages - 3) * CPW);   // slice ks+1 has landed
#pragma unroll
          for (int i = 0; i < CPA; ++i) issue_a(ksrc, slot, i);
        }
      } else if (!first) {
#pragma unroll
        for (int c = 0; c < CPB; ++c) issue_b(ksrc, slot, c);
      }
      read_frags(ks, KK, nl_c);
      // scheduling barriers keep each phase's instructions on its side of the barriers
      __builtin_amdgcn_sched_barrier(0);
      // The barrier after a memory phase does not wait for the phase's fragment reads
      // (the MFMAs wait for their operands), so the other wave on the SIMD starts its
      // memory phase under them, except where a refill follows: the lagging waves'
      // second-half reads are the last reads of slice ks, whose slot the other waves
      // refill right after this barrier (MEM(2 ks + 2)).  The other waves' reads of a
      // slice complete before their own MFMA phase, before the barrier ahead of any
      // refill of that slot.
      if constexpr (KK == 1) {
        if (lag) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mfma_block(nl_c);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    // The same schedule with the half and the first slice decided at run time (one
    // loop body).
    auto ping_pong_rt = [&](auto nl_c) {
    for (int t = 0; t < 2 * nk; ++t) {
      const int ks = t >> 1, kk = t & 1;
      // the refill of slice ks-1's slot (after every wave's last read of slice ks-1):
      // the A copies in the first half's memory phase, the B copies in the second
      // half's (measured faster for both ops than all copies in the first half, for
      // gate/up once its barriers stopped waiting for the fragment reads)
      const int ksrc = min(ks - 1 + kStages, nk - 1);
      const int slot = (ks + kStages - 1) % kStages;
      if (kk == 0) {
        if (ks == 0) {
          MOE_WAIT_VMCNT((kStages - 2) * CPW);   // slice 1 has landed
        } else {
          MOE_WAIT_VMCNT((kStages - 3) * CPW);   // slice ks+1 has landed
#pragma unroll
          for (int i = 0; i < CPA; ++i) issue_a(ksrc, slot, i);
        }
      } else if (ks > 0) {
#pragma unroll
        for (int c = 0; c < CPB; ++c) issue_b(ksrc, slot, c);
      }
      read_frags(ks, kk, nl_c);
      // scheduling barriers keep each phase's instructions on its side of the barriers
      __builtin_amdgcn_sched_barrier(0);
      // The barrier after a memory phase does not wait for the phase's fragment reads
      // (the MFMAs wait for their operands), so the other wave on the SIMD starts its
      // memory phase under them, except where a refill follows: the lagging waves'
      // second-half reads are the last reads of slice ks, whose slot the other waves
      // refill right after this barrier (MEM(2 ks + 2)).  The other waves' reads of a
      // slice complete before their own MFMA phase, before the barrier ahead of any
      // refill of that slot.
      if (lag && kk == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mfma_block(nl_c);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    };
    // The bf16 forward ops run the first slice on its own and then both halves of each
    // slice with no branch between them.  The SwiGLU-backward op unrolls the two halves
    // but tests for the first slice at run time, and the fp8 ops keep one loop over
    // half-slices: with the duplicated first slice their register allocation puts spill
    // reloads into the loop.
    auto ping_pong = [&](auto nl_c) {
      if constexpr (!FP8 && !BWD) {
        half(0, K0{}, std::true_type{}, nl_c);
        half(0, K1{}, std::true_type{}, nl_c);
        for (int ks = 1; ks < nk; ++ks) {
          half(ks, K0{}, std::false_type{}, nl_c);
          half(ks, K1{}, std::false_type{}, nl_c);
        }
      } else if constexpr (BWD) {
        for (int ks = 0; ks < nk; ++ks) {
          half(ks, K0{}, ks == 0, nl_c);
          half(ks, K1{}, ks == 0, nl_c);
        }
      } else {
        ping_pong_rt(nl_c);
      }
    };
    // The SwiGLU-backward op runs one instance over every subtile: with one instance
    // per live count its register-heavy epilogue pushes spill reloads (and the waits
    // for them, which also drain the copies in flight) into the K loop.
    if constexpr (BWD) ping_pong(AllSub{});
    else dispatch_live<MI>(live, ping_pong);
    if (!lag) __syncthreads();
    MOE_WAIT_VMCNT(0);  // no copy may land in the ring once it is reused below
    __syncthreads();

    // Epilogue through LDS: each wave converts 64 output columns at a time to bf16 into
    // a private [WR][64 + 8] staging tile, then stores whole 16-byte row chunks.  32x32
    // accumulator layout: element q of lane l is row (q/4)*8 + (l/32)*4 + q%4, column
    // l%32 of the subtile.
    if constexpr (BWD) {
      // SwiGLU backward (op 2): per 32-row subtile, the wave's [32][64] block of the
      // incoming gradient dact is copied to LDS (four 16-byte copies per lane; rows past
      // the valid ones and columns past N read row 0 / column 0, never stored), then dg
      // and du are computed from one sigmoid, staged side by side and stored into
      // C = [rows, 2N] (dg in columns [0, N), du in [N, 2N)).
      constexpr int kLd = 64 + 8;
      bf16_t* so = reinterpret_cast<bf16_t*>(lds) + wave * 2 * 32 * kLd;
      unsigned char* sda = lds + NW * 2 * 32 * kLd * 2 + wave * 4096;
      const bf16_t* dbase = uniform_ptr(ops.D + (size_t)m0 * N);
      const int dcol = n0 + ch * 64 + (lane & 7) * 8;
      const int dcc = dcol < N ? dcol : 0;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r0s = rsub(i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = r0s + 8 * j + (lane >> 3);
          const int rr = r < valid ? r : 0;
          copy16_to_lds(dbase, (uint32_t)(rr * N + dcc) * 2u, sda + j * 1024);
        }
        MOE_WAIT_VMCNT(0);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int c = jj * 32 + (lane & 31);
            const float da = bf16_to_f32(*reinterpret_cast<const bf16_t*>(sda + (r * 64 + c) * 2));
            const float gv = acc[i][jj][q], uv = acc[i][jj + 2][q];
            const float sg = sigmoid_f32(gv);
            so[r * kLd + c] = f32_to_bf16(da * uv * (sg * (1.0f + gv * (1.0f - sg))));
            so[(32 + r) * kLd + c] = f32_to_bf16(da * gv * sg);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
          for (int r0 = 0; r0 < 32; r0 += 8) {
            const int r = r0 + (lane >> 3);
            const int grow = r0s + r;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(so + (ps * 32 + r) * kLd + (lane & 7) * 8);
            if (grow < valid && dcol < N)
              *reinterpret_cast<u32x4_t*>(C + (size_t)(m0 + grow) * 2 * N + ps * N + dcol) = v;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    } else {
    constexpr int kLd = 64 + 8;
    constexpr int kPasses = GU ? 1 : 2;
    bf16_t* stg = reinterpret_cast<bf16_t*>(lds) + wave * WR * kLd;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            float v;
            if (GU) {
              v = silu_f32(acc[i][jj][q]) * acc[i][jj + 2][q];
            } else {
              v = acc[i][ps * 2 + jj][q];
            }
            stg[r * kLd + jj * 32 + (lane & 31)] = f32_to_bf16(v);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int col0 = n0 + (GU ? ch * 64 : ch * 128 + ps * 64);
#pragma unroll 4
      for (int r0 = 0; r0 < WR; r0 += 8) {
        const int r = r0 + (lane >> 3);
        const int c8 = lane & 7;
        const int grow = rsub(r0 >> 5) + (r & 31);   // staging row r: subtile r / 32
        const int gcol = col0 + c8 * 8;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * kLd + c8 * 8);
        if (grow < valid && gcol < N)
          *reinterpret_cast<u32x4_t*>(C + (size_t)(m0 + grow) * N + gcol) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    }
    __syncthreads();  // staging reads done before the next item refills the ring
  }
}

static constexpr int kWideWaves = 8;

moe_status launch_gg_wide(int op, const GGOperands& ro, const GGOperands& dn, int K, int N,
                          const int32_t* block_meta, const int32_t* num_blocks, int32_t max_blocks,
                          int64_t max_rows, int E, int32_t dense_rows, hipStream_t st, bool fp8) {
  const int out_cols = op == MOE_OP_DOWN ? 256 : 128;
  const int n_tiles = (int)ceil_div(N, out_cols);
  // groups: at most one per block, and at most a third of the blocks plus one per expert
  const int64_t mb = max_blocks > 0 ? max_blocks : 0;
  const int64_t groups_ub = std::min<int64_t>(mb, ceil_div(mb, 3) + std::min<int64_t>(E, mb)) +
                            ceil_div(dense_rows, kWRows);
  const int64_t items = groups_ub * n_tiles;
  const int cus = device_cu_count();
  int64_t grid = items < cus ? items : cus;
  // MOE_GG_GRID_CAP=n caps the persistent grid (tests use it so that one work group
  // walks more than 64 items and rebuilds its group list)
  if (const char* cap = getenv("MOE_GG_GRID_CAP")) {
    const int64_t c = atoll(cap);
    if (c >= 1 && c < grid) grid = c;
  }
  if (grid < 1) grid = 1;
  constexpr int NT = kWideWaves * 64;
#define MOE_WIDE_LAUNCH(OPV, F8)                                                               \
  hipLaunchKernelGGL((k_gg_wide<OPV, kWideWaves, F8>), dim3((unsigned)grid), dim3(NT), 0, st, ro, \
                     dn, K, N, block_meta, num_blocks, max_blocks, E, max_rows, dense_rows, n_tiles)
  if (fp8) {
    if (op == MOE_OP_GATEUP_SWIGLU) MOE_WIDE_LAUNCH(MOE_OP_GATEUP_SWIGLU, true);
    else if (op == MOE_OP_DOWN) MOE_WIDE_LAUNCH(MOE_OP_DOWN, true);
    else return MOE_ENOTSUP;
  } else if (op == MOE_OP_GATEUP_SWIGLU) {
    MOE_WIDE_LAUNCH(MOE_OP_GATEUP_SWIGLU, false);
  } else if (op == kOpGateUpBwd) {
    MOE_WIDE_LAUNCH(kOpGateUpBwd, false);
  } else {
    MOE_WIDE_LAUNCH(MOE_OP_DOWN, false);
  }
#undef MOE_WIDE_LAUNCH
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
