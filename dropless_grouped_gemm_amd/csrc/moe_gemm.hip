// Grouped GEMM over contiguous, block_m-aligned expert segments.
//
// One launch covers every expert.  The kernel is organised by output tile, not by
// expert: a work item is (row block, column tile); the row block's entry in the
// device-side table [expert, m_start, valid_m] says which expert's weights to read,
// so a tile only ever loads its own expert's weight panel and no capacity box or
// dense batched layout exists (TileLang chapter "MoE, MLA and sparse-attention
// operators", section 2.4 (a); dropless notes sections 3, 5 and 7).  The grid is
// persistent and sized from a host-side upper bound; the real number of blocks is
// read from device memory, so the host never synchronises.
//
// GATEUP_SWIGLU is the dual GEMM: one pass over A feeds both W1 (gate) and W3 (up)
// and the epilogue writes silu(gate) * up (TileLang chapter section 2.4 (c)); DOWN is
// the plain second GEMM.
//
// bf16 kernel (gfx950):
//   * 256 threads = 4 waves; work tile 128 rows x 256 B-columns x 64 K per stage.
//     GATEUP: 128 gate + 128 up columns -> a 128 x 128 act tile.  DOWN: 128 x 256.
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulators: every wave owns all 128 rows and
//     64 B-columns (GATEUP: 32 gate + the 32 matching up columns, so the SiLU*mul
//     epilogue is register-local).
//   * LDS double buffer (2 x 48 KB).  A and B are both stored K-contiguous with a
//     16-byte-chunk XOR swizzle (chunk ^ (row & 7)), so MFMA operand reads
//     (ds_read_b128, 32 consecutive rows at one chunk) are bank-conflict free.
//   * Weights are row-major [K, N] (N contiguous).  Each thread loads an 8 x 8 (k x n)
//     block with eight 16-byte loads and transposes it in registers before the LDS
//     store, so W never needs a separate transposed copy.
//   * Rows past valid_m and columns past N are never read or written; K tails are
//     zero-filled in the staging loads.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "moe_gemm_common.h"

namespace moe {

static constexpr int kBM = 128;     // rows per tile
static constexpr int kBK = 64;      // K per pipeline stage
static constexpr int kBNB = 256;    // B columns per tile
static constexpr int kThreads = 256;
static constexpr int kALdsBytes = kBM * kBK * 2;        // 16 KB
static constexpr int kBLdsBytes = kBNB * kBK * 2;       // 32 KB
static constexpr int kStageBytes = kALdsBytes + kBLdsBytes;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }


template <int OP>
__global__ void __launch_bounds__(kThreads, 1)
k_gg_bf16(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0,
          const bf16_t* __restrict__ B1, bf16_t* __restrict__ C, int K, int N,
          const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
          int max_blocks, int E, int64_t max_rows, int dense_rows, int block_m, int n_tiles) {
  __shared__ __align__(16) unsigned char lds[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kOutCols = OP == MOE_OP_GATEUP_SWIGLU ? 128 : 256;
  const int tpb = block_m / kBM;  // 128-row sub-tiles per metadata block
  const int nblocks =
      dense_rows > 0 ? (dense_rows + block_m - 1) / block_m : clamp_block_count(num_blocks_ptr, max_blocks);
  const int total = nblocks * tpb * n_tiles;
  const int nk = (K + kBK - 1) / kBK;

  // Staging-load roles.
  const int a_chunk = tid & 7;        // 16-byte chunk of the 128-byte A row slice
  const int a_row0 = tid >> 3;        // rows a_row0 + 32 i
  const int b_kg = tid & 7;           // k rows b_kg*8 .. +7
  const int b_ng = tid >> 3;          // B columns b_ng*8 .. +7 (of 256)

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int nt = w % n_tiles;
    const int mt = w / n_tiles;
    Tile tile;
    if (!decode_block(mt / tpb, mt % tpb, kBM, block_m, meta, dense_rows, E, max_rows, tile)) continue;
    const int n0 = nt * kOutCols;

    // B source for this thread's 8 columns.
    const bf16_t* bsrc;
    int bcol;
    if (OP == MOE_OP_GATEUP_SWIGLU) {
      const bool up = b_ng >= 16;
      bcol = n0 + (b_ng & 15) * 8;
      bsrc = (up ? B1 : B0) + (size_t)tile.e * K * N;
    } else {
      bcol = n0 + b_ng * 8;
      bsrc = B0 + (size_t)tile.e * K * N;
    }
    const bool bcol_ok = bcol < N;
    const bf16_t* asrc = A + (size_t)tile.m0 * K;

    u32x4_t ra[4];
    u32x4_t rb[8];
    auto load_global = [&](int ks) {
      const int k0 = ks * kBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = a_row0 + 32 * i;
        const int kk = k0 + a_chunk * 8;
        if (r < tile.valid && kk < K)
          ra[i] = *reinterpret_cast<const u32x4_t*>(asrc + (size_t)r * K + kk);
        else
          ra[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kk = k0 + b_kg * 8 + r;
        if (bcol_ok && kk < K)
          rb[r] = *reinterpret_cast<const u32x4_t*>(bsrc + (size_t)kk * N + bcol);
        else
          rb[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    auto store_lds = [&](int stage) {
      unsigned char* sa = lds + stage * kStageBytes;
      unsigned char* sb = sa + kALdsBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = a_row0 + 32 * i;
        *reinterpret_cast<u32x4_t*>(sa + r * 128 + swz(r, a_chunk) * 16) = ra[i];
      }
      // transpose the 8 (k) x 8 (n) block: column c gets the 8 k values of n = 8*b_ng + c
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int m = c >> 1;
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = rb[2 * q][m], hi = rb[2 * q + 1][m];
          v[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int n = b_ng * 8 + c;
        *reinterpret_cast<u32x4_t*>(sb + n * 128 + swz(n, b_kg) * 16) = v;
      }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // B rows (LDS "n" index) of this wave's two 32-column subtiles.
    const int nsub0 = OP == MOE_OP_GATEUP_SWIGLU ? wave * 32 : wave * 64;
    const int nsub1 = OP == MOE_OP_GATEUP_SWIGLU ? 128 + wave * 32 : wave * 64 + 32;

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int stage = ks & 1;
      if (ks + 1 < nk) load_global(ks + 1);
      const unsigned char* sa = lds + stage * kStageBytes;
      const unsigned char* sb = sa + kALdsBytes;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int chunk = kk * 2 + (lane >> 5);
        bf16x8_t af[4], bf[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8_t*>(sa + r * 128 + swz(r, chunk) * 16);
        }
        {
          const int n = nsub0 + (lane & 31);
          bf[0] = *reinterpret_cast<const bf16x8_t*>(sb + n * 128 + swz(n, chunk) * 16);
          const int n1 = nsub1 + (lane & 31);
          bf[1] = *reinterpret_cast<const bf16x8_t*>(sb + n1 * 128 + swz(n1, chunk) * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if (ks + 1 < nk) store_lds(stage ^ 1);
      __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: element q of lane l is row
    // (q/4)*8 + (l/32)*4 + q%4, column l%32 of the 32x32 subtile.
    const int col_in = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        if (r >= tile.valid) continue;
        bf16_t* crow = C + (size_t)(tile.m0 + r) * N;
        if (OP == MOE_OP_GATEUP_SWIGLU) {
          const int col = n0 + wave * 32 + col_in;
          if (col < N) crow[col] = f32_to_bf16(silu_f32(acc[i][0][q]) * acc[i][1][q]);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = n0 + wave * 64 + j * 32 + col_in;
            if (col < N) crow[col] = f32_to_bf16(acc[i][j][q]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel, asynchronous-copy version (K % 32 == 0).
//
//   * Work tile 128 rows x 512 B-columns, 8 waves (two per SIMD, so one wave's MFMAs
//     cover the other's copies, LDS reads and barrier waits).  Wave w owns all 128
//     rows and 64 B-columns: GATEUP gate columns [32w, 32w+32) with the matching up
//     columns, DOWN columns [64w, 64w+64); a 4 x 2 grid of 32x32 accumulators.
//   * Operands go HBM -> LDS with 16-byte global_load_lds copies into a 3-stage ring
//     of 32-deep K slices.  Every copy has a wave-uniform SGPR base and a per-lane
//     32-bit offset that is fixed for the whole tile.
//   * A (rows, K-contiguous) is read with ds_read_b128.  B stays [k][n] in LDS, split
//     in two 256-column halves (GATEUP: W1 and W3; DOWN: the two halves of the 512
//     columns), and is read with ds_read_b64_tr_b16: in each 16-lane group lane 4r+c
//     points at row r, columns 4c..4c+3 of a 4 x 16 block and receives column
//     (lane % 16), so two such reads give a lane the 8 consecutive k values of one
//     column that the 32x32x16 MFMA takes.
//   * LDS swizzles (16-byte chunks) measured conflict-free on gfx950: A chunk c of
//     row r at c ^ ((r >> 2) & 3); B chunk c of row k at c ^ 4 * (k & 3).
//   * Rows past valid_m and columns past N copy row 0 / column 0 instead (their
//     results are never stored), so every lane issues every copy and the copy count
//     per slice is uniform - the vmcnt-based waits rely on that.
// ---------------------------------------------------------------------------
static constexpr int kV2Threads = 512;            // 8 waves
static constexpr int kV2BK = 32;                  // K per stage
static constexpr int kV2NB = 512;                 // B columns per tile
static constexpr int kV2ABytes = kBM * kV2BK * 2; // 8 KB
static constexpr int kV2BHalf = kV2BK * 256 * 2;  // 16 KB per 256-column half
static constexpr int kV2Stage = kV2ABytes + 2 * kV2BHalf;
static constexpr int kV2Stages = 4;
static constexpr int kV2CopiesPerThread = 1 + 4;  // A: 8 windows / 8 waves, B: 32 / 8
static constexpr bool kUseSuper = false;  // XCD-aware super-tile order
static constexpr int kGroupM = 16, kGroupN = 2;







// One launch covers two segment sets with the same K and N: a dense segment of
// dense_rows rows through one expert (the shared expert; dense_rows == 0: none),
// taken first, then the routed segments of the block table (max_blocks == 0: none).
template <int OP>
__global__ void __launch_bounds__(kV2Threads, 1)
k_gg_bf16_v2(GGOperands routed, GGOperands dense, int K, int N,
             const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
             int max_blocks, int E, int64_t max_rows, int dense_rows, int block_m,
             int n_tiles) {
  __shared__ __align__(1024) unsigned char lds[kV2Stages * kV2Stage];
  // op 2 (kOpGateUpBwd) runs the gate/up main loop; its epilogue writes dg | du
  constexpr bool GU = OP == MOE_OP_GATEUP_SWIGLU || OP == kOpGateUpBwd;
  constexpr bool BWD = OP == kOpGateUpBwd;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int kOutCols = GU ? 256 : 512;
  const int tpb = block_m / kBM;
  const int nb_dense = (dense_rows + block_m - 1) / block_m;
  const int nblocks = nb_dense + (max_blocks > 0 ? clamp_block_count(num_blocks_ptr, max_blocks) : 0);
  const int total = nblocks * tpb * n_tiles;
  const int nk = K / kV2BK;

  // B-fragment geometry (fixed per lane): 16-lane group g, row r, column quad c4, and
  // for each of the wave's two 32-column subtiles its LDS half and first column.
  const int g = lane >> 4, gi = lane & 15, tr_r = gi >> 2, tr_c4 = gi & 3;
  int bhalf[2], bcol0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bhalf[j] = GU ? j : wave >> 2;
    bcol0[j] = GU ? wave * 32 : (wave & 3) * 64 + j * 32;
  }

  // Work order.  Work groups are dispatched to the 8 XCDs round-robin (group b on
  // XCD b % 8), and each XCD has its own L2.  Tiles are taken in super-tiles of
  // kGroupM row blocks x kGroupN column tiles, one super-tile per XCD at a time, so
  // the 32 groups of an XCD share kGroupM A blocks and kGroupN B panels in its L2.
  const int nm = nblocks * tpb;
  const int mgroups = (nm + kGroupM - 1) / kGroupM;
  const int ngroups = (n_tiles + kGroupN - 1) / kGroupN;
  const int n_super = mgroups * ngroups;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, slots = gridDim.x / 8;
  const bool use_super = kUseSuper && gridDim.x % 8 == 0 && slots == kGroupM * kGroupN;
  const int iters = use_super ? (n_super + 7) / 8 : (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  for (int it = 0; it < iters; ++it) {
    int nt, mt;
    if (use_super) {
      const int sidx = xcd + 8 * it;
      if (sidx >= n_super) break;
      const int mg = sidx % mgroups, ng = sidx / mgroups;
      mt = mg * kGroupM + slot / kGroupN;
      nt = ng * kGroupN + slot % kGroupN;
      if (mt >= nm || nt >= n_tiles) continue;
    } else {
      const int w = blockIdx.x + it * gridDim.x;
      nt = w % n_tiles;
      mt = w / n_tiles;
    }
    Tile tile;
    const int blk = mt / tpb;
    const bool in_dense = blk < nb_dense;
    if (in_dense) {
      if (!decode_block(blk, mt % tpb, kBM, block_m, nullptr, dense_rows, 1, dense_rows, tile))
        continue;
    } else {
      if (!decode_block(blk - nb_dense, mt % tpb, kBM, block_m, meta, 0, E, max_rows, tile))
        continue;
    }
    const GGOperands& ops = in_dense ? dense : routed;
    bf16_t* const C = ops.C;
    const int n0 = nt * kOutCols;
    const bf16_t* asrc = ops.A + (size_t)tile.m0 * K;
    const bf16_t* b0e = ops.B0 + (size_t)tile.e * K * N;
    const bf16_t* b1e = GU ? ops.B1 + (size_t)tile.e * K * N : b0e;
    // the two 256-column halves of the tile's B columns: matrix and first column
    const bf16_t* bh_base[2] = {b0e, GU ? b1e : b0e};
    const int bh_col0[2] = {n0, GU ? n0 : n0 + 256};

    // A copy (one per wave per slice): window = this wave's 16 rows.
    uint32_t a_voff;
    {
      const int row = wave * 16 + (lane >> 2);
      const int c = swz_a(row, lane & 3);   // the swizzle is an involution
      const int rr = row < tile.valid ? row : 0;
      // with a gather: the token behind the permuted row, addressed from the start of A
      const int src = ops.gather ? gather_row(ops, tile.m0 + rr) : rr;
      a_voff = (uint32_t)(src * K + c * 8) * 2u;
    }
    asrc = uniform_ptr(ops.gather ? ops.A : asrc);
    // B copies: instruction i of this wave covers rows 2p, 2p+1 of half h, where
    // (h, p) = ((wave*4 + i) / 16, (wave*4 + i) % 16); lanes 0-31 take row 2p, lanes
    // 32-63 row 2p+1.  The lane offset depends on the row parity only through the
    // swizzle (k & 3 = 2*(p & 1) + lane/32), so two offsets per half suffice.
    uint32_t b_voff[2][2];  // [half][p & 1]
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int k = 2 * pp + (lane >> 5);
        const int c = swz_b(k, lane & 31);
        int col = bh_col0[h] + c * 8;     // absolute column; past N -> column 0
        if (col >= N) col = 0;
        b_voff[h][pp] = (uint32_t)((lane >> 5) * N + col) * 2u;
      }
    // copy `part` (0: this wave's A window, 1..4: its B row pairs) of slice ks into
    // ring slot `slot`
    auto issue_part_to = [&](int ks, int slot, int part) {
      unsigned char* st = lds + slot * kV2Stage;
      const int k0 = ks * kV2BK;
      if (part == 0) {
        copy16_to_lds(asrc + k0, a_voff, st + wave * 1024);
      } else {
        const int q = wave * 4 + part - 1;  // 0..31: half q / 16, row pair q % 16
        const int h = q >> 4, pr = q & 15;
        copy16_to_lds(bh_base[h] + (size_t)(k0 + 2 * pr) * N, b_voff[h][pr & 1],
                      st + kV2ABytes + h * kV2BHalf + pr * 1024);
      }
    };
    auto issue = [&](int ks) {
#pragma unroll
      for (int part = 0; part < kV2CopiesPerThread; ++part) issue_part_to(ks, ks % kV2Stages, part);
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // 32-row subtiles holding valid rows (decode: usually one): the others are neither
    // read nor multiplied, so a weight-streaming item does a quarter of the MFMAs.
    const int nsub = __builtin_amdgcn_readfirstlane(min(4, (tile.valid + 31) >> 5));
    bf16x8_t af0[4], bf0[2], af1[4], bf1[2];
    auto read_frags = [&](int stage, int kk, bf16x8_t* a, bf16x8_t* b) {
      const unsigned char* sa = lds + stage * kV2Stage;
      const unsigned char* sb = sa + kV2ABytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nsub) break;
        const int row = i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8_t*>(sa + row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16);
      }
      const int kbase = kk * 16 + (g >> 1) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ncol = bcol0[j] + (g & 1) * 16 + 4 * tr_c4;
        const unsigned char* hb = sb + bhalf[j] * kV2BHalf;
        i16x4_t hv[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = kbase + hh * 4 + tr_r;
          hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MOE_LDS i16x4_t*)(hb + k * 512 + swz_b(k, ncol >> 3) * 16 + (ncol & 7) * 2));
        }
        b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto mfma_block = [&](const bf16x8_t* a, const bf16x8_t* b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nsub) break;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    };

    // Prologue: every slot in flight (slices past the end re-copy the last slice into
    // a slot that is never read again, so every iteration issues the same number of
    // copies and the waits below are constants), then wait for slice 0.
#pragma unroll
    for (int p = 0; p < kV2Stages; ++p) issue(min(p, nk - 1));
    MOE_WAIT_VMCNT((kV2Stages - 1) * kV2CopiesPerThread);
    __syncthreads();
    read_frags(0, 0, af0, bf0);

    // Slice ks: the barrier sits between its two 16-deep halves, so while the waves
    // sync and fetch slice ks+1's first fragments, the second half's MFMAs are still
    // to issue.  Slot ks % S is refilled with slice ks+S right after the barrier,
    // once every wave has read it; the refill copies are spread between the second
    // half's MFMAs (a burst of copies right after the barrier stalls the waves on the
    // memory-instruction queue).
    for (int ks = 0; ks < nk - 1; ++ks) {
      read_frags(ks % kV2Stages, 1, af1, bf1);
      mfma_block(af0, bf0);
      // slice ks+1 has landed once only slices ks+2 .. ks+S-1 are outstanding
      MOE_WAIT_VMCNT((kV2Stages - 2) * kV2CopiesPerThread);
      __syncthreads();
      read_frags((ks + 1) % kV2Stages, 0, af0, bf0);
      const int ksrc = min(ks + kV2Stages, nk - 1);
      const int slot = ks % kV2Stages;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        issue_part_to(ksrc, slot, i);
        if (i < nsub) {
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2)
            acc[i][j2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j2], acc[i][j2], 0, 0, 0);
        }
      }
      issue_part_to(ksrc, slot, 4);
    }
    // last slice (peeled, so the loop body has no branch around its LDS reads)
    read_frags((nk - 1) % kV2Stages, 1, af1, bf1);
    mfma_block(af0, bf0);
    mfma_block(af1, bf1);
    MOE_WAIT_VMCNT(0);  // no copy may land in the ring once it is reused below
    __syncthreads();

    // Epilogue through LDS: each wave converts its accumulators to bf16 into a private
    // [rows][cols + 8] staging tile, then stores whole 16-byte row chunks.  32x32
    // accumulator layout: element q of lane l is row (q/4)*8 + (l/32)*4 + q%4, column
    // l%32 of the 32x32 subtile.
    if constexpr (BWD) {
      // SwiGLU backward (op 2): per 32-row subtile, the wave's [32][32] block of dact is
      // copied to LDS (two 16-byte copies per lane; rows past the valid ones and columns
      // past N read row 0 / column 0, never stored), then dg and du come from one
      // sigmoid, are staged side by side and stored into C = [rows, 2N] (dg in columns
      // [0, N), du in [N, 2N)).
      constexpr int kLd = 32 + 8;
      bf16_t* so = reinterpret_cast<bf16_t*>(lds) + wave * 2 * 32 * kLd;
      unsigned char* sda = lds + kV2Threads / 64 * 2 * 32 * kLd * 2 + wave * 2048;
      const bf16_t* dbase = uniform_ptr(ops.D + (size_t)tile.m0 * N);
      const int dcol = n0 + wave * 32 + (lane & 3) * 8;
      const int dcc = dcol < N ? dcol : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i * 32 >= tile.valid) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = i * 32 + 16 * j + (lane >> 2);
          const int rr = r < tile.valid ? r : 0;
          copy16_to_lds(dbase, (uint32_t)(rr * N + dcc) * 2u, sda + j * 1024);
        }
        MOE_WAIT_VMCNT(0);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          const int c = lane & 31;
          const float da = bf16_to_f32(*reinterpret_cast<const bf16_t*>(sda + (r * 32 + c) * 2));
          const float gv = acc[i][0][q], uv = acc[i][1][q];
          const float sg = sigmoid_f32(gv);
          so[r * kLd + c] = f32_to_bf16(da * uv * (sg * (1.0f + gv * (1.0f - sg))));
          so[(32 + r) * kLd + c] = f32_to_bf16(da * gv * sg);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
          for (int r0 = 0; r0 < 32; r0 += 16) {
            const int r = r0 + (lane >> 2);
            const int grow = i * 32 + r;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(so + (ps * 32 + r) * kLd + (lane & 3) * 8);
            if (grow < tile.valid && dcol < N)
              *reinterpret_cast<u32x4_t*>(C + (size_t)(tile.m0 + grow) * 2 * N + ps * N + dcol) = v;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    } else {
    constexpr int kWCols = GU ? 32 : 64;   // output columns per wave
    constexpr int kHalves = GU ? 1 : 2;    // row passes
    constexpr int kRowsPer = 128 / kHalves;
    constexpr int kLd = kWCols + 8;                                 // staging row pitch
    bf16_t* stg = reinterpret_cast<bf16_t*>(lds) + wave * kRowsPer * kLd;
    const int col0 = n0 + (GU ? wave * 32 : (wave >> 2) * 256 + (wave & 3) * 64);
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i / (4 / kHalves) != hv) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = (i % (4 / kHalves)) * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          if (GU) {
            stg[r * kLd + (lane & 31)] = f32_to_bf16(silu_f32(acc[i][0][q]) * acc[i][1][q]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              stg[r * kLd + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][q]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int kChunks = kWCols / 8;           // 16-byte chunks per staged row
      constexpr int kRowsPerPass = 64 / kChunks;
#pragma unroll 4
      for (int r0 = 0; r0 < kRowsPer; r0 += kRowsPerPass) {
        const int r = r0 + lane / kChunks;
        const int ch = lane % kChunks;
        const int grow = hv * kRowsPer + r;
        const int gcol = col0 + ch * 8;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * kLd + ch * 8);
        if (grow < tile.valid && gcol < N)
          *reinterpret_cast<u32x4_t*>(C + (size_t)(tile.m0 + grow) * N + gcol) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    }
    __syncthreads();  // staging reads done before the next tile refills the ring
  }
}

// ---------------------------------------------------------------------------
// fp32 path: LDS-tiled FMA GEMM, 32 rows x 64 output columns per work group.
// ---------------------------------------------------------------------------
static constexpr int kFM = 32, kFN = 64, kFK = 16;

template <int OP>
__global__ void __launch_bounds__(256)
k_gg_f32(const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
         float* __restrict__ C, int K, int N, const int32_t* __restrict__ meta,
         const int32_t* __restrict__ num_blocks_ptr, int max_blocks, int E, int64_t max_rows,
         int dense_rows, int block_m, int n_tiles) {
  constexpr int NB = OP == MOE_OP_GATEUP_SWIGLU ? 2 : 1;
  __shared__ float As[kFK][kFM + 1];
  __shared__ float Bs[NB][kFK][kFN];
  const int tid = threadIdx.x;
  const int tpb = (block_m + kFM - 1) / kFM;
  const int nblocks =
      dense_rows > 0 ? (dense_rows + block_m - 1) / block_m : clamp_block_count(num_blocks_ptr, max_blocks);
  const int total = nblocks * tpb * n_tiles;
  const int ty = tid / 16, tx = tid % 16;  // rows ty*2 + {0,1}, cols tx*4 + {0..3}
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int nt = w % n_tiles;
    const int mt = w / n_tiles;
    Tile tile;
    if (!decode_block(mt / tpb, mt % tpb, kFM, block_m, meta, dense_rows, E, max_rows, tile)) continue;
    const int n0 = nt * kFN;
    const float* asrc = A + (size_t)tile.m0 * K;
    float acc[NB][2][4] = {};
    for (int k0 = 0; k0 < K; k0 += kFK) {
      __syncthreads();
      for (int i = tid; i < kFM * kFK; i += 256) {
        const int r = i / kFK, kk = i % kFK;
        As[kk][r] = (r < tile.valid && k0 + kk < K) ? asrc[(size_t)r * K + k0 + kk] : 0.f;
      }
      for (int i = tid; i < NB * kFK * kFN; i += 256) {
        const int nb = i / (kFK * kFN);
        const int rem = i % (kFK * kFN);
        const int kk = rem / kFN, c = rem % kFN;
        const float* bsrc = (nb ? B1 : B0) + (size_t)tile.e * K * N;
        Bs[nb][kk][c] = (k0 + kk < K && n0 + c < N) ? bsrc[(size_t)(k0 + kk) * N + n0 + c] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kFK; ++kk) {
        const float a0 = As[kk][ty * 2], a1 = As[kk][ty * 2 + 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float b = Bs[nb][kk][tx * 4 + c];
            acc[nb][0][c] = fmaf(a0, b, acc[nb][0][c]);
            acc[nb][1][c] = fmaf(a1, b, acc[nb][1][c]);
          }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = ty * 2 + r;
      if (row >= tile.valid) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = n0 + tx * 4 + c;
        if (col >= N) continue;
        const float v = OP == MOE_OP_GATEUP_SWIGLU ? silu_f32(acc[0][r][c]) * acc[NB - 1][r][c]
                                                   : acc[0][r][c];
        C[(size_t)(tile.m0 + row) * N + col] = v;
      }
    }
  }
}

// One segment set on the register-staged or fp32 kernels (dense_rows > 0: dense mode).
static moe_status launch_other(const moe_shape& s, int op, const void* A, const void* B0,
                               const void* B1, int K, int N, const int32_t* block_meta,
                               const int32_t* num_blocks, int32_t max_blocks, int32_t dense_rows,
                               void* C, hipStream_t st) {
  const int64_t blocks_ub =
      dense_rows > 0 ? ceil_div(dense_rows, s.block_m) : (int64_t)max_blocks;
  // rows of A and C: the dense operand has dense_rows rows, the permuted ones
  // max_blocks * block_m
  const int64_t max_rows = dense_rows > 0 ? (int64_t)dense_rows : routed_rows_bound(s, max_blocks);
  const int E = dense_rows > 0 ? 1 : s.E;
  const int cus = device_cu_count();
  if (s.dtype == MOE_DTYPE_BF16) {
    const int out_cols = op == MOE_OP_GATEUP_SWIGLU ? 128 : 256;
    const int n_tiles = (int)ceil_div(N, out_cols);
    int64_t items = blocks_ub * (s.block_m / kBM) * n_tiles;
    int64_t grid = items < cus ? items : cus;
    if (grid < 1) grid = 1;
    if (op == MOE_OP_GATEUP_SWIGLU)
      hipLaunchKernelGGL(k_gg_bf16<MOE_OP_GATEUP_SWIGLU>, dim3((unsigned)grid), dim3(kThreads), 0, st,
                         static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(B0),
                         static_cast<const bf16_t*>(B1), static_cast<bf16_t*>(C), K, N, block_meta,
                         num_blocks, max_blocks, E, max_rows, dense_rows, s.block_m, n_tiles);
    else
      hipLaunchKernelGGL(k_gg_bf16<MOE_OP_DOWN>, dim3((unsigned)grid), dim3(kThreads), 0, st,
                         static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(B0), nullptr,
                         static_cast<bf16_t*>(C), K, N, block_meta, num_blocks, max_blocks, E,
                         max_rows, dense_rows, s.block_m, n_tiles);
  } else {
    const int n_tiles = (int)ceil_div(N, kFN);
    int64_t items = blocks_ub * ceil_div(s.block_m, kFM) * n_tiles;
    int64_t grid = items < (int64_t)cus * 4 ? items : (int64_t)cus * 4;
    if (grid < 1) grid = 1;
    if (op == MOE_OP_GATEUP_SWIGLU)
      hipLaunchKernelGGL(k_gg_f32<MOE_OP_GATEUP_SWIGLU>, dim3((unsigned)grid), dim3(256), 0, st,
                         static_cast<const float*>(A), static_cast<const float*>(B0),
                         static_cast<const float*>(B1), static_cast<float*>(C), K, N, block_meta,
                         num_blocks, max_blocks, E, max_rows, dense_rows, s.block_m, n_tiles);
    else
      hipLaunchKernelGGL(k_gg_f32<MOE_OP_DOWN>, dim3((unsigned)grid), dim3(256), 0, st,
                         static_cast<const float*>(A), static_cast<const float*>(B0), nullptr,
                         static_cast<float*>(C), K, N, block_meta, num_blocks, max_blocks, E,
                         max_rows, dense_rows, s.block_m, n_tiles);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Wide tiles (384-row groups of one expert's blocks) pay off when experts own many
// 128-row blocks; with a few rows per expert (decode) the 128-row tiles stream the
// weights with less copy traffic per weight byte.
// MOE_GG_TILE_ROWS=128 or 384 forces one tile height where both apply (tests use it to
// cover both kernels on the same shapes); unset or anything else: automatic.
static bool use_wide_tiles(const moe_shape& s, const GemmSegments& g) {
  if (s.block_m != 128) return false;
  if (g.max_blocks > 0 && g.max_blocks > wide_max_blocks()) return false;
  const char* force = getenv("MOE_GG_TILE_ROWS");
  if (force && strcmp(force, "128") == 0) return false;
  if (force && strcmp(force, "384") == 0) return true;
  if (g.max_blocks > 0) {
    const int64_t M = (int64_t)s.T * s.k;
    return g.max_blocks <= wide_max_blocks() && M >= 256 * std::min<int64_t>(s.E, M);
  }
  return g.dense_rows >= 384;
}

bool gather_supported(const moe_shape& s) {
  // gathered rows are addressed with 32-bit byte offsets from the start of x
  return s.dtype == MOE_DTYPE_BF16 && s.d % kV2BK == 0 &&
         (int64_t)s.T * s.d * 2 + 4096 < ((int64_t)1 << 32);
}

moe_status launch_grouped_gemm(const moe_shape& s, int op, const GemmSegments& g, hipStream_t st) {
  const bool routed = g.max_blocks > 0;
  const bool dense = g.dense_rows > 0;
  if (!routed && !dense) return MOE_OK;
  const int cus = device_cu_count();
  const bool v2_routed = s.dtype == MOE_DTYPE_BF16 && g.K % kV2BK == 0;
  if (routed && g.gather && !v2_routed) return MOE_ENOTSUP;
  if (op == kOpGateUpBwd && ((routed && !v2_routed) ||
                             (dense && !(s.dtype == MOE_DTYPE_BF16 && g.Kd % kV2BK == 0))))
    return MOE_ENOTSUP;
  const bool v2_dense = s.dtype == MOE_DTYPE_BF16 && g.Kd % kV2BK == 0;
  // one launch when both sets fit the async-copy kernel with the same K and N
  if ((!routed || v2_routed) && (!dense || v2_dense) && (!routed || !dense || (g.K == g.Kd && g.N == g.Nd))) {
    const int K = routed ? g.K : g.Kd, N = routed ? g.N : g.Nd;
    if (use_wide_tiles(s, g)) {
      const GGOperands ro{static_cast<const bf16_t*>(g.A), static_cast<const bf16_t*>(g.B0),
                          static_cast<const bf16_t*>(g.B1), static_cast<bf16_t*>(g.C),
                          g.gather, g.gather_div, g.gather_rows, static_cast<const bf16_t*>(g.D)};
      const GGOperands dn{static_cast<const bf16_t*>(g.Ad), static_cast<const bf16_t*>(g.B0d),
                          static_cast<const bf16_t*>(g.B1d), static_cast<bf16_t*>(g.Cd), nullptr, 1, 1,
                          static_cast<const bf16_t*>(g.Dd)};
      return launch_gg_wide(op, ro, dn, K, N, g.block_meta, g.num_blocks, routed ? g.max_blocks : 0,
                            routed_rows_bound(s, routed ? g.max_blocks : 0), s.E,
                            dense ? g.dense_rows : 0, st);
    }
    const int out_cols = op == MOE_OP_DOWN ? 512 : 256;   // the kernel's kOutCols
    const int n_tiles = (int)ceil_div(N, out_cols);
    const int64_t blocks_ub = (routed ? (int64_t)g.max_blocks : 0) +
                              (dense ? ceil_div(g.dense_rows, s.block_m) : 0);
    int64_t items = blocks_ub * (s.block_m / kBM) * n_tiles;
    int64_t grid = items < cus ? items : cus;
    if (grid < 1) grid = 1;
    const GGOperands ro{static_cast<const bf16_t*>(g.A), static_cast<const bf16_t*>(g.B0),
                        static_cast<const bf16_t*>(g.B1), static_cast<bf16_t*>(g.C),
                        g.gather, g.gather_div, g.gather_rows, static_cast<const bf16_t*>(g.D)};
    const GGOperands dn{static_cast<const bf16_t*>(g.Ad), static_cast<const bf16_t*>(g.B0d),
                        static_cast<const bf16_t*>(g.B1d), static_cast<bf16_t*>(g.Cd), nullptr, 1, 1,
                        static_cast<const bf16_t*>(g.Dd)};
    const int64_t max_rows = routed_rows_bound(s, g.max_blocks);
    if (op == MOE_OP_GATEUP_SWIGLU)
      hipLaunchKernelGGL(k_gg_bf16_v2<MOE_OP_GATEUP_SWIGLU>, dim3((unsigned)grid), dim3(kV2Threads), 0,
                         st, ro, dn, K, N, g.block_meta, g.num_blocks, g.max_blocks, s.E, max_rows,
                         g.dense_rows, s.block_m, n_tiles);
    else if (op == kOpGateUpBwd)
      hipLaunchKernelGGL(k_gg_bf16_v2<kOpGateUpBwd>, dim3((unsigned)grid), dim3(kV2Threads), 0,
                         st, ro, dn, K, N, g.block_meta, g.num_blocks, g.max_blocks, s.E, max_rows,
                         g.dense_rows, s.block_m, n_tiles);
    else
      hipLaunchKernelGGL(k_gg_bf16_v2<MOE_OP_DOWN>, dim3((unsigned)grid), dim3(kV2Threads), 0, st,
                         ro, dn, K, N, g.block_meta, g.num_blocks, g.max_blocks, s.E, max_rows,
                         g.dense_rows, s.block_m, n_tiles);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  // otherwise each set on its own launch
  moe_status st2 = MOE_OK;
  if (dense) {
    if (v2_dense) {
      GemmSegments d = g;
      d.max_blocks = 0;  // dense set alone: takes the single-launch path above
      st2 = launch_grouped_gemm(s, op, d, st);
    } else {
      st2 = launch_other(s, op, g.Ad, g.B0d, g.B1d, g.Kd, g.Nd, nullptr, nullptr, 0, g.dense_rows,
                         g.Cd, st);
    }
  }
  if (st2 != MOE_OK) return st2;
  if (routed) {
    if (v2_routed) {
      GemmSegments r = g;
      r.dense_rows = 0;
      st2 = launch_grouped_gemm(s, op, r, st);
    } else {
      st2 = launch_other(s, op, g.A, g.B0, g.B1, g.K, g.N, g.block_meta, g.num_blocks,
                         g.max_blocks, 0, g.C, st);
    }
  }
  return st2;
}

}  // namespace moe
