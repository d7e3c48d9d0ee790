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
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

static constexpr int kBM = 128;     // rows per tile
static constexpr int kBK = 64;      // K per pipeline stage
static constexpr int kBNB = 256;    // B columns per tile
static constexpr int kThreads = 256;
static constexpr int kALdsBytes = kBM * kBK * 2;        // 16 KB
static constexpr int kBLdsBytes = kBNB * kBK * 2;       // 32 KB
static constexpr int kStageBytes = kALdsBytes + kBLdsBytes;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

struct Tile {
  int e, m0, valid;
};

// Work-item decoding shared by both kernels: returns false if the item is empty.
__device__ __forceinline__ bool decode_block(int b, int sub, int sub_rows, int block_m,
                                             const int32_t* __restrict__ meta, int dense_rows,
                                             int E, int64_t max_rows, Tile& t) {
  int e, m_start, vm;
  if (dense_rows > 0) {
    e = 0;
    m_start = b * block_m;
    vm = min(block_m, dense_rows - m_start);
  } else {
    e = meta[3 * b + 0];
    m_start = meta[3 * b + 1];
    vm = meta[3 * b + 2];
  }
  t.e = e;
  t.m0 = m_start + sub * sub_rows;
  t.valid = min(sub_rows, vm - sub * sub_rows);
  // a table entry that does not fit the expert range or the row buffers is skipped
  if (e < 0 || e >= E || m_start < 0 || vm > block_m || (int64_t)m_start + vm > max_rows)
    return false;
  return t.valid > 0;
}

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
      dense_rows > 0 ? (dense_rows + block_m - 1) / block_m : min(num_blocks_ptr[0], max_blocks);
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
      dense_rows > 0 ? (dense_rows + block_m - 1) / block_m : min(num_blocks_ptr[0], max_blocks);
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

moe_status launch_grouped_gemm(const moe_shape& s, int op, const void* A, const void* B0,
                               const void* B1, int K, int N, const int32_t* block_meta,
                               const int32_t* num_blocks, int32_t max_blocks, int32_t dense_rows,
                               void* C, hipStream_t st) {
  const int64_t blocks_ub =
      dense_rows > 0 ? ceil_div(dense_rows, s.block_m) : (int64_t)max_blocks;
  // rows of A and C: the dense operand has dense_rows rows, the permuted ones
  // max_blocks * block_m
  const int64_t max_rows = dense_rows > 0 ? (int64_t)dense_rows : (int64_t)max_blocks * s.block_m;
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

}  // namespace moe
