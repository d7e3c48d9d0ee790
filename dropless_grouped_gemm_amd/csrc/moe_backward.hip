// Backward pass of the dropless MoE layer (dropless notes: the gradients of grouped
// GEMMs are grouped GEMMs over the same segments - data gradients through the
// transposed weights, weight gradients reducing over each expert's rows - and the
// permutation is replayed from the saved indices).  The chain rule step by step:
//   combine   dy[pos[t,j]] = w[t,j] dout[t];  dw[t,j] = <dout[t], y[pos[t,j]]>
//   down      dact = dy W2[e]^T                     (k_gg_nt, data gradient)
//             dW2[e] = act_e^T dy_e                   (k_gg_wgrad)
//   SwiGLU    gate/up recomputed, dg | du = SwiGLU'  (the forward kernels, op 2)
//   gate/up   dx_perm = dg W1[e]^T + du W3[e]^T      (k_gg_nt over K = 2 d_e)
//             dW1[e] | dW3[e] = x_perm_e^T (dg | du)  (k_gg_wgrad)
//   permute   dx[t] = sum_j dx_perm[pos[t,j]]        (the combine kernel, unit weights)
//   router    dlogits through the softmax (and renormalisation), selection fixed
//             (k_router_bwd); dW_g = x^T dlogits, dbias = sum_t dlogits
//             (k_router_wgrad); dx += dlogits W_g^T (k_router_dx_v8, k_router_dx)
//
// The GEMM kernels keep the 128-row kernel's structure (8 waves, 128 x 512 tiles,
// four 40 KB ring slots of 32-deep slices filled by 16-byte global->LDS copies, fp32
// accumulators of v_mfma_f32_32x32x16_bf16):
//   * k_gg_nt: B is read transposed, i.e. the weight is stored [N][K] with K contiguous
//     (W2[e] as [d_e][d]; W1[e], W3[e] as [d][d_e]), so B slices are staged exactly like
//     A slices ([n][32 k], 64 bytes per row, chunk swizzle c ^ ((n >> 2) & 3)) and read
//     with ds_read_b128.  The contraction may switch matrices at ksplit (dg | du against
//     W1 | W3).
//   * k_gg_wgrad: C[e] = X_e^T D_e, reducing over the expert's rows: both operands are
//     row-major slices [32 rows][cols] in LDS, read with ds_read_b64_tr_b16 (X as the A
//     operand, D as B).  Rows past the expert's count copy its first row and are zeroed
//     in LDS by the wave that copied them once its copies have landed.  fp32 output;
//     experts without rows get zeros.
// No floating-point atomics: every output element has one writer and a fixed summation
// order.  The one atomic is an integer work-queue counter in k_gg_wgrad, which only
// decides which work group takes which item, so results do not depend on scheduling.
#include "moe_gemm_common.h"

namespace moe {

// ---------------------------------------------------------------------------
// combine backward
// ---------------------------------------------------------------------------
static constexpr int kCbWaves = 8;    // kCbSplit waves per token
static constexpr int kCbSplit = 4;
static constexpr int kCbVec = 4;      // 16-byte vectors per lane per wave (rows up to 8192 bf16)
static constexpr int kCbMaxK = 1024;

// kCbSplit waves per token, wave q of them over vectors [256 q, 256 q + 256) of the row.
// dout's part stays packed (bf16 pairs widen exactly to fp32 on use); the token's k rows
// of y stream through two register buffers, row j+1's loads in flight while row j is
// used.  Each wave's dot is a fixed-order lane sum of its fma chain; dw is the sum of
// the parts in wave order, through LDS: the same sums on every run.
__global__ void __launch_bounds__(64 * kCbWaves)
k_combine_bwd(const u32x4_t* __restrict__ dout, const u32x4_t* __restrict__ y,
              const int32_t* __restrict__ pos, const float* __restrict__ w, int T, int k,
              int nvec, int64_t max_rows, u32x4_t* __restrict__ dy, float* __restrict__ dw) {
  __shared__ float s_part[kCbWaves][kCbMaxK];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok = wave / kCbSplit, part = wave % kCbSplit;
  constexpr int kTok = kCbWaves / kCbSplit;      // tokens per block and iteration
  const int v0 = part * kCbVec * 64 + lane;      // this lane's first vector
  for (int tb = blockIdx.x * kTok; tb < T; tb += gridDim.x * kTok) {
    const int t = tb + tok;
    if (t < T) {
      u32x4_t gv[kCbVec];
#pragma unroll
      for (int i = 0; i < kCbVec; ++i) {
        const int v = v0 + 64 * i;
        gv[i] = v < nvec ? dout[(size_t)t * nvec + v] : u32x4_t{0u, 0u, 0u, 0u};
      }
      auto load_row = [&](int j, u32x4_t* yv) {
        const int p = pos[(size_t)t * k + j];
        const bool ok = p >= 0 && p < max_rows;
#pragma unroll
        for (int i = 0; i < kCbVec; ++i) {
          const int v = v0 + 64 * i;
          yv[i] = (ok && v < nvec) ? y[(size_t)p * nvec + v] : u32x4_t{0u, 0u, 0u, 0u};
        }
      };
      auto use_row = [&](int j, const u32x4_t* yv) {
        const int p = pos[(size_t)t * k + j];
        const bool ok = p >= 0 && p < max_rows;
        if (p < -1 || p >= max_rows) MOE_DEBUG_REPORT(MOE_DBG_POSITION);
        const float wj = w[(size_t)t * k + j];
        float dot = 0.f;
        if (ok) {
#pragma unroll
          for (int i = 0; i < kCbVec; ++i) {
            const int v = v0 + 64 * i;
            if (v >= nvec) continue;
            u32x4_t o;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const float g0 = __uint_as_float(gv[i][h] << 16);
              const float g1 = __uint_as_float(gv[i][h] & 0xffff0000u);
              dot = fmaf(g0, __uint_as_float(yv[i][h] << 16), dot);
              dot = fmaf(g1, __uint_as_float(yv[i][h] & 0xffff0000u), dot);
              o[h] = pack_bf16x2(wj * g0, wj * g1);
            }
            dy[(size_t)p * nvec + v] = o;
          }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
        if (lane == 0) s_part[wave][j] = dot;
      };
      u32x4_t ya[kCbVec], yb[kCbVec];
      load_row(0, ya);
      for (int j = 0; j < k; j += 2) {
        if (j + 1 < k) load_row(j + 1, yb);
        use_row(j, ya);
        if (j + 1 < k) {
          if (j + 2 < k) load_row(j + 2, ya);
          use_row(j + 1, yb);
        }
      }
    }
    __syncthreads();
    if (t < T && part == 0) {
      for (int j = lane; j < k; j += 64) {
        float sum = s_part[wave][j];
#pragma unroll
        for (int q = 1; q < kCbSplit; ++q) sum += s_part[wave + q][j];
        dw[(size_t)t * k + j] = sum;
      }
    }
    __syncthreads();   // partials read before the next tokens overwrite them
  }
}

moe_status launch_combine_bwd(const moe_shape& s, const void* dout, const void* y,
                              const int32_t* pos, const float* topk_w, void* dy, float* dw,
                              int64_t max_rows, hipStream_t st) {
  const int nvec = (int)((int64_t)s.d * 2 / 16);
  if (nvec > kCbSplit * 64 * kCbVec || s.k > kCbMaxK) return MOE_ENOTSUP;
  int64_t blocks = ceil_div(s.T, kCbWaves / kCbSplit);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_combine_bwd, dim3((unsigned)blocks), dim3(64 * kCbWaves), 0, st,
                     static_cast<const u32x4_t*>(dout), static_cast<const u32x4_t*>(y), pos, topk_w,
                     s.T, s.k, nvec, max_rows, static_cast<u32x4_t*>(dy), dw);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// data-gradient grouped GEMM with transposed B
// ---------------------------------------------------------------------------
static constexpr int kBThreads = 512;
static constexpr int kBBK = 32;
static constexpr int kBABytes = 128 * kBBK * 2;      // 8 KB of A
static constexpr int kBBBytes = 512 * kBBK * 2;      // 32 KB of B
static constexpr int kBStage = kBABytes + kBBBytes;  // 40 KB
static constexpr int kBStages = 4;
static constexpr int kBCopies = 1 + 4;

struct NTOperands {
  const bf16_t* A;     // [rows, K]
  const bf16_t* Bt0;   // per expert [N][ldb]: B[k][n] = Bt0[n][k] for k < ksplit
  const bf16_t* Bt1;   // ... = Bt1[n][k - ksplit] for k >= ksplit (NULL: unused)
  bf16_t* C;           // [rows, N]
  int ldb, ksplit;
};

__global__ void __launch_bounds__(kBThreads, 1)
k_gg_nt(NTOperands ops, int K, int N, const int32_t* __restrict__ meta,
        const int32_t* __restrict__ num_blocks_ptr, int max_blocks, int E, int64_t max_rows,
        int dense_rows, int block_m, int n_tiles) {
  __shared__ __align__(1024) unsigned char lds[kBStages * kBStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // items: (block, 128-row sub-tile, 512-column tile); a dense set uses 128-row blocks
  const int bm = dense_rows > 0 ? 128 : block_m;
  const int nsub = bm / 128;
  const int nblocks = dense_rows > 0 ? (dense_rows + 127) / 128 : clamp_block_count(num_blocks_ptr, max_blocks);
  const int total = nblocks * nsub * n_tiles;
  const int nk = K / kBBK;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int nt = w % n_tiles;
    const int sub = (w / n_tiles) % nsub;
    const int blk = w / (n_tiles * nsub);
    Tile tile;
    if (!decode_block(blk, sub, 128, bm, meta, dense_rows, E, max_rows, tile)) continue;
    const int n0 = nt * 512;
    const bf16_t* asrc = uniform_ptr(ops.A + (size_t)tile.m0 * K);
    const bf16_t* bt0 = uniform_ptr(ops.Bt0 + (size_t)tile.e * N * ops.ldb);
    const bf16_t* bt1 = uniform_ptr(ops.Bt1 ? ops.Bt1 + (size_t)tile.e * N * ops.ldb : bt0);
    // the logical chunk of lane l in every 16-row window: (l & 3) ^ ((l >> 4) & 3)
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t a_voff;
    {
      const int row = wave * 16 + (lane >> 2);
      const int rr = row < tile.valid ? row : 0;
      a_voff = (uint32_t)(rr * K + c * 8) * 2u;
    }
    uint32_t b_voff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int n = n0 + (wave * 4 + p) * 16 + (lane >> 2);
      const int nn = n < N ? n : 0;        // columns past N copy column 0
      b_voff[p] = (uint32_t)(nn * ops.ldb + c * 8) * 2u;
    }
    auto issue_part_to = [&](int ks, int slot, int part) {
      unsigned char* st = lds + slot * kBStage;
      const int k0 = ks * kBBK;
      if (part == 0) {
        copy16_to_lds(asrc + k0, a_voff, st + wave * 1024);
      } else {
        const bool second = k0 >= ops.ksplit;
        const bf16_t* base = (second ? bt1 : bt0) + (second ? k0 - ops.ksplit : k0);
        copy16_to_lds(base, b_voff[part - 1], st + kBABytes + (wave * 4 + part - 1) * 1024);
      }
    };
    auto issue = [&](int ks, int slot) {
#pragma unroll
      for (int part = 0; part < kBCopies; ++part) issue_part_to(ks, slot, part);
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    bf16x8_t af0[4], bf0[2], af1[4], bf1[2];
    auto read_frags = [&](int stage, int kk, bf16x8_t* a, bf16x8_t* b) {
      const unsigned char* sa = lds + stage * kBStage;
      const unsigned char* sb = sa + kBABytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8_t*>(sa + row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wave * 64 + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8_t*>(sb + n * 64 + swz_a(n, kk * 2 + (lane >> 5)) * 16);
      }
    };
    auto mfma_block = [&](const bf16x8_t* a, const bf16x8_t* b) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    };

    // The 128-row kernel's pipeline: every slot in flight, the barrier between the two
    // 16-deep halves of a slice, the consumed slot refilled between the second half's
    // MFMAs, constant waits (slots past the last slice take copies of it, never read).
#pragma unroll
    for (int p = 0; p < kBStages; ++p) issue(min(p, nk - 1), p);
    MOE_WAIT_VMCNT((kBStages - 1) * kBCopies);
    __syncthreads();
    read_frags(0, 0, af0, bf0);
    for (int ks = 0; ks < nk - 1; ++ks) {
      read_frags(ks % kBStages, 1, af1, bf1);
      mfma_block(af0, bf0);
      MOE_WAIT_VMCNT((kBStages - 2) * kBCopies);
      __syncthreads();
      read_frags((ks + 1) % kBStages, 0, af0, bf0);
      const int ksrc = min(ks + kBStages, nk - 1);
      const int slot = ks % kBStages;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        issue_part_to(ksrc, slot, i);
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2)
          acc[i][j2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j2], acc[i][j2], 0, 0, 0);
      }
      issue_part_to(ksrc, slot, 4);
    }
    read_frags((nk - 1) % kBStages, 1, af1, bf1);
    mfma_block(af0, bf0);
    mfma_block(af1, bf1);
    MOE_WAIT_VMCNT(0);
    __syncthreads();

    // Epilogue: bf16 staging per wave ([64 rows][64 + 8], two row passes), 16-byte stores.
    constexpr int kLd = 64 + 8;
    bf16_t* stg = reinterpret_cast<bf16_t*>(lds) + wave * 64 * kLd;
    const int col0 = n0 + wave * 64;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i / 2 != hv) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = (i % 2) * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
#pragma unroll
          for (int j = 0; j < 2; ++j) stg[r * kLd + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][q]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 4
      for (int r0 = 0; r0 < 64; r0 += 8) {
        const int r = r0 + (lane >> 3);
        const int c8 = lane & 7;
        const int grow = hv * 64 + r;
        const int gcol = col0 + c8 * 8;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * kLd + c8 * 8);
        if (grow < tile.valid && gcol < N)
          *reinterpret_cast<u32x4_t*>(ops.C + (size_t)(tile.m0 + grow) * N + gcol) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
  }
}

moe_status launch_gg_nt(const void* A, const void* Bt0, const void* Bt1, int ldb, int ksplit,
                        void* C, int K, int N, const int32_t* meta, const int32_t* num_blocks,
                        int32_t max_blocks, int E, int block_m, int64_t max_rows,
                        int32_t dense_rows, hipStream_t st) {
  const int n_tiles = (int)ceil_div(N, 512);
  const int64_t blocks_ub = dense_rows > 0 ? ceil_div(dense_rows, 128)
                                           : (int64_t)max_blocks * (block_m / 128);
  const int64_t items = blocks_ub * n_tiles;
  const int cus = device_cu_count();
  int64_t grid = items < cus ? items : cus;
  if (grid < 1) grid = 1;
  const NTOperands ops{static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(Bt0),
                       static_cast<const bf16_t*>(Bt1), static_cast<bf16_t*>(C), ldb,
                       Bt1 ? ksplit : K};
  if (dense_rows > 0) max_rows = dense_rows;
  hipLaunchKernelGGL(k_gg_nt, dim3((unsigned)grid), dim3(kBThreads), 0, st, ops, K, N, meta,
                     num_blocks, max_blocks, dense_rows > 0 ? 1 : E, max_rows, dense_rows, block_m,
                     n_tiles);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// weight transpose: wt[e][c][r] = w[e][r][c]
// ---------------------------------------------------------------------------
// With the weights transposed once, a data gradient C = A B^T is the plain product
// C = A (B^T) that the forward grouped-GEMM kernels compute.  64 x 64 tiles through LDS:
// 16-byte row loads, then each thread gathers 8 consecutive r of one column c from LDS
// and stores them as one 16-byte chunk of wt's row c.
static constexpr int kTrTile = 64;

__global__ void __launch_bounds__(256)
k_transpose_bf16(const bf16_t* __restrict__ w, int R, int C, bf16_t* __restrict__ wt,
                 int64_t wt_estride, int wt_ld) {
  __shared__ bf16_t tile[kTrTile][kTrTile + 2];
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * kTrTile, c0 = blockIdx.x * kTrTile;
  const bf16_t* src = w + (size_t)e * R * C;
  bf16_t* dst = wt + (size_t)e * wt_estride;
  // load: 64 rows x 8 chunks of 8 columns, two per thread
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + h * 256;
    const int rr = i >> 3, cc = (i & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4_t*>(src + (size_t)r * C + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[rr][cc + 2 * q] = (bf16_t)(v[q] & 0xffffu);
      tile[rr][cc + 2 * q + 1] = (bf16_t)(v[q] >> 16);
    }
  }
  __syncthreads();
  // store: 64 columns x 8 chunks of 8 rows, two per thread
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + h * 256;
    const int cc = i >> 3, rr = (i & 7) * 8;
    const int c = c0 + cc, r = r0 + rr;
    if (c < C && r < R) {
      u32x4_t v;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = (uint32_t)tile[rr + 2 * q][cc] | ((uint32_t)tile[rr + 2 * q + 1][cc] << 16);
      *reinterpret_cast<u32x4_t*>(dst + (size_t)c * wt_ld + r) = v;
    }
  }
}

moe_status launch_transpose_bf16(int E, int R, int C, const void* w, void* wt, int64_t wt_estride,
                                 int wt_ld, hipStream_t st) {
  if (E <= 0 || R <= 0 || C <= 0) return MOE_OK;
  hipLaunchKernelGGL(k_transpose_bf16,
                     dim3((unsigned)ceil_div(C, kTrTile), (unsigned)ceil_div(R, kTrTile), (unsigned)E),
                     dim3(256), 0, st, static_cast<const bf16_t*>(w), R, C, static_cast<bf16_t*>(wt),
                     wt_estride, wt_ld);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// weight-gradient grouped GEMM: C[e] = X_e^T D_e over each expert's rows
// ---------------------------------------------------------------------------
static constexpr int kWgXBytes = kBBK * 128 * 2;     // [32 rows][128 m] = 8 KB
static constexpr int kWgDBytes = kBBK * 512 * 2;     // [32 rows][512 n] = 32 KB
static constexpr int kWgStage = kWgXBytes + kWgDBytes;

struct WgOperands {
  const bf16_t* X;     // [rows, Km]
  const bf16_t* D;     // [rows, Nn]
  float* C0;           // per expert [Km][nsplit]      (columns n < nsplit)
  float* C1;           // per expert [Km][Nn - nsplit] (columns n >= nsplit; NULL: none)
  int nsplit;
};

// Largest expert first: order[r] is the expert of rank r by row count (ties: lower id),
// and the work queue counter starts at zero.  One block; counts staged in LDS.
__global__ void __launch_bounds__(256)
k_wgrad_order(const int32_t* __restrict__ counts, int E, int32_t* __restrict__ order,
              int32_t* __restrict__ queue) {
  __shared__ int32_t s_cnt[1024];
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = counts[e];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const int c = s_cnt[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (s_cnt[f] > c) || (s_cnt[f] == c && f < e);
    order[rank] = e;
  }
  if (threadIdx.x == 0) *queue = 0;
}

// Items (expert, m tile, n tile).  Without a queue, work group b takes items b, b + grid,
// ...  in expert order.  With one, items are numbered largest expert first (order[]) and
// each work group takes the next number from the queue counter when it starts an item:
// the longest items go first and the short ones fill in behind them, so experts of
// unequal size do not leave work groups idle at the end.  Which work group computes an
// item does not change its result.
__global__ void __launch_bounds__(kBThreads, 1)
k_gg_wgrad(WgOperands ops, int Km, int Nn, const int32_t* __restrict__ counts,
           const int32_t* __restrict__ row_off, int E, int dense_rows, int m_tiles, int n_tiles,
           int32_t* __restrict__ queue, const int32_t* __restrict__ order) {
  __shared__ __align__(1024) unsigned char lds[kBStages * kWgStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, gi = lane & 15, tr_r = gi >> 2, tr_c4 = gi & 3;
  const int total = E * m_tiles * n_tiles;
  // the next item number, handed to every wave through the (idle) first LDS word
  auto take_next = [&](int v) {
    __syncthreads();
    if (tid == 0) *reinterpret_cast<int*>(lds) = v;
    __syncthreads();
    const int r = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(lds));
    __syncthreads();   // read by all before the next item's copies land there
    return r;
  };
  int w = blockIdx.x;
  if (queue) w = take_next(tid == 0 ? atomicAdd(queue, 1) : 0);
  while (w < total) {
    int nxt = 0;
    if (queue && tid == 0) nxt = atomicAdd(queue, 1);   // fetched while this item runs
    const int nt = w % n_tiles;
    const int mt = (w / n_tiles) % m_tiles;
    const int e = queue ? order[w / (n_tiles * m_tiles)] : w / (n_tiles * m_tiles);
    const int cnt = __builtin_amdgcn_readfirstlane(dense_rows > 0 ? dense_rows : (counts ? counts[e] : 0));
    const int r0e = __builtin_amdgcn_readfirstlane(dense_rows > 0 || !counts ? 0 : row_off[e]);
    const int m0 = mt * 128, n0 = nt * 512;
    const int ns = (cnt + kBBK - 1) / kBBK;   // 32-row slices of this expert
    // Copies: wave w owns slice rows 4w .. 4w+3: one X copy (4 rows x 256 B, 16 lanes
    // per row) and four D copies (one 1 KB row each).  A lane's 16 bytes land at
    // physical chunk (lane & 15) of its X row / lane of its D row, which holds logical
    // chunk swz_b(row, physical) (the swizzle is an involution).  Rows past the count
    // read the expert's first row (in bounds) and are zeroed in LDS afterwards.
    int mcol, ncol[4];
    {
      const int rr = 4 * wave + (lane >> 4);
      mcol = m0 + swz_b(rr, lane & 15) * 8;
      if (mcol >= Km) mcol = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        ncol[p] = n0 + swz_b(4 * wave + p, lane) * 8;
        if (ncol[p] >= Nn) ncol[p] = 0;
      }
    }
    const bf16_t* xe = uniform_ptr(ops.X + (size_t)r0e * Km);
    const bf16_t* de = uniform_ptr(ops.D + (size_t)r0e * Nn);
    auto issue = [&](int s, int slot) {
      unsigned char* st = lds + slot * kWgStage;
      const int rbase = 32 * s + 4 * wave;
      const int xb = rbase < cnt ? rbase : 0;
      const int lr = rbase + (lane >> 4) < cnt ? (lane >> 4) : 0;
      copy16_to_lds(xe + (size_t)xb * Km, (uint32_t)(lr * Km + mcol) * 2u, st + wave * 1024);
      if (rbase + 4 <= cnt) {
        // the four D rows as one group behind one M0 load: copy p lands at +1 KB p (the
        // instruction's immediate moves both addresses), its global row is corrected
        // through the lane offset against a base 3 KB below row rbase
        set_lds_dma_base(st + kWgXBytes + 4 * wave * 1024);
        const unsigned char* db = reinterpret_cast<const unsigned char*>(de + (size_t)rbase * Nn) - 3 * 1024;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          copy16_to_lds_nth(p, db, (uint32_t)(p * Nn + ncol[p]) * 2u + (uint32_t)(3 - p) * 1024u);
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = rbase + p;
          const int rr = r < cnt ? r : 0;
          copy16_to_lds(de + (size_t)rr * Nn, (uint32_t)ncol[p] * 2u,
                        st + kWgXBytes + (4 * wave + p) * 1024);
        }
      }
    };
    // zero this wave's rows of slice s that lie past the count (after its copies landed)
    auto zero_tail = [&](int s) {
      const int rbase = 32 * s + 4 * wave;
      if (rbase + 4 <= cnt) return;
      unsigned char* st = lds + (s % kBStages) * kWgStage;
      const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
      if (rbase + (lane >> 4) >= cnt) *reinterpret_cast<u32x4_t*>(st + wave * 1024 + lane * 16) = z;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (rbase + p >= cnt)
          *reinterpret_cast<u32x4_t*>(st + kWgXBytes + (4 * wave + p) * 1024 + lane * 16) = z;
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // transposed 4 x 16 reads: A (X^T) subtile i reads columns m = 32 i + ..., B (D)
    // subtile j columns n = 64 wave + 32 j + ...
    bf16x8_t af[4], bf[2];
    auto read_frags = [&](int s, int kk) {
      const unsigned char* sx = lds + (s % kBStages) * kWgStage;
      const unsigned char* sd = sx + kWgXBytes;
      const int kbase = kk * 16 + (g >> 1) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = i * 32 + (g & 1) * 16 + 4 * tr_c4;
        i16x4_t hv[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = kbase + hh * 4 + tr_r;
          hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MOE_LDS i16x4_t*)(sx + k * 256 + swz_b(k, col >> 3) * 16 + (col & 7) * 2));
        }
        af[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wave * 64 + j * 32 + (g & 1) * 16 + 4 * tr_c4;
        i16x4_t hv[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = kbase + hh * 4 + tr_r;
          hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MOE_LDS i16x4_t*)(sd + k * 1024 + swz_b(k, col >> 3) * 16 + (col & 7) * 2));
        }
        bf[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };

    if (ns > 0) {
      // every slot in flight (slots past the last slice take copies of it that are
      // never read: they must not land in the slot that slice really uses, which is
      // zeroed past the count), then slice 0
#pragma unroll
      for (int p = 0; p < kBStages; ++p) issue(min(p, ns - 1), p);
      MOE_WAIT_VMCNT((kBStages - 1) * kBCopies);
      zero_tail(0);
      __syncthreads();
      for (int s = 0; s < ns; ++s) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          read_frags(s, kk);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < ns) {
          // slot s % S is free once every wave is past this barrier; slice s+1 must land
          MOE_WAIT_VMCNT((kBStages - 2) * kBCopies);
          zero_tail(s + 1);
          __syncthreads();
          issue(min(s + kBStages, ns - 1), s % kBStages);
        }
      }
      MOE_WAIT_VMCNT(0);
      __syncthreads();
    }

    // fp32 stores straight from the accumulators (32 lanes write 128 contiguous bytes)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = m0 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          const int n = n0 + wave * 64 + j * 32 + (lane & 31);
          if (m >= Km || n >= Nn) continue;
          if (n < ops.nsplit)
            ops.C0[((size_t)e * Km + m) * ops.nsplit + n] = acc[i][j][q];
          else
            ops.C1[((size_t)e * Km + m) * (Nn - ops.nsplit) + (n - ops.nsplit)] = acc[i][j][q];
        }
    w = queue ? take_next(nxt) : w + (int)gridDim.x;
  }
}

size_t wgrad_sched_bytes(int E) { return (size_t)(E + 64) * 4; }

moe_status launch_gg_wgrad(const void* X, const void* D, float* C0, float* C1, int nsplit, int Km,
                           int Nn, const int32_t* counts, const int32_t* row_off, int E,
                           int32_t dense_rows, void* sched, hipStream_t st) {
  const int m_tiles = (int)ceil_div(Km, 128), n_tiles = (int)ceil_div(Nn, 512);
  const int64_t items = (int64_t)E * m_tiles * n_tiles;
  const int cus = device_cu_count();
  int64_t grid = items < cus ? items : cus;
  if (grid < 1) grid = 1;
  const WgOperands ops{static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(D), C0, C1,
                       C1 ? nsplit : Nn};
  // the work queue applies to the routed experts (counts given) when scratch is given:
  // [0, 64) the counter (its own 256-byte line), then order[E]
  int32_t* queue = nullptr;
  int32_t* order = nullptr;
  if (sched && counts && dense_rows == 0 && E > 1 && E <= 1024) {
    queue = static_cast<int32_t*>(sched);
    order = queue + 64;
    hipLaunchKernelGGL(k_wgrad_order, dim3(1), dim3(256), 0, st, counts, E, order, queue);
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  hipLaunchKernelGGL(k_gg_wgrad, dim3((unsigned)grid), dim3(kBThreads), 0, st, ops, Km, Nn,
                     counts, row_off, E, dense_rows, m_tiles, n_tiles, queue, order);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// router backward
// ---------------------------------------------------------------------------
// dlogits[t, :] from dw[t, :]: p = softmax(logits[t]) in fp32; the selected experts'
// probabilities ps_j (renormalised: w_j = ps_j / Z, dps_j = (dw_j - <dw, w>) / Z;
// otherwise dps = dw); dp[e] = sum of dps_j over the slots choosing e (ascending j);
// dlogits[e] = p[e] (dp[e] - <dp, p>).  One wave per token, experts strided over
// lanes, fixed-order reductions.
static constexpr int kRbMaxPerLane = 16;   // E <= 1024

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// p[e] of expert e, held by lane e % 64 as element e / 64 (e wave-uniform): each lane
// selects its element e / 64 without indexing the register array, then lane e % 64's
// copy is broadcast.
__device__ __forceinline__ float expert_value(const float (&p)[kRbMaxPerLane], int e) {
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) v = (i == (e >> 6)) ? p[i] : v;
  return __shfl(v, e & 63, 64);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ void __launch_bounds__(256)
k_router_bwd(const float* __restrict__ logits, const int32_t* __restrict__ idx,
             const float* __restrict__ dw, int T, int E, int k, int renorm,
             float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lt = logits + (size_t)t * E;
  float p[kRbMaxPerLane];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? lt[e] : -INFINITY;
    mx = fmaxf(mx, p[i]);
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? expf(p[i] - mx) : 0.f;
    sum += p[i];
  }
  sum = wave_sum(sum);
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) p[i] /= sum;
  // selected probabilities and their gradient, slot by slot (lane j holds slot j)
  float Z = 0.f, dwdotw = 0.f;
  if (renorm) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      Z += expert_value(p, e);
    }
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      dwdotw += dw[(size_t)t * k + j] * (expert_value(p, e) / Z);
    }
  }
  float dp[kRbMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) dp[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    const float g = renorm ? (dw[(size_t)t * k + j] - dwdotw) / Z : dw[(size_t)t * k + j];
#pragma unroll
    for (int i = 0; i < kRbMaxPerLane; ++i)
      if (lane + 64 * i == e) dp[i] += g;
  }
  float dotp = 0.f;
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) dotp += dp[i] * p[i];
  dotp = wave_sum(dotp);
#pragma unroll
  for (int i = 0; i < kRbMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    if (e < E) dlogits[(size_t)t * E + e] = p[i] * (dp[i] - dotp);
  }
}

// dW_g = sum over the chunks in order (and dbias likewise; either output may be NULL).
__global__ void __launch_bounds__(256)
k_router_wgrad_reduce(const float* __restrict__ pw, const float* __restrict__ pb, int nchunks,
                      int64_t n, int E, float* __restrict__ dwg, float* __restrict__ dbias) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (dwg && i < n) {
    float v = 0.f;
#pragma unroll 8
    for (int z = 0; z < nchunks; ++z) v += pw[(size_t)z * n + i];
    dwg[i] = v;
  }
  if (dbias && i < E) {
    float v = 0.f;
    for (int z = 0; z < nchunks; ++z) v += pb[(size_t)z * E + i];
    dbias[i] = v;
  }
}

// dW_g[c, e] = sum_t x[t, c] dlogits[t, e]; dbias[e] = sum_t dlogits[t, e], for rows whose
// width is a multiple of 8 (16-byte aligned).  The tokens are cut into contiguous chunks of
// tchunk (blockIdx.z); a block owns 256 columns and 8 experts of one chunk, its 256 threads
// being 32 groups of 8 adjacent columns (one 16-byte load of x per token) x 8 token phases.
// A thread sums tokens t = begin + phase, + 8, ... in ascending order and the 8 phase sums
// are added in phase order through LDS.  Chunk z's sums go to ow + z * ow_stride ([d][E])
// and ob + z * ob_stride ([E]; ob NULL: not written); k_router_wgrad_reduce adds the chunks
// in order when there are several.  dl_vec: the dlogits rows are 16-byte aligned and E a
// multiple of 4, so a full group of 8 experts is read as two float4 (same values otherwise).
static constexpr int kRvExp = 8, kRvCols = 256;

__device__ __forceinline__ void unpack_bf16x8(const u32x4_t v, float* f) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    f[2 * h] = __uint_as_float(v[h] << 16);
    f[2 * h + 1] = __uint_as_float(v[h] & 0xffff0000u);
  }
}

__global__ void __launch_bounds__(256)
k_router_wgrad(const bf16_t* __restrict__ x, const float* __restrict__ dl, int T, int d,
                  int E, int tchunk, float* __restrict__ ow, size_t ow_stride,
                  float* __restrict__ ob, size_t ob_stride, int dl_vec) {
  __shared__ float s_w[kRvExp][kRvCols + 4];
  __shared__ float s_b[kRvExp];
  const int cg = threadIdx.x % 32, ph = threadIdx.x / 32;
  const int c = blockIdx.x * kRvCols + cg * 8, e0 = blockIdx.y * kRvExp;
  const int ne = min(kRvExp, E - e0);
  const bool full4 = ne == kRvExp && dl_vec;
  const bool cok = c < d;
  const int tb = blockIdx.z * tchunk, te = min(T, tb + tchunk);
  float acc[kRvExp][8], bacc[kRvExp];
#pragma unroll
  for (int i = 0; i < kRvExp; ++i) {
    bacc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  }
#pragma unroll 4
  for (int t = tb + ph; t < te; t += 8) {
    u32x4_t xv = {0u, 0u, 0u, 0u};
    if (cok) xv = *reinterpret_cast<const u32x4_t*>(x + (size_t)t * d + c);
    const float* dr = dl + (size_t)t * E + e0;
    float g[kRvExp];
    if (full4) {
      const float4 g0 = reinterpret_cast<const float4*>(dr)[0];
      const float4 g1 = reinterpret_cast<const float4*>(dr)[1];
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
      g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    } else {
#pragma unroll
      for (int i = 0; i < kRvExp; ++i) g[i] = i < ne ? dr[i] : 0.f;
    }
    float xf[8];
    unpack_bf16x8(xv, xf);
#pragma unroll
    for (int i = 0; i < kRvExp; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xf[j], g[i], acc[i][j]);
      bacc[i] += g[i];
    }
  }
  for (int p = 0; p < 8; ++p) {
    if (ph == p) {
#pragma unroll
      for (int i = 0; i < kRvExp; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          s_w[i][cg * 8 + j] = p == 0 ? acc[i][j] : s_w[i][cg * 8 + j] + acc[i][j];
        if (cg == 0) s_b[i] = p == 0 ? bacc[i] : s_b[i] + bacc[i];
      }
    }
    __syncthreads();
  }
  float* const w = ow + blockIdx.z * ow_stride;
  for (int o = threadIdx.x; o < kRvCols * kRvExp; o += 256) {
    const int oc = o / kRvExp, oi = o % kRvExp;
    const int cc = blockIdx.x * kRvCols + oc;
    if (ow && cc < d && oi < ne) w[(size_t)cc * E + e0 + oi] = s_w[oi][oc];
  }
  if (ob && blockIdx.x == 0 && threadIdx.x < ne)
    ob[blockIdx.z * ob_stride + e0 + threadIdx.x] = s_b[threadIdx.x];
}

// Token chunks of the router's weight gradient: blocks that all fit on the chip at once
// (about 768: 3 per compute unit at the kernel's register use), chunks of at least 256 tokens.
static int router_wgrad_chunks(const moe_shape& s) {
  const int64_t blocks2d = ceil_div(s.d, kRvCols) * ceil_div(s.E, kRvExp);
  const int64_t want = 768 / blocks2d;
  const int64_t most = ceil_div(s.T, 256);
  int64_t n = want < most ? want : most;
  return (int)(n < 1 ? 1 : n);
}

size_t router_bwd_scratch_bytes(const moe_shape& s) {
  const int n = router_wgrad_chunks(s);
  return n > 1 ? (size_t)n * ((size_t)s.d * s.E + s.E) * sizeof(float) : 0;
}

// dx_out[t, c] = (base[t, c] if base) + sum_e dlogits[t, e] W_g[c, e], rounded once to
// bf16.  A block owns 16 tokens (their dlogits rows in LDS, read as broadcasts) and 256
// columns (one per thread, its W_g row read once for all 16 tokens).
static constexpr int kRdTok = 16;

__global__ void __launch_bounds__(256)
k_router_dx(const float* __restrict__ dl, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ base,
            int T, int d, int E, bf16_t* __restrict__ out) {
  extern __shared__ float s_dl[];   // [kRdTok][E]
  const int t0 = blockIdx.x * kRdTok;
  const int nt = min(kRdTok, T - t0);
  for (int i = threadIdx.x; i < kRdTok * E; i += 256) {
    const int tt = i / E;
    s_dl[i] = tt < nt ? dl[(size_t)(t0 + tt) * E + i % E] : 0.f;
  }
  __syncthreads();
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= d) return;
  float v[kRdTok];
#pragma unroll
  for (int tt = 0; tt < kRdTok; ++tt) v[tt] = 0.f;
  const bf16_t* wr = wg + (size_t)c * E;
  for (int e = 0; e < E; ++e) {
    const float w = bf16_to_f32(wr[e]);
#pragma unroll
    for (int tt = 0; tt < kRdTok; ++tt) v[tt] = fmaf(s_dl[tt * E + e], w, v[tt]);
  }
#pragma unroll
  for (int tt = 0; tt < kRdTok; ++tt) {
    if (tt >= nt) break;
    const size_t o = (size_t)(t0 + tt) * d + c;
    out[o] = f32_to_bf16(base ? bf16_to_f32(base[o]) + v[tt] : v[tt]);
  }
}

// The same for rows whose width and E are multiples of 8 (16-byte aligned operands): a
// thread owns 8 adjacent columns and 8 of the block's 16 tokens (one 16-byte store per
// token), the block being 128 column groups (1024 columns) x 2 token groups.  W_g is read
// 8 columns x 8 experts at a time (eight 16-byte loads) and every output sums e in
// ascending order, so the result equals k_router_dx's bit for bit.
static constexpr int kRdvCols = 1024;

__global__ void __launch_bounds__(256)
k_router_dx_v8(const float* __restrict__ dl, const bf16_t* __restrict__ wg,
               const bf16_t* __restrict__ base, int T, int d, int E, bf16_t* __restrict__ out) {
  extern __shared__ float s_dl[];   // [kRdTok][E]
  const int t0 = blockIdx.x * kRdTok;
  const int nt = min(kRdTok, T - t0);
  const int cg = threadIdx.x % (kRdvCols / 8), tg = threadIdx.x / (kRdvCols / 8);
  const int c = blockIdx.y * kRdvCols + cg * 8;
  // the base rows are loaded first, to be in flight during the sums
  u32x4_t bv[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    bv[tt] = u32x4_t{0u, 0u, 0u, 0u};
    if (base && c < d && tg * 8 + tt < nt)
      bv[tt] = *reinterpret_cast<const u32x4_t*>(base + (size_t)(t0 + tg * 8 + tt) * d + c);
  }
  for (int i = threadIdx.x; i < kRdTok * E; i += 256) {
    const int tt = i / E;
    s_dl[i] = tt < nt ? dl[(size_t)(t0 + tt) * E + i % E] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  const float* sd = s_dl + tg * 8 * E;
  float v[8][8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[tt][j] = 0.f;
  for (int e = 0; e < E; e += 8) {
    u32x4_t wp[8];   // column c + j: experts e .. e + 7, packed
#pragma unroll
    for (int j = 0; j < 8; ++j) wp[j] = *reinterpret_cast<const u32x4_t*>(wg + (size_t)(c + j) * E + e);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j] = __uint_as_float(i & 1 ? wp[j][i >> 1] & 0xffff0000u : wp[j][i >> 1] << 16);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const float g = sd[tt * E + e + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[tt][j] = fmaf(g, w[j], v[tt][j]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    if (tg * 8 + tt >= nt) break;
    const size_t o = (size_t)(t0 + tg * 8 + tt) * d + c;
    float b[8];
    if (base) {
      unpack_bf16x8(bv[tt], b);
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] += v[tt][j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = v[tt][j];
    }
    u32x4_t r;
#pragma unroll
    for (int h = 0; h < 4; ++h) r[h] = pack_bf16x2(b[2 * h], b[2 * h + 1]);
    *reinterpret_cast<u32x4_t*>(out + o) = r;
  }
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moe_status launch_router_bwd(const moe_shape& s, const void* x, const void* w_gate,
                             const float* logits, const int32_t* idx, const float* dw,
                             float* dlogits, float* dw_gate, float* dbias, const void* dx_base,
                             void* dx_out, void* scratch, hipStream_t st) {
  if (s.E > 64 * kRbMaxPerLane) return MOE_ENOTSUP;
  if (s.T > 0) {
    hipLaunchKernelGGL(k_router_bwd, dim3((unsigned)ceil_div(s.T, 4)), dim3(256), 0, st, logits,
                       idx, dw, s.T, s.E, s.k, s.renormalize, dlogits);
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  // with T == 0 the weight gradients are zeros (the kernel reads no rows)
  if (dw_gate || dbias) {
    const int nch = router_wgrad_chunks(s);
    const int tchunk = (int)(ceil_div(ceil_div(s.T, nch), 8) * 8);
    const int64_t n = (int64_t)s.d * s.E;
    if (s.d % 8 || !aligned16(x)) return MOE_EINVAL;
    const int dl_vec = s.E % 4 == 0 && aligned16(dlogits);
    const dim3 grid((unsigned)ceil_div(s.d, kRvCols), (unsigned)ceil_div(s.E, kRvExp),
                    (unsigned)nch);
    auto sums = [&](float* ow, size_t ows, float* ob, size_t obs) {
      hipLaunchKernelGGL(k_router_wgrad, grid, dim3(256), 0, st,
                         static_cast<const bf16_t*>(x), dlogits, s.T, s.d, s.E, tchunk, ow, ows,
                         ob, obs, dl_vec);
    };
    if (nch == 1) {
      // one chunk: the sums go straight to the outputs (either may be NULL)
      sums(dw_gate, 0, dbias, 0);
    } else {
      if (!scratch) return MOE_EWORKSPACE;
      float* pw = static_cast<float*>(scratch);
      float* pb = pw + (size_t)nch * n;
      sums(pw, (size_t)n, pb, (size_t)s.E);
      if (hipGetLastError() != hipSuccess) return MOE_EHIP;
      hipLaunchKernelGGL(k_router_wgrad_reduce, dim3((unsigned)ceil_div(n > s.E ? n : s.E, 256)),
                         dim3(256), 0, st, pw, pb, nch, n, s.E, dw_gate, dbias);
    }
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  if (s.T > 0) {
    const bool vec = s.d % 8 == 0 && s.E % 8 == 0 && aligned16(w_gate) && aligned16(dx_out) &&
                     (!dx_base || aligned16(dx_base));
    const dim3 grid((unsigned)ceil_div(s.T, kRdTok),
                    (unsigned)ceil_div(s.d, vec ? kRdvCols : 256));
    const size_t lds = (size_t)kRdTok * s.E * sizeof(float);
    if (vec)
      hipLaunchKernelGGL(k_router_dx_v8, grid, dim3(256), lds, st, dlogits,
                         static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(dx_base),
                         s.T, s.d, s.E, static_cast<bf16_t*>(dx_out));
    else
      hipLaunchKernelGGL(k_router_dx, grid, dim3(256), lds, st, dlogits,
                         static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(dx_base),
                         s.T, s.d, s.E, static_cast<bf16_t*>(dx_out));
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace moe
