// fp8 (OCP e4m3) expert weights with a scale per 128 x 128 block (dropless notes
// section 12: fp8 weights carry a scale per quantisation block; dequantise before
// the product when the block is narrower than the matrix unit's contraction, else the
// scale can go after it).  Here the bf16 MFMA takes 16-deep slices, narrower than the
// 128-deep block, so either order works; the weights are dequantised in registers
// just before the MFMA (code -> fp32, times the block scale, rounded to bf16), which
// keeps one accumulator set and costs 16 VALU operations per 32 x 16 B fragment.
//
//   * k_quantize_fp8: one work group per 128 x 128 block of one expert matrix:
//     amax, scale = amax / 448 (1 for an all-zero block), codes = round-to-nearest-
//     even of clamp(w / scale, -448, 448), all in fp32.
//   * k_gg_fp8w: the grouped GEMM of the 128-row asynchronous-copy kernel with fp8
//     B.  The copies move fp8 bytes (half the bf16 bytes), so a 24 KB slice (8 KB of A,
//     16 KB of B for 32 x 512) fits a six-slot ring.  B stays [k][n] in LDS with the
//     16-byte chunk swizzle c ^ (k & 15) and is read with ds_read_b64_tr_b8: in each
//     16-lane group lane i points at row i / 2, bytes 8 (i % 2) .. +7 of an 8 x 16 block
//     and receives column i's 8 rows, exactly the 8 consecutive k values one lane
//     supplies to v_mfma_f32_32x32x16_bf16 (lane layout established with a probe).
//     Rows may be gathered from x through row_src as in the bf16 kernels.
#include "moe_gemm_common.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

namespace moe {

static constexpr int kQBlock = 128;        // quantisation block (k and n)
static constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// quantiser
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_quantize_fp8(const bf16_t* __restrict__ w, uint8_t* __restrict__ q, float* __restrict__ scales,
               int K, int N) {
  __shared__ float s_max[4];
  const int nb = blockIdx.x, kb = blockIdx.y, e = blockIdx.z;
  const int NB = gridDim.x, KB = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c8 = tid & 15;          // 8-column chunk of the block
  const int r0 = tid >> 4;          // rows r0 + 16 i
  const int col = nb * kQBlock + c8 * 8;
  const bf16_t* src = w + (size_t)e * K * N;
  u32x4_t v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = kb * kQBlock + r0 + 16 * i;
    if (row < K && col < N) {
      v[i] = *reinterpret_cast<const u32x4_t*>(src + (size_t)row * N + col);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][h] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][h] & 0xffff0000u)));
      }
    } else {
      v[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float scale = amax > 0.f ? amax / kE4M3Max : 1.0f;
  if (tid == 0) scales[((size_t)e * KB + kb) * NB + nb] = scale;
  uint8_t* dst = q + (size_t)e * K * N;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = kb * kQBlock + r0 + 16 * i;
    if (row >= K || col >= N) continue;
    uint32_t packed[2];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float lo = fminf(fmaxf(__uint_as_float(v[i][h] << 16) / scale, -kE4M3Max), kE4M3Max);
      const float hi = fminf(fmaxf(__uint_as_float(v[i][h] & 0xffff0000u) / scale, -kE4M3Max),
                             kE4M3Max);
      // two codes into bytes 2(h & 1), 2(h & 1) + 1 of packed[h >> 1]
      const int word = __builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false) & 0xffff;
      if (h & 1)
        packed[h >> 1] |= (uint32_t)word << 16;
      else
        packed[h >> 1] = (uint32_t)word;
    }
    *reinterpret_cast<uint2*>(dst + (size_t)row * N + col) = make_uint2(packed[0], packed[1]);
  }
}

moe_status launch_quantize_fp8(int E, int K, int N, const void* w, uint8_t* q, float* scales,
                               hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(N, kQBlock), (unsigned)ceil_div(K, kQBlock), (unsigned)E);
  hipLaunchKernelGGL(k_quantize_fp8, grid, dim3(256), 0, st, static_cast<const bf16_t*>(w), q,
                     scales, K, N);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Dequantisation to bf16: w[e][k][n] = bf16(code * scale[e][k / 128][n / 128]), the code
// decoded to fp32 by the hardware conversion and the product rounded to nearest even -
// exactly what the fp8 grouped GEMM does to each fragment before its MFMA.  One thread
// per 8 consecutive codes of a row (N % 8 == 0, so 8 codes never straddle a block).
__global__ void __launch_bounds__(256)
k_dequantize_fp8(const uint8_t* __restrict__ q, const float* __restrict__ scales, int64_t n8,
                 int K, int N, int KB, int NB, bf16_t* __restrict__ w) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const int64_t el = i * 8;                 // first element of the 8
    const int n = (int)(el % N);
    const int64_t ek = el / N;                // e * K + k
    const int k = (int)(ek % K);
    const int64_t e = ek / K;
    const float sc = scales[((size_t)e * KB + k / 128) * NB + n / 128];
    const uint2 raw = *reinterpret_cast<const uint2*>(q + el);
    const uint32_t rw[2] = {raw.x, raw.y};
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(rw[h], false);   // bytes 0, 1
      const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(rw[h], true);    // bytes 2, 3
      const __bf16 b0 = static_cast<__bf16>(f0[0] * sc), b1 = static_cast<__bf16>(f0[1] * sc);
      const __bf16 b2 = static_cast<__bf16>(f1[0] * sc), b3 = static_cast<__bf16>(f1[1] * sc);
      o[2 * h] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      o[2 * h + 1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
    }
    *reinterpret_cast<u32x4_t*>(w + el) = o;
  }
}

moe_status launch_dequantize_fp8(int E, int K, int N, const uint8_t* q, const float* scales,
                                 void* w, hipStream_t st) {
  const int64_t n8 = (int64_t)E * K * N / 8;
  if (n8 == 0) return MOE_OK;
  int64_t blocks = ceil_div(n8, 256);
  const int64_t cap = (int64_t)device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_dequantize_fp8, dim3((unsigned)blocks), dim3(256), 0, st, q, scales, n8, K,
                     N, (int)ceil_div(K, 128), (int)ceil_div(N, 128), static_cast<bf16_t*>(w));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// grouped GEMM with fp8 B
// ---------------------------------------------------------------------------
static constexpr int kFThreads = 512;                 // 8 waves
static constexpr int kFBK = 32;                       // K per ring slot
static constexpr int kFABytes = 128 * kFBK * 2;       // 8 KB of A (bf16)
static constexpr int kFBHalf = kFBK * 256;            // 8 KB per 256-column half (fp8)
static constexpr int kFStage = kFABytes + 2 * kFBHalf;  // 24 KB
static constexpr int kFStages = 6;
static constexpr int kFCopies = 1 + 2;                // per wave per slice: A, B
static constexpr int kFMaxKB = 256;                   // k-blocks per item held in LDS

// Operands of one segment set with fp8 B: codes and scales per matrix.
struct GGOperandsF8 {
  GGOperands base;          // A, C, gather; base.B0 / base.B1 unused
  const uint8_t* Q0;
  const uint8_t* Q1;
  const float* S0;
  const float* S1;
};

__device__ __forceinline__ int swz_q(int k, int chunk) { return chunk ^ (k & 15); }

template <int OP>
__global__ void __launch_bounds__(kFThreads, 1)
k_gg_fp8w(GGOperandsF8 routed, GGOperandsF8 dense, int K, int N,
          const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
          int max_blocks, int E, int64_t max_rows, int dense_rows, int n_tiles) {
  constexpr bool GU = OP == MOE_OP_GATEUP_SWIGLU;
  constexpr int kOutCols = GU ? 256 : 512;
  __shared__ __align__(1024) unsigned char lds[kFStages * kFStage];
  // the item's block scales: [kb][4] (GATEUP: W1 n-blocks 0, 1 then W3 n-blocks 0, 1
  // of the tile; DOWN: n-blocks 0..3 of the tile)
  __shared__ float s_scale[kFMaxKB * 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb_dense = (dense_rows + 127) / 128;
  const int nblocks = nb_dense + (max_blocks > 0 ? clamp_block_count(num_blocks_ptr, max_blocks) : 0);
  const int total = nblocks * n_tiles;
  const int nk = K / kFBK;
  const int KB = (K + kQBlock - 1) / kQBlock, NBq = (N + kQBlock - 1) / kQBlock;

  // B fragment reads: 16-lane group g, lane gi of it; subtile j of the wave: LDS half
  // and first column within the half.
  const int g = lane >> 4, gi = lane & 15;
  int bhalf[2], bcol0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bhalf[j] = GU ? j : wave >> 2;
    bcol0[j] = GU ? wave * 32 : (wave & 3) * 64 + j * 32;
  }
  uint32_t b_lane[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = 8 * (g >> 1) + (gi >> 1);                // row within a 16-deep step
    const int chunk = bcol0[j] / 16 + (g & 1);
    b_lane[j] = (uint32_t)(bhalf[j] * kFBHalf + k * 256 + swz_q(k, chunk) * 16 + (gi & 1) * 8);
  }
  // the scale slot of subtile j: [kb][4] index
  int sidx[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    sidx[j] = GU ? j * 2 + (bcol0[j] >> 7) : (bhalf[j] * 256 + bcol0[j]) >> 7;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int nt = w % n_tiles;
    const int blk = w / n_tiles;
    const bool in_dense = blk < nb_dense;
    Tile tile;
    if (in_dense) {
      if (!decode_block(blk, 0, 128, 128, nullptr, dense_rows, 1, dense_rows, tile)) continue;
    } else {
      if (!decode_block(blk - nb_dense, 0, 128, 128, meta, 0, E, max_rows, tile)) continue;
    }
    const GGOperandsF8& ops = in_dense ? dense : routed;
    bf16_t* const C = ops.base.C;
    const int n0 = nt * kOutCols;
    const int e = tile.e;

    // block scales of this item's columns, every k-block
    {
      const float* s0 = ops.S0 + (size_t)e * KB * NBq;
      const float* s1 = GU ? ops.S1 + (size_t)e * KB * NBq : s0;
      for (int i = tid; i < KB * 4; i += kFThreads) {
        const int kb = i >> 2, slot = i & 3;
        int nb;
        const float* sp;
        if (GU) {
          nb = (n0 >> 7) + (slot & 1);
          sp = slot < 2 ? s0 : s1;
        } else {
          nb = (n0 >> 7) + slot;
          sp = s0;
        }
        s_scale[i] = nb < NBq ? sp[(size_t)kb * NBq + nb] : 1.0f;
      }
    }

    // A copy (one per wave per slice): the wave's 16-row window; rows past valid_m
    // copy row 0, gathered rows come from x.
    const bf16_t* asrc = ops.base.A + (size_t)tile.m0 * K;
    uint32_t a_voff;
    {
      const int row = wave * 16 + (lane >> 2);
      const int c = swz_a(row, lane & 3);
      const int rr = row < tile.valid ? row : 0;
      const int src = ops.base.gather ? gather_row(ops.base, tile.m0 + rr) : rr;
      a_voff = (uint32_t)(src * K + c * 8) * 2u;
    }
    asrc = uniform_ptr(ops.base.gather ? ops.base.A : asrc);
    // B copies: copy u = 2 wave + p of 16 moves rows 4u'..4u'+3 (u' = u % 8) of half
    // u / 8, 16 lanes per 256-byte row; the logical chunk of lane l is
    // (l & 15) ^ ((4u' + (l >> 4)) & 15).  Columns past N copy column 0.
    const uint8_t* bh_base[2];
    int bh_col0[2];
    bh_base[0] = ops.Q0 + (size_t)e * K * N;
    bh_base[1] = GU ? ops.Q1 + (size_t)e * K * N : bh_base[0];
    bh_col0[0] = n0;
    bh_col0[1] = GU ? n0 : n0 + 256;
    uint32_t b_voff[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int u = wave * 2 + p;
      const int uu = u & 7, h = u >> 3;
      const int k = 4 * uu + (lane >> 4);
      int col = bh_col0[h] + swz_q(k, lane & 15) * 16;
      if (col >= N) col = 0;
      b_voff[p] = (uint32_t)((lane >> 4) * N + col);
    }
    const int bu_h = (wave * 2) >> 3;                      // both copies in one half
    const uint8_t* bsrc = uniform_ptr(bh_base[bu_h]);
    auto issue = [&](int ks, int slot) {
      unsigned char* st = lds + slot * kFStage;
      const int k0 = ks * kFBK;
      copy16_to_lds(asrc + k0, a_voff, st + wave * 1024);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int uu = (wave * 2 + p) & 7;
        copy16_to_lds(bsrc + (size_t)(k0 + 4 * uu) * N, b_voff[p],
                      st + kFABytes + bu_h * kFBHalf + uu * 1024);
      }
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
    bf16x8_t af[4], bf[2];
    auto read_frags = [&](int ks, int kk) {
      const unsigned char* sa = lds + (ks % kFStages) * kFStage;
      const unsigned char* sb = sa + kFABytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nsub) break;
        const int row = i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16);
      }
      const int kb = (ks * kFBK) >> 7;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        typedef int v2i __attribute__((ext_vector_type(2)));
        const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (MOE_LDS v2i*)(sb + b_lane[j] + kk * 16 * 256));
        const float sc = s_scale[kb * 4 + sidx[j]];
        bf16x8_t o;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[h], false);   // bytes 0, 1
          const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[h], true);    // bytes 2, 3
          o[4 * h + 0] = static_cast<__bf16>(f0[0] * sc);
          o[4 * h + 1] = static_cast<__bf16>(f0[1] * sc);
          o[4 * h + 2] = static_cast<__bf16>(f1[0] * sc);
          o[4 * h + 3] = static_cast<__bf16>(f1[1] * sc);
        }
        bf[j] = o;
      }
    };
    auto mfma_block = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nsub) break;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    };

    // Prologue: every slot in flight (slices past the end re-copy the last slice into a
    // slot that is never read), then wait for slice 0.  The scale table was written by
    // plain LDS stores; the barrier publishes it too.
#pragma unroll
    for (int p = 0; p < kFStages; ++p) issue(min(p, nk - 1), p);
    MOE_WAIT_VMCNT((kFStages - 1) * kFCopies);
    __syncthreads();

    // Slice ks: two 16-deep halves, then a barrier once slice ks+1 has landed; the
    // barrier that ended slice ks-1 freed its slot, which slice ks-1+S refills.
    for (int ks = 0; ks < nk; ++ks) {
      if (ks > 0) issue(min(ks - 1 + kFStages, nk - 1), (ks - 1) % kFStages);
      read_frags(ks, 0);
      mfma_block();
      read_frags(ks, 1);
      mfma_block();
      if (ks + 1 < nk) {
        MOE_WAIT_VMCNT((kFStages - 2) * kFCopies);   // slice ks+1 has landed
        __syncthreads();
      }
    }
    MOE_WAIT_VMCNT(0);  // no copy may land in the ring once it is reused below
    __syncthreads();

    // Epilogue through LDS (as the bf16 kernel): bf16 staging per wave, 16-byte stores.
    constexpr int kWCols = GU ? 32 : 64;
    constexpr int kHalves = GU ? 1 : 2;
    constexpr int kRowsPer = 128 / kHalves;
    constexpr int kLd = kWCols + 8;
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
      constexpr int kChunks = kWCols / 8;
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
    __syncthreads();  // staging and scale reads done before the next item refills
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with fp8 B for few rows per expert (decode): the launch streams the
// weights, so a work item is 64 rows (a half of a 128-row block; halves without valid
// rows are skipped, 32-row subtiles without valid rows are not multiplied) and wide
// columns: 512 act columns for gate/up (512 bytes of each of W1 and W3 per k row) and
// 1024 columns for down (1 KB per k row), so that every 32-deep slice moves 32 KB of
// weights as 1 KB copies of one or two rows - the memory shape of the bf16 128-row
// kernel, which streams its weights near 6.1 TB/s.  8 waves; wave w owns 64 act columns
// (gate/up: W1 and the matching W3 columns) or 128 down columns, two 32-row subtiles x
// four 32-column tiles of v_mfma_f32_32x32x16_bf16.  Fragments are dequantised in
// registers as in k_gg_fp8w.
//
// Last round.  A persistent grid of G work groups runs the V items in ceil(V / G)
// rounds, the last with only R = V mod G of them.  Given scratch (and a table whose
// blocks all hold at most 64 rows, as decode's do), the kernel runs the first V - R
// items as above and then spreads the R items' R * nk slices evenly over all G work
// groups: work group q takes slices [q R nk / G, (q+1) R nk / G) of them, a contiguous
// range that touches at most two items, and writes each piece's fp32 sums (valid rows)
// to scratch slot 2q or 2q+1.  k_fp8d_tail then adds an item's pieces in slice order
// (fixed, so the result does not depend on timing) and applies the epilogue.
// ---------------------------------------------------------------------------
static constexpr int kDRows = 64;                          // rows per work item
static constexpr int kDABytes = kDRows * kFBK * 2;        // 4 KB of A per slice
static constexpr int kDBBytes = 32 * 1024;                // 32 KB of B per slice
static constexpr int kDStage = kDABytes + kDBBytes;       // 36 KB
static constexpr int kDStages = 4;
static constexpr int kDBCopies = kDBBytes / 1024 / 8;     // 4 B copies per wave per slice
// last-round scratch: a 256-byte header (the plan: on, F, R, written by work group 0),
// then two slots per work group of at most kDTailGrid, each 64 rows x 1024 fp32
// (gate/up: 512 gate sums then 512 up sums; down: 1024 sums)
static constexpr int kDTailGrid = 256;
static constexpr int kDTailCols = 1024;
static constexpr int kDTailHeader = 64;                    // floats
static constexpr size_t kDTailSlot = (size_t)kDRows * kDTailCols * 4;
static constexpr int kDTailRowGroups = 8;                  // tail kernel: row strides

size_t fp8_tail_scratch_bytes() { return kDTailHeader * 4 + 2 * (size_t)kDTailGrid * kDTailSlot; }

// Whether the last round of a 64-row launch over G work groups splits along K, and its
// shape: V items (all of them valid, the blocks' first halves), F full rounds, R items
// left.  Every work group of both kernels derives the same answer from the table.
struct FP8Tail {
  int V, F, R;
  bool on;
};
__device__ __forceinline__ bool fp8d_table_fits(const int32_t* __restrict__ meta, int nroutes,
                                                int E, int64_t max_rows, int dense_rows,
                                                int wave, int lane, int* s_flag) {
  // one wave checks every entry (in range, 1..64 rows); the answer goes through LDS
  if (wave == 0) {
    bool bad = dense_rows > kDRows;
    for (int b = lane; b < nroutes; b += 64) {
      const int e = meta[3 * b], m = meta[3 * b + 1], v = meta[3 * b + 2];
      bad |= e < 0 || e >= E || m < 0 || v < 1 || v > kDRows || (int64_t)m + v > max_rows;
    }
    const bool any = __ballot(bad) != 0ull;
    if (lane == 0) *s_flag = any ? 0 : 1;
  }
  __syncthreads();
  const bool fits = *s_flag != 0;
  __syncthreads();
  return fits;
}
__device__ __forceinline__ FP8Tail fp8d_tail_plan(bool fits, int per_half, int G) {
  FP8Tail t;
  t.V = per_half;
  t.F = per_half / G;
  t.R = per_half - t.F * G;
  // worth it while the last round is at most 90 % full; with at least G / 16 items left
  // every work group takes at least nk / 16 - 1 slices, so an item has at most 34 pieces
  t.on = fits && G <= kDTailGrid && t.R > 0 && 10 * t.R <= 9 * G && 16 * t.R >= G;
  return t;
}

template <int OP>
__global__ void __launch_bounds__(kFThreads, 1)
k_gg_fp8d(GGOperandsF8 routed, GGOperandsF8 dense, int K, int N,
          const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
          int max_blocks, int E, int64_t max_rows, int dense_rows, int n_tiles,
          float* __restrict__ tail) {
  constexpr bool GU = OP == MOE_OP_GATEUP_SWIGLU;
  constexpr int kOutCols = GU ? 512 : 1024;               // output columns per item
  constexpr int kPitch = GU ? 512 : 1024;                 // bytes per staged B row (per matrix)
  __shared__ __align__(1024) unsigned char lds[kDStages * kDStage];
  // block scales of two items (the current one and the next, double-buffered): [kb][8]
  // (gate/up: W1 n-blocks 0..3 of the tile, then W3's; down: n-blocks 0..7)
  __shared__ float s_scale[2][kFMaxKB * 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb_dense = (dense_rows + 127) / 128;
  const int nblocks = nb_dense + (max_blocks > 0 ? clamp_block_count(num_blocks_ptr, max_blocks) : 0);
  // items (half, block, column tile), half outermost: decode blocks rarely have a second
  // half, and with the half inner a persistent grid would give some work groups only
  // empty items
  const int per_half = nblocks * n_tiles;
  const int total = 2 * per_half;
  const int nk = K / kFBK;
  const int KB = (K + kQBlock - 1) / kQBlock, NBq = (N + kQBlock - 1) / kQBlock;
  const bool has_a = wave < kDABytes / 1024;               // waves 0..3 copy A
  // consecutive items of a work group run as one stream of slices: the last refills of
  // an item fetch the next item's first slices (the launcher guarantees nk >= the ring
  // depth)

  // B fragment reads (ds_read_b64_tr_b8, as k_gg_fp8w): 16-lane group g, lane gi; tile j
  // of the wave: matrix region and first column within it.
  const int g = lane >> 4, gi = lane & 15;
  uint32_t b_lane[4];
  int sidx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int region = GU ? (j >> 1) : 0;                 // gate/up: W1 for j < 2, W3 after
    const int col0 = GU ? wave * 64 + (j & 1) * 32 : wave * 128 + j * 32;
    const int k = 8 * (g >> 1) + (gi >> 1);               // row within a 16-deep step
    const int chunk = col0 / 16 + (g & 1);
    b_lane[j] = (uint32_t)(region * (kDBBytes / 2) + k * kPitch + (chunk ^ (k & 15)) * 16 +
                           (gi & 1) * 8);
    sidx[j] = GU ? region * 4 + (col0 >> 7) : (col0 >> 7);
  }

  // One work item's operands: slices [k0, k0 + n) of item w, written to C (slot < 0) or
  // as fp32 sums to scratch slot `slot`.
  struct Item {
    int w;                        // item number, -1: none
    int k0, n, slot;
    Tile tile;
    int n0;
    bool dense;
    const bf16_t* asrc;           // A base (wave-uniform)
    uint32_t a_voff;              // this lane's A offset (waves 0..3)
    const uint8_t* bsrc;          // the wave's B matrix base (wave-uniform)
    uint32_t b_voff[kDBCopies];
  };
  // the first slice row of B copy p of this wave (the same for every item): gate/up copies
  // two rows, 2 (u % 16) and the next, down one, u (u = kDBCopies wave + p)
  auto b_row = [&](int p) {
    const int u = wave * kDBCopies + p;
    return GU ? 2 * (u & 15) : u;
  };
  // item w's tile, if it has valid rows
  auto decode_item = [&](int w, Item& it) {
    const int half = w / per_half;
    const int rem = w - half * per_half;
    const int nt = rem % n_tiles;
    const int blk = rem / n_tiles;
    const bool in_dense = blk < nb_dense;
    bool ok;
    if (in_dense)
      ok = decode_block(blk, half, kDRows, 128, nullptr, dense_rows, 1, dense_rows, it.tile);
    else
      ok = decode_block(blk - nb_dense, half, kDRows, 128, meta, 0, E, max_rows, it.tile);
    it.dense = in_dense;
    it.n0 = nt * kOutCols;
    return ok;
  };
  // the copy offsets of a decoded item
  auto setup_item = [&](Item& it) {
    const GGOperandsF8& ops = it.dense ? dense : routed;
    const int e = it.tile.e;
    // A copy (waves 0..3, one per slice): 16 rows x 64 bytes; rows past valid_m copy
    // row 0, gathered rows come from x.
    it.a_voff = 0;
    if (has_a) {
      const int row = wave * 16 + (lane >> 2);
      const int c = swz_a(row, lane & 3);
      const int rr = row < it.tile.valid ? row : 0;
      const int src = ops.base.gather ? gather_row(ops.base, it.tile.m0 + rr) : rr;
      it.a_voff = (uint32_t)(src * K + c * 8) * 2u;
    }
    it.asrc = uniform_ptr(ops.base.gather ? ops.base.A : ops.base.A + (size_t)it.tile.m0 * K);
    // B copies: copy u = 4 wave + p of 32.  Gate/up: region u / 16 (W1, W3), rows
    // 2 (u % 16) and 2 (u % 16) + 1 of the region, 32 lanes per 512-byte row; down:
    // row u, 64 lanes per 1 KB row.  The logical chunk of lane l is its position
    // XOR (k & 15); columns past N copy column 0.
    const uint8_t* qb0 = ops.Q0 + (size_t)e * K * N;
    const uint8_t* qb1 = GU ? ops.Q1 + (size_t)e * K * N : qb0;
#pragma unroll
    for (int p = 0; p < kDBCopies; ++p) {
      const int u = wave * kDBCopies + p;
      int k, pos;
      if (GU) {
        k = 2 * (u & 15) + (lane >> 5);
        pos = lane & 31;
      } else {
        k = u;
        pos = lane;
      }
      int col = it.n0 + (pos ^ (k & 15)) * 16;
      if (col >= N) col = 0;
      it.b_voff[p] = (uint32_t)((k - b_row(p)) * N + col);
    }
    it.bsrc = uniform_ptr((GU && ((wave * kDBCopies) >> 4)) ? qb1 : qb0);
  };
  // the first valid item at or after number w of this work group's sequence, below
  // `limit`: all its slices, to C
  auto find_item = [&](int w, int limit, Item& it) {
    it.w = -1;
    for (; w < limit; w += gridDim.x) {
      if (!decode_item(w, it)) continue;
      it.w = w;
      break;
    }
    if (it.w < 0) return;
    it.k0 = 0;
    it.n = nk;
    it.slot = -1;
    setup_item(it);
  };
  // slice ks of an item into ring slot `slot`
  auto issue = [&](const Item& it, int ks, int slot) {
    unsigned char* st = lds + slot * kDStage;
    const int k0 = ks * kFBK;
    if (has_a) copy16_to_lds(it.asrc + k0, it.a_voff, st + wave * 1024);
#pragma unroll
    for (int p = 0; p < kDBCopies; ++p) {
      const int u = wave * kDBCopies + p;
      copy16_to_lds(it.bsrc + (size_t)(k0 + b_row(p)) * N, it.b_voff[p], st + kDABytes + u * 1024);
    }
  };
  // an item's block scales into buffer `buf` (plain LDS stores: a barrier publishes them)
  auto load_scales = [&](const Item& it, int buf) {
    const GGOperandsF8& ops = it.dense ? dense : routed;
    const int e = it.tile.e;
    const float* s0 = ops.S0 + (size_t)e * KB * NBq;
    const float* s1 = GU ? ops.S1 + (size_t)e * KB * NBq : s0;
    for (int i = tid; i < KB * 8; i += kFThreads) {
      const int kb = i >> 3, slot = i & 7;
      const int nb = (it.n0 >> 7) + (GU ? (slot & 3) : slot);
      const float* sp = (GU && slot >= 4) ? s1 : s0;
      s_scale[buf][i] = nb < NBq ? sp[(size_t)kb * NBq + nb] : 1.0f;
    }
  };
  // every copy a wave has issued lands in order: wait until at most n slices of its
  // copies are outstanding (waves 0..3 issue one more copy per slice)
  auto wait_slices = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    if (has_a) MOE_WAIT_VMCNT(n * (kDBCopies + 1));
    else MOE_WAIT_VMCNT(n * kDBCopies);
  };

  // Item `cur` and, for whole items, the ones after it in this work group's sequence
  // below `limit`, as one stream of slices through the ring; returns with every copy
  // landed.
  auto run = [&](Item cur, int limit) {
    Item nxt;
    nxt.w = -1;
    if (cur.slot < 0) find_item(cur.w + gridDim.x, limit, nxt);
    load_scales(cur, 0);
    // Prologue: every slot in flight (slices past the end re-copy the last slice into a
    // slot that is never read), then wait for slice 0; the barrier also publishes the
    // scale table.
#pragma unroll
    for (int p = 0; p < kDStages; ++p) issue(cur, cur.k0 + min(p, cur.n - 1), p);
    wait_slices(std::integral_constant<int, kDStages - 1>{});
    __syncthreads();

    int gbase = 0;      // stream position of the current item's first slice
    int buf = 0;        // its scale buffer
    while (true) {
      // the next item's scales, read only once its slices are computed (the barriers in
      // between publish them)
      if (nxt.w >= 0) load_scales(nxt, buf ^ 1);
      const int nsub = __builtin_amdgcn_readfirstlane(min(2, (cur.tile.valid + 31) >> 5));
      f32x16_t acc[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

      bf16x8_t af[2], bf[4];
      auto read_frags = [&](int slot, int ks, int kk) {
        const unsigned char* sa = lds + slot * kDStage;
        const unsigned char* sb = sa + kDABytes;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (i >= nsub) break;
          const int row = i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8_t*>(sa + row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16);
        }
        const int kb = (ks * kFBK) >> 7;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          typedef int v2i __attribute__((ext_vector_type(2)));
          const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (MOE_LDS v2i*)(sb + b_lane[j] + kk * 16 * kPitch));
          const float sc = s_scale[buf][kb * 8 + sidx[j]];
          bf16x8_t o;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[h], false);   // bytes 0, 1
            const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(raw[h], true);    // bytes 2, 3
            o[4 * h + 0] = static_cast<__bf16>(f0[0] * sc);
            o[4 * h + 1] = static_cast<__bf16>(f0[1] * sc);
            o[4 * h + 2] = static_cast<__bf16>(f1[0] * sc);
            o[4 * h + 3] = static_cast<__bf16>(f1[1] * sc);
          }
          bf[j] = o;
        }
      };
      auto mfma_block = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (i >= nsub) break;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
      };

      for (int ks = 0; ks < cur.n; ++ks) {
        const int gs = gbase + ks;
        if (gs > 0) {
          // refill the slot of stream slice gs-1 (every wave has read it) with stream
          // slice gs-1+S: this item's, the next item's, or a re-copy of this item's last
          // slice (whole items have n = nk >= S slices; the launcher checks)
          const int t = gs - 1 + kDStages - gbase;
          const int slot = (gs - 1) % kDStages;
          if (t < cur.n) issue(cur, cur.k0 + t, slot);
          else if (nxt.w >= 0) issue(nxt, nxt.k0 + t - cur.n, slot);
          else issue(cur, cur.k0 + cur.n - 1, slot);
        }
        const int slot = gs % kDStages;
        read_frags(slot, cur.k0 + ks, 0);
        mfma_block();
        read_frags(slot, cur.k0 + ks, 1);
        mfma_block();
        if (ks + 1 < cur.n || nxt.w >= 0) {
          wait_slices(std::integral_constant<int, kDStages - 2>{});   // stream slice gs+1 landed
          __syncthreads();
        }
      }

      // Epilogue: 16-bit stores straight from the accumulators (32 lanes store 64
      // contiguous bytes of a row), valid rows and columns only; a piece of a split item
      // stores its fp32 sums to its scratch slot instead.  The ring is not touched, so
      // the next item's slices keep landing.
      {
        const GGOperandsF8& ops = cur.dense ? dense : routed;
        bf16_t* const C = ops.base.C;
        constexpr int kWCols = GU ? 64 : 128;
        const int col0 = cur.n0 + wave * kWCols;
        if (cur.slot >= 0) {
          // a piece: its fp32 sums to its scratch slot (one loop nest of its own, so that
          // its addresses do not share registers with the bf16 stores below)
          // lane base: row (l >> 5) * 4, this wave's first column; every store then adds
          // a constant
          float* const pl = tail + kDTailHeader + (size_t)cur.slot * (kDTailSlot / 4) +
                            (size_t)((lane >> 5) * 4) * kDTailCols +
                            (GU ? wave * 64 : wave * 128) + (lane & 31);
          const int vrow = cur.tile.valid - (lane >> 5) * 4;   // rows r_off < vrow are valid
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            if (i >= nsub) break;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r_off = i * 32 + (q >> 2) * 8 + (q & 3);
              if (r_off >= vrow) continue;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int c = GU ? (j >> 1) * 512 + (j & 1) * 32 : j * 32;
                pl[r_off * kDTailCols + c] = acc[i][j][q];
              }
            }
          }
        } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (i >= nsub) break;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
            if (r >= cur.tile.valid) continue;
            bf16_t* crow = C + (size_t)(cur.tile.m0 + r) * N;
            if (GU) {
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const int col = col0 + j * 32 + (lane & 31);
                if (col < N) crow[col] = f32_to_bf16(silu_f32(acc[i][j][q]) * acc[i][j + 2][q]);
              }
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int col = col0 + j * 32 + (lane & 31);
                if (col < N) crow[col] = f32_to_bf16(acc[i][j][q]);
              }
            }
          }
        }
        }
      }
      if (nxt.w < 0) break;
      gbase += cur.n;
      cur = nxt;
      find_item(cur.w + gridDim.x, limit, nxt);
      buf ^= 1;
    }
    MOE_WAIT_VMCNT(0);  // the re-copies past the last slice land before the ring is reused
  };

  // the last round split along K where it applies (tail: scratch, or NULL)
  const bool fits = tail != nullptr &&
                    fp8d_table_fits(meta, nblocks - nb_dense, E, max_rows, dense_rows, wave, lane,
                                    reinterpret_cast<int*>(lds));
  const FP8Tail plan = fp8d_tail_plan(fits, per_half, (int)gridDim.x);
  const int limit = plan.on ? plan.F * (int)gridDim.x : total;
  if (tail && blockIdx.x == 0 && tid == 0) {   // the plan, for k_fp8d_tail
    int* hdr = reinterpret_cast<int*>(tail);
    hdr[0] = plan.on ? 1 : 0;
    hdr[1] = plan.F;
    hdr[2] = plan.R;
  }
  {
    Item first;
    find_item(blockIdx.x, limit, first);
    if (first.w >= 0) run(first, limit);
  }
  if (!plan.on) return;
  // this work group's slices of the last R items: [lo, hi) of R * nk
  const int64_t S = (int64_t)plan.R * nk, G = gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * S / G, hi = ((int64_t)blockIdx.x + 1) * S / G;
  for (int64_t sl = lo; sl < hi;) {
    const int r = (int)(sl / nk);
    Item pc;
    pc.w = plan.F * (int)gridDim.x + r;
    decode_item(pc.w, pc);             // valid: every item below V is (the table fits)
    pc.k0 = (int)(sl - (int64_t)r * nk);
    const int64_t end = (int64_t)(r + 1) * nk;
    pc.n = (int)((hi < end ? hi : end) - sl);
    pc.slot = 2 * (int)blockIdx.x + (sl == lo ? 0 : 1);
    setup_item(pc);
    __syncthreads();                   // every wave is done with the ring and the scales
    run(pc, 0);
    sl = (int64_t)(r + 1) * nk;
  }
}

typedef float tail_f32x4 __attribute__((ext_vector_type(4)));

// The last round's items of a split 64-row launch (k_gg_fp8d): item r's pieces, from the
// work groups whose slice ranges overlap it, added in slice order, then the epilogue.
// Work group (r, y) takes rows y, y + 8, ... of item r (the ones past the plan's R or the
// item's valid rows exit); each thread sums 4 adjacent columns (gate/up: of the gate and
// the up sums), issuing the loads of four pieces before adding them in order.
template <int OP>
__global__ void __launch_bounds__(256)
k_fp8d_tail(GGOperandsF8 routed, GGOperandsF8 dense, int K, int N,
            const int32_t* __restrict__ meta, const int32_t* __restrict__ num_blocks_ptr,
            int max_blocks, int E, int64_t max_rows, int dense_rows, int n_tiles, int G,
            const float* __restrict__ tail) {
  constexpr bool GU = OP == MOE_OP_GATEUP_SWIGLU;
  constexpr int kOutCols = GU ? 512 : 1024;
  constexpr int kMaxPieces = 64;
  __shared__ int s_slot[kMaxPieces];
  __shared__ int s_npieces;
  const int tid = threadIdx.x;
  const int* hdr = reinterpret_cast<const int*>(tail);
  if (hdr[0] == 0) return;
  const int F = hdr[1], R = hdr[2];
  const int r = blockIdx.x;
  if (r >= R) return;
  const int nb_dense = (dense_rows + 127) / 128;
  const int nk = K / kFBK;
  const int w = F * G + r;
  const int nt = w % n_tiles, blk = w / n_tiles;
  Tile tile;
  const bool in_dense = blk < nb_dense;
  if (in_dense) decode_block(blk, 0, kDRows, 128, nullptr, dense_rows, 1, dense_rows, tile);
  else decode_block(blk - nb_dense, 0, kDRows, 128, meta, 0, E, max_rows, tile);
  if ((int)blockIdx.y >= tile.valid) return;
  const GGOperandsF8& ops = in_dense ? dense : routed;
  bf16_t* const C = ops.base.C;
  const int n0 = nt * kOutCols;
  // The item's pieces, in slice order: the slots of the work groups whose ranges
  // [q S / G, (q+1) S / G) overlap its slices [a, b) (S = R nk <= 256 * 1024, so the
  // products stay within 32 bits), listed once by thread 0.
  if (tid == 0) {
    const int S = R * nk;
    const int a = r * nk, b = a + nk;
    int q = a / (S / G + 1);              // a start; the loops find the first overlap
    while (q > 0 && q * S / G > a) --q;
    while ((q + 1) * S / G <= a) ++q;
    int n = 0;
    for (; q < G && n < kMaxPieces; ++q) {
      const int lo = q * S / G, hi = (q + 1) * S / G;
      if (lo >= b) break;
      if (hi <= lo) continue;
      s_slot[n++] = 2 * q + (lo >= a ? 0 : 1);   // its first piece, or its second
    }
    s_npieces = n;
  }
  __syncthreads();
  const int np = s_npieces;
  const int c = tid * 4;                  // this thread's first column of the item
  if (c >= kOutCols) return;
  const float* base = tail + kDTailHeader;
  for (int row = blockIdx.y; row < tile.valid; row += gridDim.y) {
    const size_t roff = (size_t)row * kDTailCols + c;
    tail_f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < np; p0 += 4) {
      tail_f32x4 vg[4], vu[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (p0 + t < np) {
          const float* prow = base + (size_t)s_slot[p0 + t] * (kDTailSlot / 4) + roff;
          vg[t] = *reinterpret_cast<const tail_f32x4*>(prow);
          if (GU) vu[t] = *reinterpret_cast<const tail_f32x4*>(prow + 512);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (p0 + t < np) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            g[i] += vg[t][i];
            if (GU) u[i] += vu[t][i];
          }
        }
      }
    }
    bf16_t* crow = C + (size_t)(tile.m0 + row) * N + n0 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n0 + c + i < N) crow[i] = f32_to_bf16(GU ? silu_f32(g[i]) * u[i] : g[i]);
  }
}

bool fp8_gemm_supported(int K, int N) {
  return K % kFBK == 0 && N % 16 == 0 && ceil_div(K, kQBlock) <= kFMaxKB;
}

moe_status launch_grouped_gemm_fp8(int op, const GemmSegmentsF8& g, int E, int64_t max_rows,
                                   Fp8Kernel kind, hipStream_t st) {
  const bool routed = g.max_blocks > 0, dense = g.dense_rows > 0;
  if (!routed && !dense) return MOE_OK;
  // MOE_FP8_ITEM_ROWS=64, 128 or 384 forces one kernel (tests run each on the same
  // shapes; 384 needs a block table of at most wide_max_blocks() entries)
  if (const char* f = getenv("MOE_FP8_ITEM_ROWS")) {
    if (strcmp(f, "64") == 0) kind = kFp8Rows64;
    if (strcmp(f, "128") == 0) kind = kFp8Rows128;
    if (strcmp(f, "384") == 0 && g.max_blocks <= wide_max_blocks()) kind = kFp8Wide;
  }
  // the 64-row kernel streams consecutive items' slices through its ring: K >= 4 slices
  if (kind == kFp8Rows64 && g.K / kFBK < kDStages) kind = kFp8Rows128;
  const bool few_rows = kind == kFp8Rows64;
  if (kind == kFp8Wide) {
    GGOperands ro{static_cast<const bf16_t*>(g.A), reinterpret_cast<const bf16_t*>(g.Q0),
                  reinterpret_cast<const bf16_t*>(g.Q1), static_cast<bf16_t*>(g.C), g.gather,
                  g.gather_div, g.gather_rows, nullptr};
    ro.S0 = g.S0;
    ro.S1 = g.S1;
    GGOperands dn{static_cast<const bf16_t*>(g.Ad), reinterpret_cast<const bf16_t*>(g.Q0d),
                  reinterpret_cast<const bf16_t*>(g.Q1d), static_cast<bf16_t*>(g.Cd), nullptr, 1, 1,
                  nullptr};
    dn.S0 = g.S0d;
    dn.S1 = g.S1d;
    return launch_gg_wide(op, ro, dn, g.K, g.N, g.block_meta, g.num_blocks,
                          routed ? g.max_blocks : 0, max_rows, E, g.dense_rows, st, true);
  }
  const GGOperandsF8 rd{{static_cast<const bf16_t*>(g.A), nullptr, nullptr, static_cast<bf16_t*>(g.C),
                         g.gather, g.gather_div, g.gather_rows},
                        g.Q0, g.Q1, g.S0, g.S1};
  const GGOperandsF8 dd{{static_cast<const bf16_t*>(g.Ad), nullptr, nullptr, static_cast<bf16_t*>(g.Cd),
                         nullptr, 1, 1},
                        g.Q0d, g.Q1d, g.S0d, g.S1d};
  if (few_rows) {
    const int n_tiles = (int)ceil_div(g.N, op == MOE_OP_GATEUP_SWIGLU ? 512 : 1024);
    const int64_t blocks_ub = (routed ? (int64_t)g.max_blocks : 0) +
                              (dense ? ceil_div(g.dense_rows, 128) : 0);
    const int64_t items = blocks_ub * 2 * n_tiles;
    const int cus = device_cu_count();
    int64_t grid = items < cus ? items : cus;
    if (grid < 1) grid = 1;
    // the last round splits along K only with scratch, a grid of at most kDTailGrid work
    // groups and (decided on the device) a table whose blocks hold at most 64 rows;
    // MOE_FP8D_TAIL=0 turns it off
    float* tail = grid <= kDTailGrid ? g.tail : nullptr;
    if (const char* f = getenv("MOE_FP8D_TAIL"))
      if (strcmp(f, "0") == 0) tail = nullptr;
    if (op == MOE_OP_GATEUP_SWIGLU)
      hipLaunchKernelGGL(k_gg_fp8d<MOE_OP_GATEUP_SWIGLU>, dim3((unsigned)grid), dim3(kFThreads), 0,
                         st, rd, dd, g.K, g.N, g.block_meta, g.num_blocks, g.max_blocks, E,
                         max_rows, g.dense_rows, n_tiles, tail);
    else
      hipLaunchKernelGGL(k_gg_fp8d<MOE_OP_DOWN>, dim3((unsigned)grid), dim3(kFThreads), 0, st, rd,
                         dd, g.K, g.N, g.block_meta, g.num_blocks, g.max_blocks, E, max_rows,
                         g.dense_rows, n_tiles, tail);
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
    if (tail) {
      const int G = (int)grid;
      const dim3 tgrid((unsigned)G, kDTailRowGroups);
      if (op == MOE_OP_GATEUP_SWIGLU)
        hipLaunchKernelGGL(k_fp8d_tail<MOE_OP_GATEUP_SWIGLU>, tgrid, dim3(256), 0, st, rd, dd, g.K,
                           g.N, g.block_meta, g.num_blocks, g.max_blocks, E, max_rows, g.dense_rows,
                           n_tiles, G, tail);
      else
        hipLaunchKernelGGL(k_fp8d_tail<MOE_OP_DOWN>, tgrid, dim3(256), 0, st, rd, dd, g.K, g.N,
                           g.block_meta, g.num_blocks, g.max_blocks, E, max_rows, g.dense_rows,
                           n_tiles, G, tail);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  const int out_cols = op == MOE_OP_GATEUP_SWIGLU ? 256 : 512;
  const int n_tiles = (int)ceil_div(g.N, out_cols);
  const int64_t blocks_ub = (routed ? (int64_t)g.max_blocks : 0) + (dense ? ceil_div(g.dense_rows, 128) : 0);
  const int64_t items = blocks_ub * n_tiles;
  const int cus = device_cu_count();
  int64_t grid = items < cus ? items : cus;
  if (grid < 1) grid = 1;
  const GGOperandsF8 ro{{static_cast<const bf16_t*>(g.A), nullptr, nullptr, static_cast<bf16_t*>(g.C),
                         g.gather, g.gather_div, g.gather_rows},
                        g.Q0, g.Q1, g.S0, g.S1};
  const GGOperandsF8 dn{{static_cast<const bf16_t*>(g.Ad), nullptr, nullptr, static_cast<bf16_t*>(g.Cd),
                         nullptr, 1, 1},
                        g.Q0d, g.Q1d, g.S0d, g.S1d};
  if (op == MOE_OP_GATEUP_SWIGLU)
    hipLaunchKernelGGL(k_gg_fp8w<MOE_OP_GATEUP_SWIGLU>, dim3((unsigned)grid), dim3(kFThreads), 0, st,
                       ro, dn, g.K, g.N, g.block_meta, g.num_blocks, g.max_blocks, E, max_rows,
                       g.dense_rows, n_tiles);
  else
    hipLaunchKernelGGL(k_gg_fp8w<MOE_OP_DOWN>, dim3((unsigned)grid), dim3(kFThreads), 0, st, ro, dn,
                       g.K, g.N, g.block_meta, g.num_blocks, g.max_blocks, E, max_rows,
                       g.dense_rows, n_tiles);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
