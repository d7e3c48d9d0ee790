// Device-side pieces shared by the bf16 grouped-GEMM kernels (not part of the ABI).
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define MOE_LDS __attribute__((address_space(3)))

// s_waitcnt with vmcnt <= n and the other counters unconstrained (gfx9 encoding).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 16-byte asynchronous copy global -> LDS: lane l reads gbase + voff_bytes[l] and its
// 16 bytes land at lds_base + 16*l (gbase and lds_base are wave-uniform; lds_base
// goes through M0).  Issued as inline assembly so the compiler's own counter model
// does not see it: it would otherwise wait for every outstanding copy before each
// LDS read.  The caller waits with MOE_WAIT_VMCNT; loads complete in issue order, so
// compiler-generated waits stay correct (they can only over-wait).
__device__ __forceinline__ void copy16_to_lds(const void* gbase, uint32_t voff_bytes,
                                              const unsigned char* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const MOE_LDS void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff_bytes), "s"(gbase), "s"(m0)
               : "memory", "m0");
}

// The same copy as a group: set_lds_dma_base() loads M0 once, then each
// copy16_to_lds_at<OFF>() lands at M0 + OFF + 16*l and reads gbase + voff_bytes[l] + OFF
// (the instruction's immediate offset applies to both addresses on gfx950).  Nothing
// else in these kernels writes M0.
__device__ __forceinline__ void set_lds_dma_base(const unsigned char* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const MOE_LDS void*)lds_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(m0) : "memory", "m0");
}
template <int OFF>
__device__ __forceinline__ void copy16_to_lds_at(const void* gbase, uint32_t voff_bytes) {
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2"
               :
               : "v"(voff_bytes), "s"(gbase), "n"(OFF)
               : "memory");
}
// copy i of a group (i < 4): immediate offset 1024 * i
__device__ __forceinline__ void copy16_to_lds_nth(int i, const void* gbase, uint32_t voff_bytes) {
  switch (i) {
    case 0: copy16_to_lds_at<0>(gbase, voff_bytes); break;
    case 1: copy16_to_lds_at<1024>(gbase, voff_bytes); break;
    case 2: copy16_to_lds_at<2048>(gbase, voff_bytes); break;
    default: copy16_to_lds_at<3072>(gbase, voff_bytes); break;
  }
}

__device__ __forceinline__ int swz_a(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }
__device__ __forceinline__ int swz_b(int k, int chunk) { return chunk ^ (4 * (k & 3)); }

// Operands of one segment set: A rows, the B matrices (expert-strided) and C rows.
// gather != nullptr: row r of the segment reads A row gather[r] / gather_div (the
// permutation fused into the A loads; A is then the unpermuted [gather_rows, K]
// input; a row index outside it is clamped, so a corrupt table cannot read past A).
struct GGOperands {
  const bf16_t* A;
  const bf16_t* B0;
  const bf16_t* B1;
  bf16_t* C;
  const int32_t* gather;
  int gather_div;
  int gather_rows;
  // kOpGateUpBwd only: dact [rows, N]; C is then dg | du, [rows, 2 N]
  const bf16_t* D;
  // fp8 weights (the wide kernel's fp8 variant): B0 / B1 then point at e4m3 codes
  // [E][K][N] and these at their fp32 scales [E][ceil(K/128)][ceil(N/128)]
  const float* S0 = nullptr;
  const float* S1 = nullptr;
};

// SwiGLU backward of one element from the recomputed gate g, up u and the incoming
// gradient da of act = silu(g) u:  dg = da u silu'(g),  du = da silu(g),
// silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
__device__ __forceinline__ float swiglu_dgate(float g, float u, float da) {
  const float s = sigmoid_f32(g);
  return da * u * (s * (1.0f + g * (1.0f - s)));
}
__device__ __forceinline__ float swiglu_dup(float g, float da) { return da * silu_f32(g); }

// A wave-uniform pointer, held in scalar registers (the copies take an SGPR base).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int gather_row(const GGOperands& ops, int r) {
  const int src = ops.gather[r] / ops.gather_div;
  if (src < 0 || src >= ops.gather_rows) MOE_DEBUG_REPORT(MOE_DBG_GATHER_ROW);
  return min(max(src, 0), ops.gather_rows - 1);
}

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
  // a table entry that does not fit the expert range or the row buffers is skipped (an
  // entry without rows runs nothing either way)
  const bool bad = e < 0 || e >= E || m_start < 0 || vm > block_m || (int64_t)m_start + vm > max_rows;
  if (bad || vm < 1) MOE_DEBUG_REPORT(MOE_DBG_BLOCK_TABLE);
  if (bad) return false;
  return t.valid > 0;
}

// Wide-tile kernel (moe_gemm_wide.hip): 384-row groups of one expert's blocks x 256
// B-columns, for block_m == 128, K % 32 == 0 and max_blocks <= wide_max_blocks().
int wide_max_blocks();
// fp8: B0 / B1 of both operand sets are e4m3 codes with scales S0 / S1 (forward ops).
moe_status launch_gg_wide(int op, const GGOperands& ro, const GGOperands& dn, int K, int N,
                          const int32_t* block_meta, const int32_t* num_blocks, int32_t max_blocks,
                          int64_t max_rows, int E, int32_t dense_rows, hipStream_t st,
                          bool fp8 = false);

}  // namespace moe
