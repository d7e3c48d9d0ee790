// Internal declarations shared by the HIP sources of libmoe (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

// Internal grouped-GEMM op next to MOE_OP_GATEUP_SWIGLU and MOE_OP_DOWN: recompute the
// gate/up products and apply the SwiGLU backward in the epilogue.
constexpr int kOpGateUpBwd = 2;

// bf16 <-> fp32.  The widening is exact; the narrowing rounds to nearest even
// (gfx950 converts in hardware).
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}
// Two floats -> two packed bf16 in one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Load/store helpers for the two element types, going through fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// sigmoid(z) = 1 / (1 + e^-z) in fp32 from the hardware's base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each): e^-z = 2^(-z log2 e).  Five
// instructions instead of the ~25 of a correctly rounded expf and an IEEE division,
// which dominated the gate/up epilogues (96 values per lane per item); the error stays
// near 1e-6 relative, far below the bf16 rounding of every output.  Below z ~ -88 the
// power overflows to +inf and the reciprocal gives the limit 0.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}
// SiLU in fp32: z * sigmoid(z).
__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_f32(z); }

// ---- debug builds (-DMOE_DEBUG) ---------------------------------------------------
// Where a kernel skips or clamps an index it cannot use, MOE_DEBUG_REPORT(bits) ORs
// MOE_DBG_* bits into this translation unit's word on the device (each source file of
// the library has its own; moe_debug_flags reads all of them).  Release builds compile
// the reports away, leaving the checks themselves as they are.
#ifdef MOE_DEBUG
static __device__ uint32_t g_debug_word;
__device__ __forceinline__ void debug_report(uint32_t bits) { atomicOr(&g_debug_word, bits); }
#define MOE_DEBUG_REPORT(bits) ::moe::debug_report(bits)
// Registers a reader of one unit's word; moe_debug_flags calls every registered reader.
int debug_register(moe_status (*read)(uint32_t* acc, bool clear));
static moe_status debug_read_unit(uint32_t* acc, bool clear) {
  uint32_t w = 0;
  if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_debug_word), sizeof w) != hipSuccess) return MOE_EHIP;
  *acc |= w;
  const uint32_t zero = 0;
  if (clear && hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof zero) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}
[[maybe_unused]] static const int g_debug_registered = debug_register(&debug_read_unit);
#else
#define MOE_DEBUG_REPORT(bits) ((void)0)
#endif

// The block count a kernel runs: *num_blocks, clamped into [0, max_blocks] (the host's
// bound sizes the launch and the buffers).
__device__ __forceinline__ int clamp_block_count(const int32_t* num_blocks, int max_blocks) {
  const int n = num_blocks[0];
  if (n < 0 || n > max_blocks) MOE_DEBUG_REPORT(MOE_DBG_BLOCK_COUNT);
  return max(0, min(n, max_blocks));
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of compute units of the current device (queried once per device).
int device_cu_count();

// Rows of the permuted buffers that a block table of max_blocks entries addresses:
// max_blocks * block_m in the padded layout, the T*k rows in the unpadded one.
inline int64_t routed_rows_bound(const moe_shape& s, int64_t max_blocks) {
  return s.unpadded ? (int64_t)s.T * s.k : max_blocks * s.block_m;
}

// ---- launchers (each returns MOE_OK or MOE_EHIP) -------------------------------
// Router: partial logits over nsplit slices of d, then selection.
int router_nsplit(const moe_shape& s);
size_t router_partial_bytes(const moe_shape& s);
moe_status launch_route(const moe_shape& s, const void* x, const void* w_gate,
                        const float* bias, float* logits, int32_t* topk_idx,
                        float* topk_w, float* partial, hipStream_t st);

// Offsets: per-chunk histograms + ranks, one-block scan + metadata, scatter.
int offsets_chunk(const moe_shape& s);
int64_t offsets_nchunks(const moe_shape& s);
size_t offsets_scratch_bytes(const moe_shape& s);
// The offsets kernels' scratch as a file-scope device array (moe_build_offsets_noalloc):
// its size, and its address on the current device (looked up once per device).
size_t static_scratch_capacity();
moe_status static_scratch_address(void** out);
moe_status launch_build_offsets(const moe_shape& s, const int32_t* topk_idx,
                                int32_t* counts, int32_t* offsets, int32_t* padded,
                                int32_t* block_meta, int32_t* num_blocks, int32_t* pos,
                                int32_t* row_src, int32_t* err_flag, void* scratch,
                                hipStream_t st);

moe_status launch_permute(const moe_shape& s, const void* x, const int32_t* pos,
                          void* x_perm, hipStream_t st);
moe_status launch_combine(const moe_shape& s, const void* y, const int32_t* pos,
                          const float* topk_w, const void* shared_out, void* out,
                          hipStream_t st);  // topk_w NULL: unit weights

// Grouped GEMM over up to two segment sets with their own operands: the routed
// segments of a block table (max_blocks == 0: none) and a dense segment of
// dense_rows rows through a single expert (the shared expert; dense_rows == 0:
// none).  bf16 sets with the same K and N (K % 32 == 0) share one launch.
struct GemmSegments {
  const void* A;
  const void* B0;
  const void* B1;
  void* C;
  int K, N;
  const int32_t* block_meta;
  const int32_t* num_blocks;
  int32_t max_blocks;
  const void* Ad;
  const void* B0d;
  const void* B1d;
  void* Cd;
  int Kd, Nd;
  int32_t dense_rows;
  // routed rows gather their A rows: row r reads A row gather[r] / gather_div
  // (nullptr: A is already permuted); needs gather_supported()
  const int32_t* gather;
  int gather_div;
  int gather_rows;  // rows of the unpermuted A (row indices are clamped into it)
  // kOpGateUpBwd: the incoming gradient dact of the routed and dense sets
  const void* D;
  const void* Dd;
};
moe_status launch_grouped_gemm(const moe_shape& s, int op, const GemmSegments& g, hipStream_t st);
// The bf16 asynchronous-copy kernels can gather gate/up A rows from the unpermuted x.
bool gather_supported(const moe_shape& s);

// fp8 (e4m3) weights with fp32 scales per 128 x 128 block (moe_fp8.hip).
moe_status launch_quantize_fp8(int E, int K, int N, const void* w, uint8_t* q, float* scales,
                               hipStream_t st);
// bf16 weights from codes and scales, bit-identical to the fp8 GEMM's own dequantisation.
moe_status launch_dequantize_fp8(int E, int K, int N, const uint8_t* q, const float* scales,
                                 void* w, hipStream_t st);
// The fp8-weight grouped GEMM applies to this K (contraction) and N.
bool fp8_gemm_supported(int K, int N);
struct GemmSegmentsF8 {
  const void* A;
  const uint8_t* Q0;
  const float* S0;
  const uint8_t* Q1;
  const float* S1;
  void* C;
  int K, N;
  const int32_t* block_meta;
  const int32_t* num_blocks;
  int32_t max_blocks;
  // dense segment (the shared expert): same K and N, rows of Ad
  const void* Ad;
  const uint8_t* Q0d;
  const float* S0d;
  const uint8_t* Q1d;
  const float* S1d;
  void* Cd;
  int32_t dense_rows;
  // routed rows gathered from A (as GemmSegments::gather)
  const int32_t* gather;
  int gather_div;
  int gather_rows;
  // scratch of fp8_tail_scratch_bytes() for the 64-row kernel's split last round, or NULL
  float* tail;
};
// Scratch that lets the 64-row fp8 kernel split its last round along K.
size_t fp8_tail_scratch_bytes();
// Which fp8 grouped-GEMM kernel runs: 64-row items with wide weight rows (experts
// average at most 64 rows: weight streaming), 128-row items, or the wide bf16 kernel's
// 384-row groups with in-register dequantisation (experts average at least 256 rows).
enum Fp8Kernel { kFp8Rows64 = 0, kFp8Rows128 = 1, kFp8Wide = 2 };
// Block-table limit of the wide kernel (moe_gemm_wide.hip).
int wide_max_blocks();
moe_status launch_grouped_gemm_fp8(int op, const GemmSegmentsF8& g, int E, int64_t max_rows,
                                   Fp8Kernel kind, hipStream_t st);

// Backward kernels (moe_backward.hip).
// dy[pos[t,j]] = w[t,j] dout[t] (bf16), dw[t,j] = <dout[t], y[pos[t,j]]> (fp32); d <= 8192.
moe_status launch_combine_bwd(const moe_shape& s, const void* dout, const void* y,
                              const int32_t* pos, const float* topk_w, void* dy, float* dw,
                              int64_t max_rows, hipStream_t st);
// C[r] = A[r] B[e] with B stored transposed per expert: B[k][n] = Bt0[e][n][k] for
// k < ksplit, Bt1[e][n][k - ksplit] beyond (Bt1 NULL: ksplit = K); K % 32 == 0,
// ksplit % 32 == 0, N % 8 == 0.  Routed rows from the block table, or dense_rows rows
// of one matrix.
moe_status launch_gg_nt(const void* A, const void* Bt0, const void* Bt1, int ldb, int ksplit,
                        void* C, int K, int N, const int32_t* meta, const int32_t* num_blocks,
                        int32_t max_blocks, int E, int block_m, int64_t max_rows,
                        int32_t dense_rows, hipStream_t st);
// wt[e][c][r] = w[e][r][c] (bf16; R % 8 == 0, C % 8 == 0): wt's expert e starts at
// e * wt_estride elements and its rows are wt_ld elements apart.
moe_status launch_transpose_bf16(int E, int R, int C, const void* w, void* wt, int64_t wt_estride,
                                 int wt_ld, hipStream_t st);
// C[e] = X_e^T D_e (fp32) over expert e's rows [row_off[e], row_off[e] + counts[e]),
// columns n < nsplit into C0 [E][Km][nsplit], the rest into C1 (C1 NULL: nsplit = Nn);
// dense_rows > 0: one expert over rows [0, dense_rows); counts NULL and dense_rows 0:
// zeros.  Km % 8 == 0, Nn % 8 == 0.
// sched: NULL, or wgrad_sched_bytes(E) bytes of device scratch: the routed experts' items
// then go through a work queue, largest expert first.
moe_status launch_gg_wgrad(const void* X, const void* D, float* C0, float* C1, int nsplit, int Km,
                           int Nn, const int32_t* counts, const int32_t* row_off, int E,
                           int32_t dense_rows, void* sched, hipStream_t st);
size_t wgrad_sched_bytes(int E);
// dlogits from dw through the softmax (and renormalisation), selection fixed; then
// dw_gate = x^T dlogits, dbias = column sums (either NULL: skipped), and
// dx_out = dx_base (NULL: 0) + dlogits w_gate^T in bf16.  scratch: router_bwd_scratch_bytes
// (the per-chunk partial sums of dw_gate and dbias).
size_t router_bwd_scratch_bytes(const moe_shape& s);
moe_status launch_router_bwd(const moe_shape& s, const void* x, const void* w_gate,
                             const float* logits, const int32_t* idx, const float* dw,
                             float* dlogits, float* dw_gate, float* dbias, const void* dx_base,
                             void* dx_out, void* scratch, hipStream_t st);

}  // namespace moe
