// C ABI of libmoe: argument validation, workspace layout and the layer pipeline.
//
// Every entry point validates its arguments on the host and returns a status before
// anything is enqueued; kernels then run on the caller's stream.  Nothing here
// allocates, frees or synchronises, and no value travels from device to host: the
// grouped GEMM is launched with a grid derived from the static upper bound
// moe_max_blocks, and reads the real block count from device memory (dropless notes
// section 7: the host only needs to know how much work to launch, not the shapes).
#include "moe_internal.h"

#include <atomic>

namespace moe {

static constexpr int kMaxDevices = 64;
static std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static int elem_bytes(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// Shape checks common to every call.  Returns MOE_OK, MOE_EINVAL or MOE_ENOTSUP.
static moe_status check_shape(const moe_shape* sp) {
  if (!sp) return MOE_EINVAL;
  const moe_shape& s = *sp;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_EINVAL;
  const int mult = s.dtype == MOE_DTYPE_BF16 ? 8 : 4;  // 16-byte rows
  if (s.T < 0 || s.d < 1 || s.E < 1 || s.k < 1 || s.d_e < 1) return MOE_EINVAL;
  if (s.d % mult || s.d_e % mult) return MOE_EINVAL;
  if (s.k > 1024) return MOE_ENOTSUP;
  if (s.E > 1024) return MOE_ENOTSUP;
  if ((int64_t)s.T * s.k >= (int64_t)1 << 31) return MOE_EINVAL;
  if (s.n_groups < 0 || s.topk_groups < 0) return MOE_EINVAL;
  if (s.n_groups == 0) {
    if (s.topk_groups != 0) return MOE_EINVAL;
  } else {
    if (s.E % s.n_groups) return MOE_EINVAL;
    if (s.topk_groups < 1 || s.topk_groups > s.n_groups) return MOE_EINVAL;
    if (s.n_groups > 64) return MOE_ENOTSUP;
  }
  if (s.renormalize != 0 && s.renormalize != 1) return MOE_EINVAL;
  if (s.unpadded != 0 && s.unpadded != 1) return MOE_EINVAL;
  if (s.block_m < 1) return MOE_EINVAL;
  if (s.d_e_shared < 0 || (s.d_e_shared % mult)) return MOE_EINVAL;
  if (s.dtype == MOE_DTYPE_BF16 && s.block_m % 128) return MOE_ENOTSUP;
  // one expert matrix is indexed with 32-bit element offsets
  const int64_t de_max = s.d_e > s.d_e_shared ? s.d_e : s.d_e_shared;
  if ((int64_t)s.d * de_max >= (int64_t)1 << 31) return MOE_ENOTSUP;
  // the tiles of the block table must stay addressable with int32 row indices: those of
  // the padded layout and, unpadded, those of its own table (ceil(T*k / block_m) tiles
  // plus up to E - 1 entries for tiles shared by two experts)
  const int64_t M = (int64_t)s.T * s.k;
  const int64_t ne = M < s.E ? M : s.E;
  const int64_t mb = (M + ne * (s.block_m - 1)) / s.block_m;
  if (mb * s.block_m >= (int64_t)1 << 31) return MOE_EINVAL;
  if (s.unpadded && M > 0 && (ceil_div(M, s.block_m) + ne - 1) * s.block_m >= (int64_t)1 << 31)
    return MOE_EINVAL;
  return MOE_OK;
}

// The router picks k distinct experts, so it needs k <= E (and, with group-limited
// routing, k <= topk_groups * E / n_groups).  Rows that arrive already routed may
// repeat an expert within a token, so the other stages accept any k.
static moe_status check_routing(const moe_shape& s) {
  if (s.k > s.E) return MOE_EINVAL;
  if (s.n_groups > 0 && (int64_t)s.k > (int64_t)s.topk_groups * (s.E / s.n_groups))
    return MOE_EINVAL;
  return MOE_OK;
}

static int64_t max_blocks_of(const moe_shape& s) {
  const int64_t M = (int64_t)s.T * s.k;
  const int64_t ne = M < s.E ? M : s.E;
  // unpadded: one entry per tile plus one per expert boundary inside a tile
  if (s.unpadded) return M == 0 ? 0 : ceil_div(M, s.block_m) + ne - 1;
  return (M + ne * (s.block_m - 1)) / s.block_m;
}

// Rows of every permuted buffer (x_perm, act, y, row_src).
static int64_t max_rows_of(const moe_shape& s) { return routed_rows_bound(s, max_blocks_of(s)); }

static size_t take(size_t& cur, size_t bytes) {
  const size_t off = cur;
  cur = align_up(cur + bytes, 256);
  return off;
}

static void layout_of(const moe_shape& s, moe_ws_layout& L) {
  const size_t b = elem_bytes(s);
  const size_t T = s.T, E = s.E, M = (size_t)s.T * s.k;
  const size_t mb = (size_t)max_blocks_of(s);
  const size_t rows = (size_t)max_rows_of(s);
  size_t cur = 0;
  L.logits = take(cur, T * E * 4);
  L.topk_idx = take(cur, M * 4);
  L.topk_w = take(cur, M * 4);
  L.counts = take(cur, E * 4);
  L.offsets = take(cur, (E + 1) * 4);
  L.padded_offsets = take(cur, (E + 1) * 4);
  L.block_meta = take(cur, mb * 3 * 4);
  L.num_blocks = take(cur, 4);
  L.pos = take(cur, M * 4);
  L.row_src = take(cur, rows * 4);
  L.err_flag = take(cur, 4);
  // where the permute is fused into the gate/up loads x_perm is never written
  L.x_perm = take(cur, gather_supported(s) ? 0 : rows * s.d * b);
  L.act = take(cur, rows * s.d_e * b);
  L.y = take(cur, rows * s.d * b);
  L.shared_act = take(cur, s.d_e_shared ? T * s.d_e_shared * b : 0);
  L.shared_out = take(cur, s.d_e_shared ? T * s.d * b : 0);
  const size_t rp = router_partial_bytes(s), os = offsets_scratch_bytes(s);
  L.scratch = take(cur, rp > os ? rp : os);
  L.total = cur;
}

// The layer's backward runs its data gradients on the forward grouped-GEMM kernels,
// against weights transposed once per call, where experts average at least 256 rows
// (where the wide forward kernel applies); otherwise k_gg_nt reads them transposed.
static bool transposed_dgrad(const moe_shape& s) {
  const int64_t M = (int64_t)s.T * s.k;
  return M > 0 && M >= 256 * (M < s.E ? M : (int64_t)s.E);
}

// The backward kernels: bf16, contraction sizes in whole 32-deep slices.
static moe_status check_bwd(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16) return MOE_ENOTSUP;
  if (s.d % 32 || s.d_e % 32 || s.d_e_shared % 32) return MOE_ENOTSUP;
  return MOE_OK;
}

static void bwd_layout_of(const moe_shape& s, moe_bwd_ws_layout& L) {
  const size_t T = s.T, E = s.E, M = (size_t)s.T * s.k;
  const size_t rows = (size_t)max_rows_of(s);
  const size_t d = s.d, de = s.d_e, ds = s.d_e_shared;
  size_t cur = 0;
  L.dy = take(cur, rows * d * 2);
  L.dact = take(cur, rows * de * 2);
  L.dgu = take(cur, rows * 2 * de * 2);
  L.x_perm = take(cur, rows * d * 2);
  L.dx_perm = take(cur, rows * d * 2);
  L.dtopk_w = take(cur, M * 4);
  L.dlogits = take(cur, T * E * 4);
  L.shared_dact = take(cur, T * ds * 2);
  L.shared_dgu = take(cur, T * 2 * ds * 2);
  L.shared_dx = take(cur, ds ? T * d * 2 : 0);
  L.router_dx = take(cur, T * d * 2);
  L.router_scratch = take(cur, router_bwd_scratch_bytes(s));
  L.wgrad_sched = take(cur, wgrad_sched_bytes(s.E));
  // the expert weights transposed for the data gradients, when the forward kernels run
  // them (transposed_dgrad)
  const bool tw = transposed_dgrad(s);
  L.w2_t = take(cur, tw ? E * d * de * 2 : 0);
  L.w13_t = take(cur, tw ? E * 2 * de * d * 2 : 0);
  L.ws2_t = take(cur, tw ? d * ds * 2 : 0);
  L.ws13_t = take(cur, tw ? 2 * ds * d * 2 : 0);
  L.total = cur;
}

#ifdef MOE_DEBUG
// The debug word readers of the library's source files, registered while the library
// loads (zero-initialised storage, so the order of the units' initialisers is free).
static moe_status (*g_debug_readers[16])(uint32_t*, bool);
static int g_debug_nreaders;
int debug_register(moe_status (*read)(uint32_t*, bool)) {
  if (g_debug_nreaders < 16) g_debug_readers[g_debug_nreaders++] = read;
  return g_debug_nreaders;
}
#endif

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_debug_flags(uint32_t* flags, int32_t clear) {
  if (!flags) return MOE_EINVAL;
  *flags = 0;
#ifdef MOE_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
  for (int i = 0; i < g_debug_nreaders; ++i) {
    const moe_status st = g_debug_readers[i](flags, clear != 0);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
#else
  (void)clear;
  return MOE_ENOTSUP;
#endif
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOTSUP: return "not supported";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t moe_max_blocks(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return -1;
  return (int32_t)max_blocks_of(*s);
}

int64_t moe_max_rows(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return -1;
  return max_rows_of(*s);
}

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  moe_ws_layout L;
  layout_of(*s, L);
  return L.total;
}

moe_status moe_workspace_layout(const moe_shape* s, moe_ws_layout* layout) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!layout) return MOE_EINVAL;
  layout_of(*s, *layout);
  return MOE_OK;
}

moe_status moe_route(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                     float* logits, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_routing(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !topk_idx || !topk_w) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned4(topk_idx) || !aligned4(topk_w) ||
      (bias && !aligned4(bias)) || (logits && !aligned4(logits)))
    return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (!ws || !aligned16(ws) || ws_bytes < router_partial_bytes(*s)) return MOE_EWORKSPACE;
  return launch_route(*s, x, w_gate, bias, logits, topk_idx, topk_w, static_cast<float*>(ws),
                      static_cast<hipStream_t>(stream));
}

moe_status moe_build_offsets(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                             int32_t* offsets, int32_t* padded_offsets, int32_t* block_meta,
                             int32_t* num_blocks, int32_t* pos, int32_t* row_src,
                             int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const void* ptrs[] = {topk_idx, counts, offsets, padded_offsets, block_meta,
                        num_blocks, pos, row_src, err_flag};
  for (const void* p : ptrs)
    if (!p || !aligned4(p)) return MOE_EINVAL;
  if (!ws || !aligned16(ws) || ws_bytes < offsets_scratch_bytes(*s)) return MOE_EWORKSPACE;
  return launch_build_offsets(*s, topk_idx, counts, offsets, padded_offsets, block_meta, num_blocks,
                              pos, row_src, err_flag, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_build_offsets_noalloc(const moe_shape* s, const int32_t* topk_idx,
                                     int32_t* counts, int32_t* offsets, int32_t* padded_offsets,
                                     int32_t* block_meta, int32_t* num_blocks, int32_t* pos,
                                     int32_t* row_src, int32_t* err_flag, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const void* ptrs[] = {topk_idx, counts, offsets, padded_offsets, block_meta,
                        num_blocks, pos, row_src, err_flag};
  for (const void* p : ptrs)
    if (!p || !aligned4(p)) return MOE_EINVAL;
  if (offsets_scratch_bytes(*s) > static_scratch_capacity()) return MOE_ENOTSUP;
  void* scratch = nullptr;
  if ((st = static_scratch_address(&scratch)) != MOE_OK) return st;
  return launch_build_offsets(*s, topk_idx, counts, offsets, padded_offsets, block_meta, num_blocks,
                              pos, row_src, err_flag, scratch, static_cast<hipStream_t>(stream));
}

size_t moe_build_offsets_noalloc_capacity(void) { return static_scratch_capacity(); }

size_t moe_build_offsets_scratch_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return offsets_scratch_bytes(*s);
}

moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* pos, void* x_perm,
                       void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!x || !pos || !x_perm || !aligned16(x) || !aligned16(x_perm) || !aligned4(pos))
    return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  return launch_permute(*s, x, pos, x_perm, static_cast<hipStream_t>(stream));
}

// operand rules shared by the grouped-GEMM entry points
static bool gemm_operands_ok(int32_t op, const void* A, const void* B0, const void* B1,
                             const void* C) {
  if (!A || !B0 || !C) return false;
  if (op == MOE_OP_GATEUP_SWIGLU && !B1) return false;
  if (op == MOE_OP_DOWN && B1) return false;
  return aligned16(A) && aligned16(B0) && (!B1 || aligned16(B1)) && aligned16(C);
}

static bool block_table_ok(const moe_shape& s, const int32_t* block_meta,
                           const int32_t* num_blocks, int32_t max_blocks) {
  return block_meta && num_blocks && aligned4(block_meta) && aligned4(num_blocks) &&
         max_blocks >= 1 && max_blocks <= max_blocks_of(s);
}

moe_status moe_grouped_gemm(const moe_shape* s, int32_t op, const void* A, const void* B0,
                            const void* B1, const int32_t* block_meta, const int32_t* num_blocks,
                            int32_t max_blocks, void* C, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return MOE_EINVAL;
  if (!gemm_operands_ok(op, A, B0, B1, C)) return MOE_EINVAL;
  const int K = op == MOE_OP_GATEUP_SWIGLU ? s->d : s->d_e;
  const int N = op == MOE_OP_GATEUP_SWIGLU ? s->d_e : s->d;
  GemmSegments g{};
  if (!block_meta && !num_blocks) {  // dense mode: one expert over all T rows
    if (max_blocks != 0) return MOE_EINVAL;
    if (s->T == 0) return MOE_OK;
    g.Ad = A; g.B0d = B0; g.B1d = B1; g.Cd = C; g.Kd = K; g.Nd = N; g.dense_rows = s->T;
  } else {
    if (!block_table_ok(*s, block_meta, num_blocks, max_blocks)) return MOE_EINVAL;
    g.A = A; g.B0 = B0; g.B1 = B1; g.C = C; g.K = K; g.N = N;
    g.block_meta = block_meta; g.num_blocks = num_blocks; g.max_blocks = max_blocks;
  }
  return launch_grouped_gemm(*s, op, g, static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_gemm_shared(const moe_shape* s, int32_t op, const void* A, const void* B0,
                                   const void* B1, const int32_t* block_meta,
                                   const int32_t* num_blocks, int32_t max_blocks, void* C,
                                   const void* A_shared, const void* B0_shared,
                                   const void* B1_shared, void* C_shared, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return MOE_EINVAL;
  if (s->d_e_shared <= 0) return MOE_EINVAL;
  if (!gemm_operands_ok(op, A, B0, B1, C) ||
      !gemm_operands_ok(op, A_shared, B0_shared, B1_shared, C_shared))
    return MOE_EINVAL;
  if (!block_table_ok(*s, block_meta, num_blocks, max_blocks)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  const bool gu = op == MOE_OP_GATEUP_SWIGLU;
  GemmSegments g{A, B0, B1, C, gu ? s->d : s->d_e, gu ? s->d_e : s->d, block_meta, num_blocks,
                 max_blocks, A_shared, B0_shared, B1_shared, C_shared,
                 gu ? s->d : s->d_e_shared, gu ? s->d_e_shared : s->d, s->T};
  return launch_grouped_gemm(*s, op, g, static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_gemm_gather(const moe_shape* s, const void* x, const int32_t* row_src,
                                   const void* w1, const void* w3, const int32_t* block_meta,
                                   const int32_t* num_blocks, int32_t max_blocks, void* act,
                                   const void* ws1, const void* ws3, void* shared_act,
                                   void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!gather_supported(*s)) return MOE_ENOTSUP;
  if (!gemm_operands_ok(MOE_OP_GATEUP_SWIGLU, x, w1, w3, act)) return MOE_EINVAL;
  if (!row_src || !aligned4(row_src)) return MOE_EINVAL;
  if (!block_table_ok(*s, block_meta, num_blocks, max_blocks)) return MOE_EINVAL;
  const bool shared = s->d_e_shared > 0;
  if (shared && !gemm_operands_ok(MOE_OP_GATEUP_SWIGLU, x, ws1, ws3, shared_act)) return MOE_EINVAL;
  if (!shared && (ws1 || ws3 || shared_act)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  GemmSegments g{x, w1, w3, act, s->d, s->d_e, block_meta, num_blocks, max_blocks,
                 shared ? x : nullptr, ws1, ws3, shared_act, s->d, s->d_e_shared,
                 shared ? s->T : 0, row_src, s->k, s->T};
  return launch_grouped_gemm(*s, MOE_OP_GATEUP_SWIGLU, g, static_cast<hipStream_t>(stream));
}

moe_status moe_quantize_fp8(int32_t E, int32_t K, int32_t N, const void* w, uint8_t* q,
                            float* scales, void* stream) {
  if (E < 1 || K < 1 || N < 8 || N % 8) return MOE_EINVAL;
  if ((int64_t)E * K * N >= ((int64_t)1 << 40)) return MOE_ENOTSUP;
  if (!w || !q || !scales || !aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 7u) ||
      !aligned4(scales))
    return MOE_EINVAL;
  return launch_quantize_fp8(E, K, N, w, q, scales, static_cast<hipStream_t>(stream));
}

// The fp8-weight path: bf16 activations, 128-row blocks, K and N the kernel takes.
static moe_status check_fp8(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16 || s.block_m != 128) return MOE_ENOTSUP;
  if (!fp8_gemm_supported(s.d, s.d_e) || !fp8_gemm_supported(s.d_e, s.d)) return MOE_ENOTSUP;
  if (s.d_e_shared > 0 &&
      (!fp8_gemm_supported(s.d, s.d_e_shared) || !fp8_gemm_supported(s.d_e_shared, s.d)))
    return MOE_ENOTSUP;
  return MOE_OK;
}

static bool fp8_operands_ok(int32_t op, const void* A, const uint8_t* Q0, const float* S0,
                            const uint8_t* Q1, const float* S1, const void* C) {
  if (!A || !Q0 || !S0 || !C) return false;
  if (op == MOE_OP_GATEUP_SWIGLU && (!Q1 || !S1)) return false;
  if (op == MOE_OP_DOWN && (Q1 || S1)) return false;
  return aligned16(A) && aligned16(Q0) && aligned4(S0) && (!Q1 || aligned16(Q1)) &&
         (!S1 || aligned4(S1)) && aligned16(C);
}

// One fp8 grouped-GEMM op over the routed segments and (optionally) the shared expert:
// one launch when their K and N agree, else two.
static moe_status run_fp8_op(const moe_shape& s, int op, const void* A, const uint8_t* Q0,
                             const float* S0, const uint8_t* Q1, const float* S1,
                             const int32_t* meta, const int32_t* nblk, int32_t mb,
                             const int32_t* row_src, void* C, const void* As,
                             const uint8_t* Q0s, const float* S0s, const uint8_t* Q1s,
                             const float* S1s, void* Cs, float* tail, hipStream_t st) {
  const bool gu = op == MOE_OP_GATEUP_SWIGLU;
  const int K = gu ? s.d : s.d_e, N = gu ? s.d_e : s.d;
  const bool shared = As != nullptr;
  const int Ks = gu ? s.d : s.d_e_shared, Ns = gu ? s.d_e_shared : s.d;
  GemmSegmentsF8 g{A, Q0, S0, Q1, S1, C, K, N, meta, nblk, mb,
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                   row_src, s.k, s.T, tail};
  // Experts averaging at most 64 rows (decode): the launch streams weights, and the
  // 64-row kernel reads them in wider rows.  At least 256 rows (and a block table the
  // wide kernel takes): compute-bound, the wide kernel with in-register dequantisation.
  // In between: 128-row items.
  const int64_t M = (int64_t)s.T * s.k;
  const int64_t act = M < s.E ? M : (int64_t)s.E;
  const Fp8Kernel kind = mb > 0 ? (M <= 64 * act ? kFp8Rows64
                                   : (M >= 256 * act && mb <= wide_max_blocks()) ? kFp8Wide
                                   : kFp8Rows128)
                                : (s.T <= 64 ? kFp8Rows64 : s.T >= 384 ? kFp8Wide : kFp8Rows128);
  if (shared && Ks == K && Ns == N) {
    g.Ad = As; g.Q0d = Q0s; g.S0d = S0s; g.Q1d = Q1s; g.S1d = S1s; g.Cd = Cs; g.dense_rows = s.T;
    return launch_grouped_gemm_fp8(op, g, s.E, max_rows_of(s), kind, st);
  }
  if (shared) {
    GemmSegmentsF8 d{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, Ks, Ns, nullptr, nullptr,
                     0, As, Q0s, S0s, Q1s, S1s, Cs, s.T, nullptr, 1, 1, tail};
    const Fp8Kernel dk = s.T <= 64 ? kFp8Rows64 : s.T >= 384 ? kFp8Wide : kFp8Rows128;
    moe_status st2 = launch_grouped_gemm_fp8(op, d, 1, s.T, dk, st);
    if (st2 != MOE_OK) return st2;
  }
  return launch_grouped_gemm_fp8(op, g, s.E, max_rows_of(s), kind, st);
}

moe_status moe_grouped_gemm_fp8(const moe_shape* s, int32_t op, const void* A, const uint8_t* Q0,
                                const float* S0, const uint8_t* Q1, const float* S1,
                                const int32_t* block_meta, const int32_t* num_blocks,
                                int32_t max_blocks, const int32_t* row_src, void* C,
                                const void* A_shared, const uint8_t* Q0_shared,
                                const float* S0_shared, const uint8_t* Q1_shared,
                                const float* S1_shared, void* C_shared, void* ws,
                                size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return MOE_EINVAL;
  if ((st = check_fp8(*s)) != MOE_OK) return st;
  if (ws && (!aligned16(ws) || ws_bytes < fp8_tail_scratch_bytes())) return MOE_EWORKSPACE;
  if (!fp8_operands_ok(op, A, Q0, S0, Q1, S1, C)) return MOE_EINVAL;
  if (!block_table_ok(*s, block_meta, num_blocks, max_blocks)) return MOE_EINVAL;
  if (row_src) {
    if (op != MOE_OP_GATEUP_SWIGLU || !aligned4(row_src)) return MOE_EINVAL;
    if (!gather_supported(*s)) return MOE_ENOTSUP;
  }
  const bool shared = A_shared || Q0_shared || S0_shared || Q1_shared || S1_shared || C_shared;
  if (shared) {
    if (s->d_e_shared <= 0) return MOE_EINVAL;
    if (!fp8_operands_ok(op, A_shared, Q0_shared, S0_shared, Q1_shared, S1_shared, C_shared))
      return MOE_EINVAL;
  }
  if (s->T == 0) return MOE_OK;
  return run_fp8_op(*s, op, A, Q0, S0, Q1, S1, block_meta, num_blocks, max_blocks, row_src, C,
                    shared ? A_shared : nullptr, Q0_shared, S0_shared, Q1_shared, S1_shared,
                    C_shared, static_cast<float*>(ws), static_cast<hipStream_t>(stream));
}

size_t moe_grouped_gemm_fp8_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return fp8_tail_scratch_bytes();
}

// The bf16 gate/up (rows gathered from x where the kernels can) and down launches of
// the layer, routed experts and the shared expert together, on the workspace laid out
// by layout_of (routes, block table and the permutation already built).
static moe_status run_bf16_experts(const moe_shape& s, const void* x, char* base,
                                   const moe_ws_layout& L, bool gather, const void* w1,
                                   const void* w3, const void* w2, const void* ws1,
                                   const void* ws3, const void* ws2, hipStream_t hs) {
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  const bool shared = s.d_e_shared > 0;
  const int32_t mb = (int32_t)max_blocks_of(s);
  const int des = s.d_e_shared;
  int32_t* meta = static_cast<int32_t*>(at(L.block_meta));
  int32_t* nblk = static_cast<int32_t*>(at(L.num_blocks));
  GemmSegments gu{gather ? x : at(L.x_perm), w1, w3, at(L.act), s.d, s.d_e, meta, nblk, mb,
                  x, ws1, ws3, at(L.shared_act), s.d, des, shared ? s.T : 0,
                  gather ? static_cast<const int32_t*>(at(L.row_src)) : nullptr, s.k, s.T};
  moe_status st = launch_grouped_gemm(s, MOE_OP_GATEUP_SWIGLU, gu, hs);
  if (st != MOE_OK) return st;
  GemmSegments dn{at(L.act), w2, nullptr, at(L.y), s.d_e, s.d, meta, nblk, mb,
                  at(L.shared_act), ws2, nullptr, at(L.shared_out), des, s.d, shared ? s.T : 0};
  return launch_grouped_gemm(s, MOE_OP_DOWN, dn, hs);
}

// With fp8 weights, where experts average at least 256 rows (the wide bf16 kernel's
// regime, compute-bound) and the workspace has room for them, the layer dequantises the
// weights once into its workspace and runs the bf16 kernels: the same bf16 weights as the
// fp8 kernels' own in-register dequantisation, and faster than the wide kernel doing that
// dequantisation itself (its 192 accumulator registers leave the extra conversions no
// room to hide).  With a workspace of moe_workspace_bytes only, the wide kernel
// dequantises in registers; below 256 rows (decode-like routing, weight streaming) the
// fp8 kernels read half the bytes.
static bool fp8_dequantised_path(const moe_shape& s) {
  const int64_t M = (int64_t)s.T * s.k;
  return M > 0 && M >= 256 * (M < s.E ? M : (int64_t)s.E);
}

// Experts averaging at most 64 rows: the 64-row fp8 kernel streams the weights, and
// scratch lets it split its last round along K.
static bool fp8_streaming_path(const moe_shape& s) {
  const int64_t M = (int64_t)s.T * s.k;
  return M > 0 && M <= 64 * (M < s.E ? M : (int64_t)s.E);
}

struct Fp8Layout {
  size_t w1, w3, w2, ws1, ws3, ws2, tail, total;
};
static void fp8_layout_of(const moe_shape& s, const moe_ws_layout& L, Fp8Layout& F) {
  size_t cur = L.total;
  const bool deq = fp8_dequantised_path(s);
  const size_t E = s.E, d = s.d, de = s.d_e, ds = s.d_e_shared;
  F.w1 = take(cur, deq ? E * d * de * 2 : 0);
  F.w3 = take(cur, deq ? E * d * de * 2 : 0);
  F.w2 = take(cur, deq ? E * de * d * 2 : 0);
  F.ws1 = take(cur, deq ? d * ds * 2 : 0);
  F.ws3 = take(cur, deq ? d * ds * 2 : 0);
  F.ws2 = take(cur, deq ? ds * d * 2 : 0);
  F.tail = take(cur, fp8_streaming_path(s) ? fp8_tail_scratch_bytes() : 0);
  F.total = cur;
}

size_t moe_fp8_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  moe_ws_layout L;
  layout_of(*s, L);
  Fp8Layout F;
  fp8_layout_of(*s, L, F);
  return F.total;
}

moe_status moe_dequantize_fp8(int32_t E, int32_t K, int32_t N, const uint8_t* q,
                              const float* scales, void* w, void* stream) {
  if (E < 1 || K < 1 || N < 8 || N % 8) return MOE_EINVAL;
  if ((int64_t)E * K * N >= ((int64_t)1 << 40)) return MOE_ENOTSUP;
  if (!w || !q || !scales || !aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 7u) ||
      !aligned4(scales))
    return MOE_EINVAL;
  return launch_dequantize_fp8(E, K, N, q, scales, w, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_fwd_fp8(const moe_shape* s, const void* x, const void* w_gate,
                             const float* bias, const uint8_t* q1, const float* s1,
                             const uint8_t* q3, const float* s3, const uint8_t* q2,
                             const float* s2, const uint8_t* qs1, const float* ss1,
                             const uint8_t* qs3, const float* ss3, const uint8_t* qs2,
                             const float* ss2, const int32_t* topk_idx_in,
                             const float* topk_w_in, void* out, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_fp8(*s)) != MOE_OK) return st;
  const bool routed = topk_idx_in && topk_w_in;
  if ((topk_idx_in != nullptr) != (topk_w_in != nullptr)) return MOE_EINVAL;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return MOE_EINVAL;
  if (!routed && !w_gate) return MOE_EINVAL;
  if (!routed && (st = check_routing(*s)) != MOE_OK) return st;
  const bool shared = s->d_e_shared > 0;
  const void* qptr[] = {q1, q3, q2};
  const void* sptr[] = {s1, s3, s2};
  for (int i = 0; i < 3; ++i)
    if (!qptr[i] || !sptr[i] || !aligned16(qptr[i]) || !aligned4(sptr[i])) return MOE_EINVAL;
  const void* qs[] = {qs1, qs3, qs2};
  const void* ss[] = {ss1, ss3, ss2};
  for (int i = 0; i < 3; ++i) {
    if (shared && (!qs[i] || !ss[i] || !aligned16(qs[i]) || !aligned4(ss[i]))) return MOE_EINVAL;
    if (!shared && (qs[i] || ss[i])) return MOE_EINVAL;
  }
  if ((w_gate && !aligned16(w_gate)) || (bias && !aligned4(bias)) ||
      (topk_idx_in && !aligned4(topk_idx_in)) || (topk_w_in && !aligned4(topk_w_in)))
    return MOE_EINVAL;
  moe_ws_layout L;
  layout_of(*s, L);
  Fp8Layout F8;
  fp8_layout_of(*s, L, F8);
  // at least the intermediates; the dequantised weights only where there is room
  if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  int32_t* idx = routed ? const_cast<int32_t*>(topk_idx_in) : static_cast<int32_t*>(at(L.topk_idx));
  float* wts = routed ? const_cast<float*>(topk_w_in) : static_cast<float*>(at(L.topk_w));
  if (!routed) {
    st = launch_route(*s, x, w_gate, bias, static_cast<float*>(at(L.logits)), idx, wts,
                      static_cast<float*>(at(L.scratch)), hs);
    if (st != MOE_OK) return st;
  }
  int32_t* meta = static_cast<int32_t*>(at(L.block_meta));
  int32_t* nblk = static_cast<int32_t*>(at(L.num_blocks));
  int32_t* pos = static_cast<int32_t*>(at(L.pos));
  int32_t* rsrc = static_cast<int32_t*>(at(L.row_src));
  st = launch_build_offsets(*s, idx, static_cast<int32_t*>(at(L.counts)),
                            static_cast<int32_t*>(at(L.offsets)),
                            static_cast<int32_t*>(at(L.padded_offsets)), meta, nblk, pos, rsrc,
                            static_cast<int32_t*>(at(L.err_flag)), at(L.scratch), hs);
  if (st != MOE_OK) return st;
  const bool gather = gather_supported(*s);
  if (!gather) {
    st = launch_permute(*s, x, pos, at(L.x_perm), hs);
    if (st != MOE_OK) return st;
  }
  if (fp8_dequantised_path(*s) && ws_bytes >= F8.total) {
    const int E = s->E, d = s->d, de = s->d_e, des = s->d_e_shared;
    st = launch_dequantize_fp8(E, d, de, q1, s1, at(F8.w1), hs);
    if (st == MOE_OK) st = launch_dequantize_fp8(E, d, de, q3, s3, at(F8.w3), hs);
    if (st == MOE_OK) st = launch_dequantize_fp8(E, de, d, q2, s2, at(F8.w2), hs);
    if (st == MOE_OK && shared) st = launch_dequantize_fp8(1, d, des, qs1, ss1, at(F8.ws1), hs);
    if (st == MOE_OK && shared) st = launch_dequantize_fp8(1, d, des, qs3, ss3, at(F8.ws3), hs);
    if (st == MOE_OK && shared) st = launch_dequantize_fp8(1, des, d, qs2, ss2, at(F8.ws2), hs);
    if (st != MOE_OK) return st;
    st = run_bf16_experts(*s, x, base, L, gather, at(F8.w1), at(F8.w3), at(F8.w2),
                          shared ? at(F8.ws1) : nullptr, shared ? at(F8.ws3) : nullptr,
                          shared ? at(F8.ws2) : nullptr, hs);
    if (st != MOE_OK) return st;
    return launch_combine(*s, at(L.y), pos, wts, shared ? at(L.shared_out) : nullptr, out, hs);
  }
  const int32_t mb = (int32_t)max_blocks_of(*s);
  // the streaming kernel's last-round scratch, where the workspace has room for it
  float* tail = (F8.total > F8.tail && ws_bytes >= F8.total) ? static_cast<float*>(at(F8.tail))
                                                              : nullptr;
  st = run_fp8_op(*s, MOE_OP_GATEUP_SWIGLU, gather ? x : at(L.x_perm), q1, s1, q3, s3, meta, nblk,
                  mb, gather ? rsrc : nullptr, at(L.act), shared ? x : nullptr, qs1, ss1, qs3, ss3,
                  shared ? at(L.shared_act) : nullptr, tail, hs);
  if (st != MOE_OK) return st;
  st = run_fp8_op(*s, MOE_OP_DOWN, at(L.act), q2, s2, nullptr, nullptr, meta, nblk, mb, nullptr,
                  at(L.y), shared ? at(L.shared_act) : nullptr, qs2, ss2, nullptr, nullptr,
                  shared ? at(L.shared_out) : nullptr, tail, hs);
  if (st != MOE_OK) return st;
  const void* sh = shared ? at(L.shared_out) : nullptr;
  return launch_combine(*s, at(L.y), pos, wts, sh, out, hs);
}

moe_status moe_combine(const moe_shape* s, const void* y, const int32_t* pos, const float* topk_w,
                       const void* shared_out, void* out, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!y || !pos || !out) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out) || !aligned4(pos) || (topk_w && !aligned4(topk_w)) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  return launch_combine(*s, y, pos, topk_w, shared_out, out, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_fwd(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                         const void* w1, const void* w3, const void* w2, const void* ws1,
                         const void* ws3, const void* ws2, const int32_t* topk_idx_in,
                         const float* topk_w_in, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const bool routed = topk_idx_in && topk_w_in;
  if ((topk_idx_in != nullptr) != (topk_w_in != nullptr)) return MOE_EINVAL;
  if (!x || !w1 || !w3 || !w2 || !out) return MOE_EINVAL;
  if (!routed && !w_gate) return MOE_EINVAL;
  if (!routed && (st = check_routing(*s)) != MOE_OK) return st;
  const bool shared = s->d_e_shared > 0;
  if (shared && (!ws1 || !ws3 || !ws2)) return MOE_EINVAL;
  if (!shared && (ws1 || ws3 || ws2)) return MOE_EINVAL;
  const void* p16[] = {x, w1, w3, w2, out};
  for (const void* p : p16)
    if (!aligned16(p)) return MOE_EINVAL;
  if (shared && (!aligned16(ws1) || !aligned16(ws3) || !aligned16(ws2))) return MOE_EINVAL;
  if ((w_gate && !aligned16(w_gate)) || (bias && !aligned4(bias)) ||
      (topk_idx_in && !aligned4(topk_idx_in)) || (topk_w_in && !aligned4(topk_w_in)))
    return MOE_EINVAL;
  moe_ws_layout L;
  layout_of(*s, L);
  Fp8Layout F8;
  fp8_layout_of(*s, L, F8);
  // at least the intermediates; the dequantised weights only where there is room
  if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  int32_t* idx = routed ? const_cast<int32_t*>(topk_idx_in) : static_cast<int32_t*>(at(L.topk_idx));
  float* wts = routed ? const_cast<float*>(topk_w_in) : static_cast<float*>(at(L.topk_w));
  if (!routed) {
    st = launch_route(*s, x, w_gate, bias, static_cast<float*>(at(L.logits)), idx, wts,
                      static_cast<float*>(at(L.scratch)), hs);
    if (st != MOE_OK) return st;
  }
  int32_t* meta = static_cast<int32_t*>(at(L.block_meta));
  int32_t* nblk = static_cast<int32_t*>(at(L.num_blocks));
  int32_t* pos = static_cast<int32_t*>(at(L.pos));
  st = launch_build_offsets(*s, idx, static_cast<int32_t*>(at(L.counts)),
                            static_cast<int32_t*>(at(L.offsets)),
                            static_cast<int32_t*>(at(L.padded_offsets)), meta, nblk, pos,
                            static_cast<int32_t*>(at(L.row_src)),
                            static_cast<int32_t*>(at(L.err_flag)), at(L.scratch), hs);
  if (st != MOE_OK) return st;
  // Gate/up reads its A rows straight from x through row_src when the kernels can
  // (the permute fused into the GEMM's loads); otherwise x is permuted first.
  const bool gather = gather_supported(*s);
  if (!gather) {
    st = launch_permute(*s, x, pos, at(L.x_perm), hs);
    if (st != MOE_OK) return st;
  }
  // Routed experts and the shared expert go through the grouped GEMM together (one
  // launch per op when their shapes agree), the shared expert as a dense segment
  // over the unpermuted x.
  st = run_bf16_experts(*s, x, base, L, gather, w1, w3, w2, ws1, ws3, ws2, hs);
  if (st != MOE_OK) return st;
  const void* sh = shared ? at(L.shared_out) : nullptr;
  return launch_combine(*s, at(L.y), pos, wts, sh, out, hs);
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
moe_status moe_combine_bwd(const moe_shape* s, const void* dout, const void* y,
                           const int32_t* pos, const float* topk_w, void* dy, float* dtopk_w,
                           void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (s->d > 8192) return MOE_ENOTSUP;
  if (!dout || !y || !pos || !topk_w || !dy || !dtopk_w) return MOE_EINVAL;
  if (!aligned16(dout) || !aligned16(y) || !aligned16(dy) || !aligned4(pos) ||
      !aligned4(topk_w) || !aligned4(dtopk_w))
    return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  return launch_combine_bwd(*s, dout, y, pos, topk_w, dy, dtopk_w, max_rows_of(*s),
                            static_cast<hipStream_t>(stream));
}

moe_status moe_swiglu_bwd(const moe_shape* s, const void* A, const int32_t* row_src,
                          const void* w1, const void* w3, const void* dact,
                          const int32_t* block_meta, const int32_t* num_blocks, int32_t max_blocks,
                          void* dgu, const void* x_shared, const void* ws1, const void* ws3,
                          const void* dact_shared, void* dgu_shared, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (!gemm_operands_ok(MOE_OP_GATEUP_SWIGLU, A, w1, w3, dgu) || !dact || !aligned16(dact))
    return MOE_EINVAL;
  if (!block_table_ok(*s, block_meta, num_blocks, max_blocks)) return MOE_EINVAL;
  if (row_src) {
    if (!aligned4(row_src)) return MOE_EINVAL;
    if (!gather_supported(*s)) return MOE_ENOTSUP;
  }
  const bool shared = x_shared || ws1 || ws3 || dact_shared || dgu_shared;
  if (shared) {
    if (s->d_e_shared <= 0) return MOE_EINVAL;
    if (!gemm_operands_ok(MOE_OP_GATEUP_SWIGLU, x_shared, ws1, ws3, dgu_shared) || !dact_shared ||
        !aligned16(dact_shared))
      return MOE_EINVAL;
  }
  if (s->T == 0) return MOE_OK;
  GemmSegments g{A, w1, w3, dgu, s->d, s->d_e, block_meta, num_blocks, max_blocks,
                 shared ? x_shared : nullptr, ws1, ws3, dgu_shared, s->d, s->d_e_shared,
                 shared ? s->T : 0, row_src, s->k, s->T, dact, dact_shared};
  return launch_grouped_gemm(*s, kOpGateUpBwd, g, static_cast<hipStream_t>(stream));
}

// A data gradient on the forward kernels: the weights transposed into wt, then the
// plain grouped product (op DOWN: no epilogue) C = A (B^T).
//   DOWN:   W2 [E][d_e][d] -> wt [E][d][d_e];     dA [rows, d_e] = dC [rows, d] wt[e]
//   GATEUP: W1, W3 [E][d][d_e] -> wt [E][2 d_e][d] (W1^T rows, then W3^T rows);
//           dA [rows, d] = dC [rows, 2 d_e] wt[e]
static moe_status dgrad_on_forward_kernels(const moe_shape& s, int op, const void* dC,
                                           const void* B0, const void* B1,
                                           const int32_t* meta, const int32_t* nblk, int32_t mb,
                                           void* dA, const void* dC_d, const void* B0_d,
                                           const void* B1_d, void* dA_d, int de_d, void* wt,
                                           void* wt_d, hipStream_t st) {
  const bool gu = op == MOE_OP_GATEUP_SWIGLU;
  const bool routed = mb > 0, dense = dC_d != nullptr;
  const int d = s.d, de = s.d_e;
  moe_status r = MOE_OK;
  if (routed) {
    r = gu ? launch_transpose_bf16(s.E, d, de, B0, wt, (int64_t)2 * de * d, d, st)
           : launch_transpose_bf16(s.E, de, d, B0, wt, (int64_t)d * de, de, st);
    if (r == MOE_OK && gu)
      r = launch_transpose_bf16(s.E, d, de, B1, static_cast<bf16_t*>(wt) + (size_t)de * d,
                                (int64_t)2 * de * d, d, st);
    if (r != MOE_OK) return r;
  }
  if (dense) {
    r = gu ? launch_transpose_bf16(1, d, de_d, B0_d, wt_d, (int64_t)2 * de_d * d, d, st)
           : launch_transpose_bf16(1, de_d, d, B0_d, wt_d, (int64_t)d * de_d, de_d, st);
    if (r == MOE_OK && gu)
      r = launch_transpose_bf16(1, d, de_d, B1_d, static_cast<bf16_t*>(wt_d) + (size_t)de_d * d,
                                (int64_t)2 * de_d * d, d, st);
    if (r != MOE_OK) return r;
  }
  GemmSegments g{};
  if (routed) {
    g.A = dC; g.B0 = wt; g.C = dA; g.K = gu ? 2 * de : d; g.N = gu ? d : de;
    g.block_meta = meta; g.num_blocks = nblk; g.max_blocks = mb;
  }
  if (dense) {
    g.Ad = dC_d; g.B0d = wt_d; g.Cd = dA_d; g.Kd = gu ? 2 * de_d : d; g.Nd = gu ? d : de_d;
    g.dense_rows = s.T;
  }
  return launch_grouped_gemm(s, MOE_OP_DOWN, g, st);
}

size_t moe_grouped_gemm_dgrad_workspace_bytes(const moe_shape* s, int32_t op) {
  if (check_shape(s) != MOE_OK) return 0;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return 0;
  return align_up((size_t)s->E * s->d * s->d_e * 2 * (op == MOE_OP_GATEUP_SWIGLU ? 2 : 1), 256);
}

moe_status moe_grouped_gemm_dgrad(const moe_shape* s, int32_t op, const void* dC, const void* B0,
                                  const void* B1, const int32_t* block_meta,
                                  const int32_t* num_blocks, int32_t max_blocks, void* dA,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return MOE_EINVAL;
  if (!gemm_operands_ok(op, dC, B0, B1, dA)) return MOE_EINVAL;
  const bool dense = !block_meta && !num_blocks;
  if (dense ? max_blocks != 0 : !block_table_ok(*s, block_meta, num_blocks, max_blocks))
    return MOE_EINVAL;
  // with a workspace the weights are transposed into it and the forward kernels run
  const bool tw = ws != nullptr;
  if (tw && (!aligned16(ws) || ws_bytes < moe_grouped_gemm_dgrad_workspace_bytes(s, op)))
    return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool gu = op == MOE_OP_GATEUP_SWIGLU;
  if (tw) {
    if (dense)
      return dgrad_on_forward_kernels(*s, op, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                      nullptr, dC, B0, B1, dA, s->d_e, nullptr, ws, hs);
    return dgrad_on_forward_kernels(*s, op, dC, B0, B1, block_meta, num_blocks, max_blocks, dA,
                                    nullptr, nullptr, nullptr, nullptr, 0, ws, nullptr, hs);
  }
  const int K = gu ? 2 * s->d_e : s->d, N = gu ? s->d : s->d_e;
  const int ldb = gu ? s->d_e : s->d;
  return launch_gg_nt(dC, B0, B1, ldb, gu ? s->d_e : K, dA, K, N, block_meta, num_blocks,
                      dense ? 0 : max_blocks, dense ? 1 : s->E, s->block_m,
                      routed_rows_bound(*s, max_blocks), dense ? s->T : 0, hs);
}

size_t moe_grouped_gemm_wgrad_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return align_up(wgrad_sched_bytes(s->E), 256);
}

moe_status moe_grouped_gemm_wgrad(const moe_shape* s, int32_t op, const void* A, const void* dC,
                                  const int32_t* counts, const int32_t* padded_offsets, float* dB0,
                                  float* dB1, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (op != MOE_OP_GATEUP_SWIGLU && op != MOE_OP_DOWN) return MOE_EINVAL;
  const bool gu = op == MOE_OP_GATEUP_SWIGLU;
  if (!A || !dC || !dB0 || (gu && !dB1) || (!gu && dB1)) return MOE_EINVAL;
  if (!aligned16(A) || !aligned16(dC) || !aligned4(dB0) || (dB1 && !aligned4(dB1)))
    return MOE_EINVAL;
  if ((counts == nullptr) != (padded_offsets == nullptr)) return MOE_EINVAL;
  if (counts && (!aligned4(counts) || !aligned4(padded_offsets))) return MOE_EINVAL;
  const bool dense = counts == nullptr;
  if (ws && (!aligned16(ws) || ws_bytes < wgrad_sched_bytes(s->E))) return MOE_EWORKSPACE;
  const int Km = gu ? s->d : s->d_e, Nn = gu ? 2 * s->d_e : s->d;
  // T == 0 still writes the (zero) gradients: the counts are not read then
  return launch_gg_wgrad(A, dC, dB0, dB1, gu ? s->d_e : Nn, Km, Nn, s->T > 0 ? counts : nullptr,
                         padded_offsets, dense ? 1 : s->E, dense ? s->T : 0, dense ? nullptr : ws,
                         static_cast<hipStream_t>(stream));
}

size_t moe_router_bwd_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return router_bwd_scratch_bytes(*s);
}

moe_status moe_router_bwd(const moe_shape* s, const void* x, const void* w_gate,
                          const float* logits, const int32_t* topk_idx, const float* dtopk_w,
                          float* dlogits, float* dw_gate, float* dbias, const void* dx_in,
                          void* dx_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !logits || !topk_idx || !dtopk_w || !dlogits || !dw_gate || !dx_out)
    return MOE_EINVAL;
  if (!aligned16(x) || !aligned4(w_gate) || !aligned4(logits) || !aligned4(topk_idx) ||
      !aligned4(dtopk_w) || !aligned4(dlogits) || !aligned4(dw_gate) || (dbias && !aligned4(dbias)) ||
      (dx_in && !aligned16(dx_in)) || !aligned16(dx_out))
    return MOE_EINVAL;
  const size_t need = router_bwd_scratch_bytes(*s);
  if (need && (!ws || !aligned16(ws) || ws_bytes < need)) return MOE_EWORKSPACE;
  return launch_router_bwd(*s, x, w_gate, logits, topk_idx, dtopk_w, dlogits, dw_gate, dbias, dx_in,
                           dx_out, need ? ws : nullptr, static_cast<hipStream_t>(stream));
}

size_t moe_bwd_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  moe_bwd_ws_layout L;
  bwd_layout_of(*s, L);
  return L.total;
}

moe_status moe_bwd_workspace_layout(const moe_shape* s, moe_bwd_ws_layout* layout) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!layout) return MOE_EINVAL;
  bwd_layout_of(*s, *layout);
  return MOE_OK;
}

moe_status moe_layer_bwd(const moe_shape* s, const void* x, const void* w_gate, const void* w1,
                         const void* w3, const void* w2, const void* ws1, const void* ws3,
                         const void* ws2, const int32_t* topk_idx_in, const float* topk_w_in,
                         const void* dout, const void* fwd_ws, size_t fwd_ws_bytes, void* dx,
                         float* dw1, float* dw3, float* dw2, float* dws1, float* dws3, float* dws2,
                         float* dw_gate, float* dbias, float* dtopk_w, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_bwd(*s)) != MOE_OK) return st;
  if (s->d > 8192) return MOE_ENOTSUP;
  const bool routed = topk_idx_in && topk_w_in;
  if ((topk_idx_in != nullptr) != (topk_w_in != nullptr)) return MOE_EINVAL;
  if (!routed && !w_gate) return MOE_EINVAL;
  if (routed && (dw_gate || dbias)) return MOE_EINVAL;
  const bool shared = s->d_e_shared > 0;
  const void* p16[] = {x, w1, w3, w2, dout, dx};
  for (const void* p : p16)
    if (!p || !aligned16(p)) return MOE_EINVAL;
  float* f4[] = {dw1, dw3, dw2};
  for (float* p : f4)
    if (!p || !aligned4(p)) return MOE_EINVAL;
  if (shared) {
    const void* sp[] = {ws1, ws3, ws2};
    for (const void* p : sp)
      if (!p || !aligned16(p)) return MOE_EINVAL;
    float* sg[] = {dws1, dws3, dws2};
    for (float* p : sg)
      if (!p || !aligned4(p)) return MOE_EINVAL;
  } else if (ws1 || ws3 || ws2 || dws1 || dws3 || dws2) {
    return MOE_EINVAL;
  }
  if ((w_gate && !aligned4(w_gate)) || (dw_gate && !aligned4(dw_gate)) ||
      (dbias && !aligned4(dbias)) || (dtopk_w && !aligned4(dtopk_w)) ||
      (topk_idx_in && !aligned4(topk_idx_in)) || (topk_w_in && !aligned4(topk_w_in)))
    return MOE_EINVAL;
  moe_ws_layout F;
  layout_of(*s, F);
  if (!fwd_ws || !aligned16(fwd_ws) || fwd_ws_bytes < F.total) return MOE_EWORKSPACE;
  moe_bwd_ws_layout L;
  bwd_layout_of(*s, L);
  if (!ws || !aligned16(ws) || ws_bytes < L.total) return MOE_EWORKSPACE;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int de = s->d_e, des = s->d_e_shared, d = s->d;
  if (s->T == 0) {
    // no rows: every weight gradient is zero
    st = launch_gg_wgrad(x, x, dw1, dw3, de, d, 2 * de, nullptr, nullptr, s->E, 0, nullptr, hs);
    if (st == MOE_OK)
      st = launch_gg_wgrad(x, x, dw2, nullptr, d, de, d, nullptr, nullptr, s->E, 0, nullptr, hs);
    if (st == MOE_OK && shared)
      st = launch_gg_wgrad(x, x, dws1, dws3, des, d, 2 * des, nullptr, nullptr, 1, 0, nullptr, hs);
    if (st == MOE_OK && shared)
      st = launch_gg_wgrad(x, x, dws2, nullptr, d, des, d, nullptr, nullptr, 1, 0, nullptr, hs);
    if (st == MOE_OK && (dw_gate || dbias))
      st = launch_router_bwd(*s, x, w_gate, nullptr, nullptr, nullptr, nullptr, dw_gate, dbias,
                             nullptr, dx, nullptr, hs);
    return st;
  }
  const char* fb = static_cast<const char*>(fwd_ws);
  auto fat = [&](size_t off) { return static_cast<const void*>(fb + off); };
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  const int32_t* idx = routed ? topk_idx_in : static_cast<const int32_t*>(fat(F.topk_idx));
  const float* wts = routed ? topk_w_in : static_cast<const float*>(fat(F.topk_w));
  const int32_t* counts = static_cast<const int32_t*>(fat(F.counts));
  const int32_t* padded = static_cast<const int32_t*>(fat(F.padded_offsets));
  const int32_t* meta = static_cast<const int32_t*>(fat(F.block_meta));
  const int32_t* nblk = static_cast<const int32_t*>(fat(F.num_blocks));
  const int32_t* pos = static_cast<const int32_t*>(fat(F.pos));
  const int32_t mb = (int32_t)max_blocks_of(*s);
  float* dtw = dtopk_w ? dtopk_w : static_cast<float*>(at(L.dtopk_w));

  // combine
  st = launch_combine_bwd(*s, dout, fat(F.y), pos, wts, at(L.dy), dtw, max_rows_of(*s), hs);
  if (st != MOE_OK) return st;
  // down: data and weight gradients (routed, then the shared expert on all tokens)
  const bool tw = transposed_dgrad(*s);
  if (tw) {
    st = dgrad_on_forward_kernels(*s, MOE_OP_DOWN, at(L.dy), w2, nullptr, meta, nblk, mb,
                                  at(L.dact), shared ? dout : nullptr, ws2, nullptr,
                                  shared ? at(L.shared_dact) : nullptr, des, at(L.w2_t),
                                  at(L.ws2_t), hs);
  } else {
    st = launch_gg_nt(at(L.dy), w2, nullptr, d, d, at(L.dact), d, de, meta, nblk, mb, s->E,
                      s->block_m, max_rows_of(*s), 0, hs);
  }
  if (st != MOE_OK) return st;
  st = launch_gg_wgrad(fat(F.act), at(L.dy), dw2, nullptr, d, de, d, counts, padded, s->E, 0,
                       at(L.wgrad_sched), hs);
  if (st != MOE_OK) return st;
  if (shared) {
    if (!tw) {
      st = launch_gg_nt(dout, ws2, nullptr, d, d, at(L.shared_dact), d, des, nullptr, nullptr, 0, 1,
                        s->block_m, max_rows_of(*s), s->T, hs);
      if (st != MOE_OK) return st;
    }
    st = launch_gg_wgrad(fat(F.shared_act), dout, dws2, nullptr, d, des, d, nullptr, nullptr, 1,
                         s->T, nullptr, hs);
    if (st != MOE_OK) return st;
  }
  // the weight gradients of gate/up reduce over x_perm's rows
  st = launch_permute(*s, x, pos, at(L.x_perm), hs);
  if (st != MOE_OK) return st;
  // SwiGLU backward with the gate/up products recomputed (both sets in one launch
  // when their sizes agree)
  GemmSegments g{at(L.x_perm), w1, w3, at(L.dgu), d, de, meta, nblk, mb,
                 shared ? x : nullptr, ws1, ws3, shared ? at(L.shared_dgu) : nullptr, d, des,
                 shared ? s->T : 0, nullptr, 1, 1, at(L.dact), shared ? at(L.shared_dact) : nullptr};
  st = launch_grouped_gemm(*s, kOpGateUpBwd, g, hs);
  if (st != MOE_OK) return st;
  // gate/up: data and weight gradients
  if (tw) {
    st = dgrad_on_forward_kernels(*s, MOE_OP_GATEUP_SWIGLU, at(L.dgu), w1, w3, meta, nblk, mb,
                                  at(L.dx_perm), shared ? at(L.shared_dgu) : nullptr, ws1, ws3,
                                  shared ? at(L.shared_dx) : nullptr, des, at(L.w13_t),
                                  at(L.ws13_t), hs);
  } else {
    st = launch_gg_nt(at(L.dgu), w1, w3, de, de, at(L.dx_perm), 2 * de, d, meta, nblk, mb, s->E,
                      s->block_m, max_rows_of(*s), 0, hs);
  }
  if (st != MOE_OK) return st;
  st = launch_gg_wgrad(at(L.x_perm), at(L.dgu), dw1, dw3, de, d, 2 * de, counts, padded, s->E, 0,
                       at(L.wgrad_sched), hs);
  if (st != MOE_OK) return st;
  if (shared) {
    if (!tw) {
      st = launch_gg_nt(at(L.shared_dgu), ws1, ws3, des, des, at(L.shared_dx), 2 * des, d, nullptr,
                        nullptr, 0, 1, s->block_m, max_rows_of(*s), s->T, hs);
      if (st != MOE_OK) return st;
    }
    st = launch_gg_wgrad(x, at(L.shared_dgu), dws1, dws3, des, d, 2 * des, nullptr, nullptr, 1,
                         s->T, nullptr, hs);
    if (st != MOE_OK) return st;
  }
  // router: dlogits, dW_g, dbias, and its dx term on top of the shared expert's
  const void* extra = shared ? at(L.shared_dx) : nullptr;
  if (!routed) {
    st = launch_router_bwd(*s, x, w_gate, static_cast<const float*>(fat(F.logits)), idx, dtw,
                           static_cast<float*>(at(L.dlogits)), dw_gate, dbias, extra,
                           at(L.router_dx), at(L.router_scratch), hs);
    if (st != MOE_OK) return st;
    extra = at(L.router_dx);
  }
  // permute backward: dx[t] = sum_j dx_perm[pos[t, j]] (+ the rest)
  return launch_combine(*s, at(L.dx_perm), pos, nullptr, extra, dx, hs);
}

}  // extern "C"
