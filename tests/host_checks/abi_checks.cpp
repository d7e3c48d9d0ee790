// Host-side checks of the C ABI, meant to be built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (the device code is not compiled): the
// sizing and layout functions over many shapes - valid, at the edges and invalid,
// including sizes near the 32-bit limits where an overflowing int would show - and every
// compute entry point with arguments it must reject before it launches anything.  No
// GPU is touched.  Exit status 0: every check held (a sanitizer report aborts first).
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe.h"

static int g_failures = 0;
#define CHECK(cond, ...)                                                   \
  do {                                                                     \
    if (!(cond)) {                                                         \
      ++g_failures;                                                        \
      std::fprintf(stderr, "FAIL line %d: ", __LINE__);                    \
      std::fprintf(stderr, __VA_ARGS__);                                   \
      std::fprintf(stderr, "\n");                                          \
    }                                                                      \
  } while (0)

// 64-bit LCG (Knuth's MMIX constants); the high bits are used
struct Rng {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(s >> 32);
  }
  int32_t pick(const int32_t* v, int n) { return v[next() % (uint32_t)n]; }
  int32_t range(int32_t lo, int32_t hi) {   // inclusive; lo when hi < lo
    if (hi <= lo) return lo;
    return lo + (int32_t)(next() % (uint32_t)((int64_t)hi - lo + 1));
  }
};

static moe_shape base_shape() {
  moe_shape s;
  std::memset(&s, 0, sizeof s);
  s.T = 64; s.d = 256; s.E = 8; s.k = 2; s.d_e = 512; s.block_m = 128; s.dtype = MOE_DTYPE_BF16;
  return s;
}

// A random shape: every field is drawn from values that are valid and near the limits
// most of the time, and from invalid or extreme ones otherwise.
static moe_shape random_shape(Rng& r) {
  static const int32_t Tv[] = {0, 1, 7, 64, 300, 4096, 8192, 16384, 1 << 20, (1 << 24) + 1, (1 << 27) - 3};
  static const int32_t Tx[] = {(1 << 28) - 1, 1 << 28, (1 << 30) + 3, 0x7fffffff, -1};
  static const int32_t dv[] = {8, 16, 32, 256, 1032, 2048, 7168, 1 << 16};
  static const int32_t dx[] = {1 << 20, 1 << 24, 1 << 28, 0x7ffffff8, 12, 4, 0, -8};
  static const int32_t Ev[] = {1, 2, 3, 4, 8, 64, 256, 1000, 1024};
  static const int32_t Ex[] = {1025, 0, -1};
  static const int32_t bv[] = {128, 256, 384, 1024, 1, 7, 32};
  static const int32_t bx[] = {1 << 20, 1 << 30, 0, -128};
  auto field = [&r](const int32_t* v, int nv, const int32_t* x, int nx) {
    return r.next() % 8 ? r.pick(v, nv) : r.pick(x, nx);
  };
#define FIELD(v, x) field(v, sizeof v / sizeof v[0], x, sizeof x / sizeof x[0])
  moe_shape s;
  std::memset(&s, 0, sizeof s);
  s.T = FIELD(Tv, Tx);
  s.d = FIELD(dv, dx);
  s.E = FIELD(Ev, Ex);
  s.k = r.next() % 8 ? r.range(1, s.E > 1 ? (s.E < 64 ? s.E : 64) : 1) : r.range(-1, 1100);
  s.d_e = FIELD(dv, dx);
  if (r.next() % 3 == 0) {
    s.n_groups = r.next() % 8 ? r.pick(Ev, 6) : r.range(-1, 66);
    s.topk_groups = r.range(r.next() % 8 ? 1 : -1, s.n_groups + (r.next() % 8 == 0));
  }
  s.renormalize = r.next() % 8 ? (int32_t)(r.next() % 2) : r.range(-1, 2);
  s.block_m = FIELD(bv, bx);
  s.d_e_shared = (r.next() % 3 == 0) ? FIELD(dv, dx) : 0;
  s.dtype = r.next() % 8 ? (int32_t)(r.next() % 2) : r.range(-1, 2);
  s.unpadded = r.next() % 8 ? (int32_t)(r.next() % 2) : r.range(-1, 2);
#undef FIELD
  return s;
}

// The block-table bound the header states, recomputed in 64 bits: padded,
// floor((T*k + min(E, T*k) * (block_m - 1)) / block_m); unpadded,
// ceil(T*k / block_m) + min(E, T*k) - 1 (0 without rows).
static int64_t expected_blocks(const moe_shape& s) {
  const int64_t M = (int64_t)s.T * s.k, ne = M < s.E ? M : s.E;
  if (s.unpadded) return M == 0 ? 0 : (M + s.block_m - 1) / s.block_m + ne - 1;
  return (M + ne * (s.block_m - 1)) / s.block_m;
}

// The regions of the forward workspace in field order with the sizes the header
// documents for them; each must fit before the next region's offset.
static void check_regions(const moe_shape& s, const moe_ws_layout& L, int64_t mb, int64_t rows) {
  const uint64_t b = s.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const uint64_t T = s.T, E = s.E, M = (uint64_t)s.T * s.k;
  const bool gathered = s.dtype == MOE_DTYPE_BF16 && s.d % 32 == 0;
  const uint64_t need[] = {T * E * 4, M * 4, M * 4, E * 4, (E + 1) * 4, (E + 1) * 4,
                           (uint64_t)mb * 12, 4, M * 4, (uint64_t)rows * 4, 4,
                           gathered ? 0 : (uint64_t)rows * s.d * b, (uint64_t)rows * s.d_e * b,
                           (uint64_t)rows * s.d * b, T * (uint64_t)s.d_e_shared * b,
                           s.d_e_shared ? T * s.d * b : 0, 0};
  const size_t off[] = {L.logits, L.topk_idx, L.topk_w, L.counts, L.offsets, L.padded_offsets,
                        L.block_meta, L.num_blocks, L.pos, L.row_src, L.err_flag, L.x_perm,
                        L.act, L.y, L.shared_act, L.shared_out, L.scratch, L.total};
  for (int i = 0; i + 1 < (int)(sizeof off / sizeof off[0]); ++i) {
    CHECK(off[i] % 16 == 0, "region %d offset %zu not 16-byte aligned", i, off[i]);
    CHECK(off[i + 1] >= off[i] && off[i + 1] - off[i] >= need[i],
          "region %d [%zu, %zu) holds fewer than %llu bytes (T=%d d=%d E=%d k=%d d_e=%d)", i, off[i],
          off[i + 1], (unsigned long long)need[i], s.T, s.d, s.E, s.k, s.d_e);
  }
}

static long g_valid = 0, g_invalid = 0;

static void check_sizing(const moe_shape& s) {
  const int32_t mb = moe_max_blocks(&s);
  const int64_t mr = moe_max_rows(&s);
  const size_t ws = moe_workspace_bytes(&s);
  moe_ws_layout L;
  std::memset(&L, 0xab, sizeof L);
  const moe_status st = moe_workspace_layout(&s, &L);
  if (st != MOE_OK) {
    ++g_invalid;
    CHECK(st == MOE_EINVAL || st == MOE_ENOTSUP, "status %d for an invalid shape", st);
    CHECK(mb == -1 && mr == -1 && ws == 0, "invalid shape must fail every sizing call (T=%d d=%d E=%d k=%d "
          "bm=%d unpadded=%d: %d %lld %zu)", s.T, s.d, s.E, s.k, s.block_m, s.unpadded, mb, (long long)mr, ws);
    CHECK(moe_fp8_workspace_bytes(&s) == 0 && moe_build_offsets_scratch_bytes(&s) == 0,
          "invalid shape in the fp8 / offsets sizing");
    return;
  }
  ++g_valid;
  const int64_t M = (int64_t)s.T * s.k;
  CHECK(M < ((int64_t)1 << 31), "accepted T*k = %lld", (long long)M);
  CHECK(mb >= 0 && mb == expected_blocks(s), "max blocks %d, expected %lld (T=%d E=%d k=%d bm=%d unpadded=%d)",
        mb, (long long)expected_blocks(s), s.T, s.E, s.k, s.block_m, s.unpadded);
  CHECK((int64_t)mb * s.block_m < ((int64_t)1 << 31), "block rows beyond int32");
  CHECK(mr == (s.unpadded ? M : (int64_t)mb * s.block_m), "max rows %lld", (long long)mr);
  CHECK(L.total == ws, "layout total %zu vs workspace bytes %zu", L.total, ws);
  check_regions(s, L, mb, mr);
  const size_t f8 = moe_fp8_workspace_bytes(&s);
  CHECK(f8 == 0 || f8 >= ws, "fp8 workspace %zu below the bf16 layout %zu", f8, ws);
  CHECK(moe_build_offsets_scratch_bytes(&s) <= L.total - L.scratch, "offsets scratch outside the layout");
  moe_bwd_ws_layout BL;
  if (moe_bwd_workspace_layout(&s, &BL) == MOE_OK) {
    CHECK(BL.total == moe_bwd_workspace_bytes(&s), "backward layout total");
    const size_t boffs[] = {BL.dy, BL.dact, BL.dgu, BL.x_perm, BL.dx_perm, BL.dtopk_w, BL.dlogits,
                            BL.shared_dact, BL.shared_dgu, BL.shared_dx, BL.router_dx,
                            BL.router_scratch, BL.wgrad_sched, BL.w2_t, BL.w13_t, BL.ws2_t, BL.ws13_t,
                            BL.total};
    const uint64_t d = s.d, de = s.d_e, T = s.T, r = (uint64_t)mr;
    const uint64_t bneed[] = {r * d * 2, r * de * 2, r * 2 * de * 2, r * d * 2, r * d * 2,
                              (uint64_t)M * 4, T * s.E * 4};
    for (int i = 0; i + 1 < (int)(sizeof boffs / sizeof boffs[0]); ++i) {
      CHECK(boffs[i] % 16 == 0 && boffs[i + 1] >= boffs[i], "backward region %d", i);
      if (i < (int)(sizeof bneed / sizeof bneed[0]))
        CHECK(boffs[i + 1] - boffs[i] >= bneed[i], "backward region %d too small", i);
    }
  }
  (void)moe_grouped_gemm_dgrad_workspace_bytes(&s, MOE_OP_GATEUP_SWIGLU);
  (void)moe_grouped_gemm_dgrad_workspace_bytes(&s, MOE_OP_DOWN);
  (void)moe_grouped_gemm_dgrad_workspace_bytes(&s, 7);
  (void)moe_grouped_gemm_wgrad_workspace_bytes(&s);
  (void)moe_router_bwd_workspace_bytes(&s);
  CHECK(moe_grouped_gemm_fp8_workspace_bytes(&s) > 0, "fp8 gemm scratch size");
}

int main() {
  // sizing over edge and random shapes
  Rng r{12345};
  for (int i = 0; i < 1000000; ++i) {
    const moe_shape s = random_shape(r);
    check_sizing(s);
  }
  CHECK(moe_max_blocks(nullptr) < 0 && moe_max_rows(nullptr) < 0 && moe_workspace_bytes(nullptr) == 0,
        "null shape in sizing");
  CHECK(moe_workspace_layout(nullptr, nullptr) == MOE_EINVAL, "null layout");
  for (int st = -3; st < 8; ++st) CHECK(moe_status_str(st) != nullptr, "status string %d", st);
  CHECK(moe_build_offsets_noalloc_capacity() > 0, "no-alloc capacity");

  // every compute entry point rejects a null shape, null pointers and a short workspace
  void* F = reinterpret_cast<void*>(0x10000);   // aligned, never dereferenced
  const moe_shape s = base_shape();
  int32_t* Fi = static_cast<int32_t*>(F);
  float* Ff = static_cast<float*>(F);
  uint8_t* Fq = static_cast<uint8_t*>(F);
  const size_t short_ws = 16;
  CHECK(moe_route(nullptr, F, F, nullptr, nullptr, Fi, Ff, F, 1 << 30, nullptr) == MOE_EINVAL, "route null shape");
  CHECK(moe_route(&s, nullptr, F, nullptr, nullptr, Fi, Ff, F, 1 << 30, nullptr) == MOE_EINVAL, "route null x");
  CHECK(moe_route(&s, F, F, nullptr, nullptr, Fi, Ff, F, short_ws, nullptr) == MOE_EWORKSPACE, "route ws");
  CHECK(moe_build_offsets(&s, nullptr, Fi, Fi, Fi, Fi, Fi, Fi, Fi, Fi, F, 1 << 30, nullptr) == MOE_EINVAL,
        "offsets null idx");
  CHECK(moe_build_offsets(&s, Fi, Fi, Fi, Fi, Fi, Fi, Fi, Fi, Fi, F, short_ws, nullptr) == MOE_EWORKSPACE,
        "offsets ws");
  CHECK(moe_build_offsets_noalloc(nullptr, Fi, Fi, Fi, Fi, Fi, Fi, Fi, Fi, Fi, nullptr) == MOE_EINVAL,
        "noalloc null shape");
  CHECK(moe_permute(&s, nullptr, Fi, F, nullptr) == MOE_EINVAL, "permute null x");
  CHECK(moe_grouped_gemm(&s, 0, nullptr, F, F, Fi, Fi, 4, F, nullptr) == MOE_EINVAL, "gemm null A");
  CHECK(moe_grouped_gemm(&s, 9, F, F, F, Fi, Fi, 4, F, nullptr) == MOE_EINVAL, "gemm bad op");
  CHECK(moe_grouped_gemm_shared(&s, 0, F, F, F, Fi, Fi, 4, F, nullptr, F, F, F, nullptr) == MOE_EINVAL,
        "shared null");
  CHECK(moe_grouped_gemm_gather(&s, nullptr, Fi, F, F, Fi, Fi, 4, F, nullptr, nullptr, nullptr, nullptr) ==
            MOE_EINVAL, "gather null x");
  CHECK(moe_combine(&s, nullptr, Fi, Ff, nullptr, F, nullptr) == MOE_EINVAL, "combine null y");
  CHECK(moe_layer_fwd(&s, F, F, nullptr, F, F, F, nullptr, nullptr, nullptr, nullptr, nullptr, F, F, short_ws,
                      nullptr) == MOE_EWORKSPACE, "layer ws");
  CHECK(moe_layer_fwd(nullptr, F, F, nullptr, F, F, F, nullptr, nullptr, nullptr, nullptr, nullptr, F, F,
                      1 << 30, nullptr) == MOE_EINVAL, "layer null shape");
  CHECK(moe_quantize_fp8(1, 256, 256, nullptr, Fq, Ff, nullptr) == MOE_EINVAL, "quantize null w");
  CHECK(moe_quantize_fp8(-1, 256, 256, F, Fq, Ff, nullptr) == MOE_EINVAL, "quantize bad E");
  CHECK(moe_dequantize_fp8(1, 256, 255, Fq, Ff, F, nullptr) == MOE_EINVAL, "dequantize bad N");
  CHECK(moe_grouped_gemm_fp8(&s, 0, nullptr, Fq, Ff, Fq, Ff, Fi, Fi, 4, nullptr, F, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr, nullptr, 0, nullptr) == MOE_EINVAL, "fp8 gemm null A");
  CHECK(moe_grouped_gemm_fp8(&s, 0, F, Fq, Ff, Fq, Ff, Fi, Fi, 4, nullptr, F, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr, F, short_ws, nullptr) == MOE_EWORKSPACE,
        "fp8 gemm short scratch");
  CHECK(moe_layer_fwd_fp8(&s, F, F, nullptr, Fq, Ff, Fq, Ff, Fq, Ff, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, F, F, short_ws, nullptr) == MOE_EWORKSPACE, "fp8 layer ws");
  CHECK(moe_combine_bwd(&s, nullptr, F, Fi, Ff, F, Ff, nullptr) == MOE_EINVAL, "combine bwd null");
  CHECK(moe_swiglu_bwd(&s, nullptr, Fi, F, F, F, Fi, Fi, 4, F, nullptr, nullptr, nullptr, nullptr, nullptr,
                       nullptr) == MOE_EINVAL, "swiglu bwd null");
  CHECK(moe_grouped_gemm_dgrad(&s, 0, nullptr, F, F, Fi, Fi, 4, F, F, 1 << 30, nullptr) == MOE_EINVAL,
        "dgrad null");
  CHECK(moe_grouped_gemm_wgrad(&s, 0, nullptr, F, Fi, Fi, Ff, Ff, F, 1 << 30, nullptr) == MOE_EINVAL,
        "wgrad null");
  CHECK(moe_router_bwd(&s, nullptr, F, Ff, Fi, Ff, Ff, Ff, Ff, nullptr, nullptr, F, 1 << 30, nullptr) ==
            MOE_EINVAL, "router bwd null");
  CHECK(moe_layer_bwd(&s, F, F, F, F, F, nullptr, nullptr, nullptr, nullptr, nullptr, F, F, short_ws, F, Ff, Ff,
                      Ff, nullptr, nullptr, nullptr, Ff, nullptr, nullptr, F, short_ws, nullptr) != MOE_OK,
        "layer bwd ws");
  std::printf("shapes: %ld valid, %ld rejected\n", g_valid, g_invalid);
  CHECK(g_valid > 100000 && g_invalid > 100000, "the random shapes must hit both sides");
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi host checks: ok\n");
  return 0;
}
