// Router GEMM and expert selection.
//
// logits = x[T, d] @ W_g[d, E] (+ bias) is a GEMM with M = T, N = E, K = d; it does
// no heavy arithmetic and is bound by reading x once (TileLang chapter "MoE, MLA and
// sparse-attention operators", section 2.2).  Selection is k rounds of "largest
// remaining logit" over the eligible experts (same section; group-limited routing
// from section 2.2 and the dropless notes, section 4 step 4).
//
// bf16 path: each wave owns 16 tokens and computes a 16 x (16*NTB) tile with
// v_mfma_f32_16x16x32_bf16.  x streams from HBM straight into the A operand (its rows
// are K-contiguous, so no LDS round trip; each load instruction covers 64 contiguous
// bytes of 16 rows and a lane keeps 8 loads in flight).  The block stages its slice
// of W_g in LDS in W_g's own [k][e] layout with 16-byte copies, and the B operand
// (8 consecutive k of one expert per lane) comes out of it with the gfx950 LDS
// transpose read ds_read_b64_tr_b16.  K is split over blockIdx.y and experts over
// blockIdx.z so that small-T shapes (decode) still spread over the chip; each K
// split writes fp32 partial logits and the selection kernel adds them in split
// order, so the result is deterministic.
#include "moe_gemm_common.h"

#include <float.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

static constexpr int kRouteThreads = 256;   // 4 waves
static constexpr int kRouteTok = 64;        // tokens per block (16 per wave)
static constexpr int kRoutePair = 256;      // K per loop step: two 128-deep windows
static constexpr int kRouteMaxSplit = 8;

// Staged W_g rows per chunk and their pitch (16 bytes of pad) per expert-tile count;
// every chunk but a split's last holds an even number of steps.
template <int NTB>
struct RouteTile {
  static constexpr int kPitch = 32 * NTB + 16;
  static constexpr int kKC = NTB == 1 ? 1024 : 512;
  static constexpr int kLds = kKC * kPitch;   // 48 KB, 40 KB, 72 KB
};

// Expert tiles (of 16) per block.  With many token blocks one block covers up to 64
// experts, so x is read once for E <= 64; with few (decode) each block takes one
// tile of 16 experts, and the expert tiles supply the parallelism.
static inline int route_ntb(const moe_shape& s) {
  const int nt = (s.E + 15) / 16;
  if (ceil_div(s.T, kRouteTok) < 64) return 1;
  int b = 1;
  while (b < nt && b < 4) b *= 2;
  return b;
}

int router_nsplit(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16) return 1;
  const int ntb = route_ntb(s);
  const int64_t blocks = ceil_div(s.T, kRouteTok) * ceil_div(s.E, 16 * ntb);
  const int64_t pairs = ceil_div(s.d, kRoutePair);
  int64_t want = ceil_div(4 * 256, blocks > 0 ? blocks : 1);  // ~4 blocks per CU
  if (want > pairs) want = pairs;
  if (want > kRouteMaxSplit) want = kRouteMaxSplit;
  if (want < 1) want = 1;
  return (int)want;
}

size_t router_partial_bytes(const moe_shape& s) {
  return (size_t)router_nsplit(s) * (size_t)s.T * (size_t)s.E * sizeof(float);
}

// ---------------------------------------------------------------------------
// bf16 router GEMM on MFMA: partial[split][t][e] over the K range of this split.
// Block (x, y, z) covers tokens [64x, 64x + 64), K slice y, experts
// [16*NTB*z, 16*NTB*(z+1)).
// ---------------------------------------------------------------------------
#define MOE_LDS __attribute__((address_space(3)))
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int NTB>
__global__ void __launch_bounds__(kRouteThreads)
k_router_bf16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, int T, int d, int E,
              int k_per_split, int wg_vec, float* __restrict__ partial) {
  constexpr int EB = 16 * NTB;
  constexpr int EV = EB / 8;               // 16-byte pieces per staged k row
  constexpr int kPitch = RouteTile<NTB>::kPitch;
  constexpr int kc = RouteTile<NTB>::kKC;
  __shared__ __align__(16) unsigned char smem_raw[RouteTile<NTB>::kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;                 // k group of the MFMA operands
  const int t0 = blockIdx.x * kRouteTok + wave * 16;
  const int e0 = blockIdx.z * EB;
  const int kbeg = blockIdx.y * k_per_split;
  const int kend = min(d, kbeg + k_per_split);

  // A operand: row t0 + lane%16, k values g*8 .. g*8+7 of each 32-deep step.  The
  // loads are unconditional, from a clamped row and column: rows past T produce
  // results that are never stored, and k positions past the split meet staged W_g
  // rows that are zero (or a window whose MFMAs are skipped), so no load needs a
  // branch and the compiler can keep two steps of loads in flight.
  const int arow = t0 + (lane & 15);
  const bf16_t* xrow = x + (size_t)min(arow, T - 1) * d;
  // B operand by transpose read: in each 16-lane group, lane 4r+c addresses k row r
  // of a 4-row block, experts 4c..4c+3; lane i receives expert i's 4 k values.
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3;
  const unsigned char* bl = smem_raw + (g * 8 + tr_r) * kPitch + tr_c * 8;

  f32x4_t acc[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto b_operand = [&](int krow, int nt) {
    i16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MOE_LDS i16x4_t*)(bl + krow * kPitch + nt * 32));
    i16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MOE_LDS i16x4_t*)(bl + (krow + 4) * kPitch + nt * 32));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto load_step = [&](bf16x8_t* a, int kp) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      a[q] = *reinterpret_cast<const bf16x8_t*>(xrow + min(kp + q * 32 + g * 8, d - 8));
  };
  // Stage W_g[kc0 .. kc0+kpad)[e0 .. e0+EB) as rows of EB experts, zeros past the
  // split (kpad = klen rounded up to 128); loads batched, 8 per thread in flight.
  auto stage = [&](int kc0) {
    const int klen = min(kc, kend - kc0);
    const int kpad = (klen + 127) / 128 * 128;
    __syncthreads();
    const int total = kpad * EV;
    for (int base = 0; base < total; base += kRouteThreads * 8) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kRouteThreads + tid;
        const int kk = i / EV, ev = i % EV;
        v[u] = u32x4_t{0u, 0u, 0u, 0u};
        if (i < total && kk < klen) {
          const bf16_t* src = wg + (size_t)(kc0 + kk) * E + e0 + ev * 8;
          if (wg_vec) {                    // E % 8 == 0 and W_g 16-byte aligned
            if (e0 + ev * 8 < E) v[u] = *reinterpret_cast<const u32x4_t*>(src);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (e0 + ev * 8 + q < E) v[u][q >> 1] |= (uint32_t)src[q] << (16 * (q & 1));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kRouteThreads + tid;
        if (i < total)
          *reinterpret_cast<u32x4_t*>(smem_raw + (i / EV) * kPitch + (i % EV) * 16) = v[u];
      }
    }
    __syncthreads();
  };
  // one step: window rows [w, w+128) and, when `two`, [w+128, w+256) of the chunk
  auto compute = [&](const bf16x8_t* a, int w, bool two) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], b_operand(w + q * 32, nt),
                                                           acc[nt], 0, 0, 0);
    if (two) {
#pragma unroll
      for (int q = 4; q < 8; ++q)
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], b_operand(w + q * 32, nt),
                                                             acc[nt], 0, 0, 0);
    }
  };

  // Chunks of kc staged rows; within a chunk, steps of 256 alternate two register
  // sets: a step computes from one set while the loads of the next fill the other.
  // Loads are unconditional (clamped), so the waits stay exact; the last load of a
  // chunk fetches the first step of the next one, which overlaps its staging.
  bf16x8_t a0[8], a1[8];
  load_step(a0, kbeg);
  for (int kc0 = kbeg; kc0 < kend; kc0 += kc) {
    stage(kc0);
    const int nst = (min(kc, kend - kc0) + kRoutePair - 1) / kRoutePair;
    for (int i = 0; i < nst; i += 2) {
      load_step(a1, kc0 + (i + 1) * kRoutePair);
      compute(a0, i * kRoutePair, kc0 + i * kRoutePair + 128 < kend);
      load_step(a0, kc0 + (i + 2) * kRoutePair);
      if (i + 1 < nst)
        compute(a1, (i + 1) * kRoutePair, kc0 + (i + 1) * kRoutePair + 128 < kend);
    }
  }
  // 16x16 output layout: lane holds column lane%16, rows (lane/16)*4 + i.
  float* out = partial + (size_t)blockIdx.y * T * E;
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int e = e0 + nt * 16 + (lane & 15);
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + (lane >> 4) * 4 + i;
      if (t < T) out[(size_t)t * E + e] = acc[nt][i];
    }
  }
}

// fp32 router: one thread per (t, e) dot product (the fp32 path serves small shapes).
__global__ void k_router_f32(const float* __restrict__ x, const float* __restrict__ wg, int T, int d,
                             int E, float* __restrict__ partial) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * d;
  float acc = 0.f;
  for (int kk = 0; kk < d; ++kk) acc = fmaf(xr[kk], wg[(size_t)kk * E + e], acc);
  partial[i] = acc;
}

// ---------------------------------------------------------------------------
// Selection: G lanes per token (G = 8 .. 64, a power of two >= min(E, 64)), so a
// wave serves 64/G tokens, and each lane holds PER experts lt + G*r.  A candidate is
// one 64-bit key: the logit's bits mapped to an unsigned order (high word) and the
// complement of the expert id (low word), so the largest key is the largest logit
// and, among equal logits, the lowest id.  Each of the k rounds is one butterfly
// max over xor offsets < G, which stays inside a token's lane group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t sel_key(float v, int id) {
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);  // -0 and +0 compare equal
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)id);
}

__device__ __forceinline__ int sel_id(uint64_t key) {
  return (int)(0xffffffffu - (uint32_t)key);
}

// The logit a key was made from (the inverse of the order mapping; -0 came in as +0).
__device__ __forceinline__ float sel_value(uint64_t key) {
  const uint32_t h = (uint32_t)(key >> 32);
  return __uint_as_float((h & 0x80000000u) ? (h & 0x7fffffffu) : ~h);
}

// All-reduce over each 16-lane row of a wave with DPP moves (no LDS round trip): swaps
// inside quads (lane xor 1, xor 2), then the 8-lane and the 16-lane mirror, so that
// every lane of the row ends with the row's maximum (sum); the combining order is
// symmetric, so all 16 lanes hold bitwise the same result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f32<kDppMirror>(v));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  return v + dpp_f32<kDppMirror>(v);
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_key_step(uint64_t k) {
  const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(k >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)k);
  return o > k ? o : k;
}

__device__ __forceinline__ uint64_t row16_max_key(uint64_t k) {
  k = max_key_step<kDppXor1>(k);
  k = max_key_step<kDppXor2>(k);
  k = max_key_step<kDppHalfMirror>(k);
  return max_key_step<kDppMirror>(k);
}

template <int G>
__device__ __forceinline__ uint64_t group_max_key(uint64_t k) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

static constexpr int kSelThreads = 256;
static constexpr int kSelLds = 4096;        // floats: (256 / G) tokens x E logits

static inline int select_lanes(int E) {
  int g = 8;
  while (g < E && g < 64) g *= 2;
  return g;
}

// The k selection rounds of one token held by its G lanes (lane lt holds experts
// lt + G*r, r < PER, with logits l[r], exp(l - max) z[r], eligibility elig[r]): k rounds
// of "largest remaining eligible logit" (one 64-bit key per candidate: the logit's
// order bits above the complemented id, so ties go to the lower id), the weights
// z / S, renormalised when asked.  Every lane of the group takes part; `live` lanes
// write slot j from lane j % G.
template <int G, int PER>
__device__ __forceinline__ void select_rounds(const float* l, const float* z, const bool* elig,
                                              float S, int E, int k, int renormalize, bool live,
                                              int t, int lt, int base_lane,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w) {
  uint64_t key[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) key[r] = elig[r] ? sel_key(l[r], lt + G * r) : 0ull;
  int my_idx[PER];
  float my_w[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) { my_idx[r] = 0; my_w[r] = 0.f; }
  float wsum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t c = key[0];
#pragma unroll
    for (int r = 1; r < PER; ++r) c = key[r] > c ? key[r] : c;
    const uint64_t b = group_max_key<G>(c);
    const int e = sel_id(b);
    const int owner = e % G, rr = e / G;
    float zo = 0.f;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      if (r == rr) {
        zo = z[r];
        if (lt == owner) key[r] = 0ull;
      }
    }
    const float p = __shfl(zo, base_lane + owner, 64) / S;
    wsum += p;
    if (lt == j % G) {
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (q == j / G) { my_idx[q] = e; my_w[q] = p; }
    }
  }
  if (!live) return;
  const float scale = 1.0f / wsum;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int j = lt + G * q;
    if (j < k) {
      if (my_idx[q] < 0 || my_idx[q] >= E) MOE_DEBUG_REPORT(MOE_DBG_EXPERT_ID);
      topk_idx[(size_t)t * k + j] = my_idx[q];
      topk_w[(size_t)t * k + j] = renormalize ? my_w[q] * scale : my_w[q];
    }
  }
}

// Logits of one token from a row its G lanes can read (LDS), their softmax over all E
// in fp32 (max-subtracted; S = the group's sum).
template <int G, int PER>
__device__ __forceinline__ void load_softmax(const float* lrow, int E, int lt, bool* has, float* l,
                                             float* z, float& S) {
  float m = -FLT_MAX;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = lt + G * r;
    has[r] = e < E;
    l[r] = has[r] ? lrow[e] : -FLT_MAX;
    if (has[r]) m = fmaxf(m, l[r]);
  }
  m = group_max<G>(m);
  float zs = 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    z[r] = has[r] ? expf(l[r] - m) : 0.f;
    zs += z[r];
  }
  S = group_sum<G>(zs);
}

// Selection of one token from its E logits (bias included) in a row `lrow` that the
// token's G lanes can read (LDS): softmax, eligibility (group-limited routing: a group
// scores its largest logit, the topk_groups best groups stay, ties to the lower group
// id; n_groups <= G), then the k rounds.
template <int G, int PER>
__device__ __forceinline__ void select_token(const float* lrow, int E, int k, int n_groups,
                                             int topk_groups, int renormalize, bool live, int t,
                                             int lt, int base_lane, int32_t* __restrict__ topk_idx,
                                             float* __restrict__ topk_w) {
  bool has[PER], elig[PER];
  float l[PER], z[PER], S;
  load_softmax<G, PER>(lrow, E, lt, has, l, z, S);
#pragma unroll
  for (int r = 0; r < PER; ++r) elig[r] = has[r];
  if (n_groups > 0) {
    const int gs = E / n_groups;
    uint64_t gkey = 0;
    if (lt < n_groups) {
      float gm = -FLT_MAX;
      for (int e = lt * gs; e < (lt + 1) * gs; ++e) gm = fmaxf(gm, lrow[e]);
      gkey = sel_key(gm, lt);
    }
    uint64_t keep = 0;
    for (int r = 0; r < topk_groups; ++r) {
      const uint64_t b = group_max_key<G>(gkey);
      const int gid = sel_id(b);
      keep |= 1ull << gid;
      if (lt == gid) gkey = 0;
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) elig[r] = has[r] && ((keep >> ((lt + G * r) / gs)) & 1ull);
  }
  select_rounds<G, PER>(l, z, elig, S, E, k, renormalize, live, t, lt, base_lane, topk_idx, topk_w);
}

// The selection kernel after the split-K router: G lanes per token add the splits'
// partial logits in split order and the bias, stage the row in LDS, then select.
template <int G, int PER>
__global__ void __launch_bounds__(kSelThreads)
k_select(const float* __restrict__ partial, int nsplit, const float* __restrict__ bias, int T, int E,
         int k, int n_groups, int topk_groups, int renormalize, float* __restrict__ logits_out,
         int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float gl[kSelLds];
  constexpr int kTokPerBlock = kSelThreads / G;
  const int lt = threadIdx.x % G;          // lane within the token's group
  const int slot = threadIdx.x / G;        // token within the block
  const int base_lane = (threadIdx.x & 63) - lt;
  const int tok = blockIdx.x * kTokPerBlock + slot;
  // Groups past T compute on the last token (so every lane of a wave takes part in
  // the butterflies) and write nothing.
  const bool live = tok < T;
  const int t = live ? tok : T - 1;
  float* tl = gl + slot * E;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = lt + G * r;
    if (e >= E) continue;
    float pv[kRouteMaxSplit];
#pragma unroll
    for (int sidx = 0; sidx < kRouteMaxSplit; ++sidx)
      pv[sidx] = sidx < nsplit ? partial[((size_t)sidx * T + t) * E + e] : 0.f;
    float acc = pv[0];
#pragma unroll
    for (int sidx = 1; sidx < kRouteMaxSplit; ++sidx)
      if (sidx < nsplit) acc += pv[sidx];
    if (bias) acc += bias[e];
    tl[e] = acc;
    if (logits_out && live) logits_out[(size_t)t * E + e] = acc;
  }
  // a token's row is written and read by the lanes of one wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  select_token<G, PER>(tl, E, k, n_groups, topk_groups, renormalize, live, t, lt, base_lane,
                       topk_idx, topk_w);
}

// ---------------------------------------------------------------------------
// Fused router for large T (bf16, E a multiple of 8 up to 64, d a multiple of the
// slice depth): one block of 4 waves owns TB tokens and the whole of K, so the logits
// are complete inside the block and the selection runs there too (no partial logits,
// no second launch).  x streams through an LDS ring of NS slices with 16-byte
// global->LDS copies whose 64 lanes cover 1 KB: two (or four) rows of 512 (256)
// contiguous bytes, instead of the 64 bytes per row a direct A-operand load covers.
// A slice also holds W_g's rows [k0, k0 + SK) - one contiguous piece of W_g - read as
// the B operand with ds_read_b64_tr_b16.  Each wave owns a 16-token MFMA tile (with
// TB < 64, TB / 16 tiles: the waves of a tile split its 32-deep steps and their partial
// logits are added in a fixed order through LDS), so a tile's logits end up in one
// wave's registers, where 16 lanes per token select with DPP reductions.
// ---------------------------------------------------------------------------
// Group-limited eligibility of one token by one lane (E <= 64): a group (n_groups
// contiguous id ranges) scores its largest logit, the topk_groups best groups stay
// (scanned upwards with a strict comparison: ties to the lower group id); returns the
// mask of eligible experts.  lrow[e * stride] holds the token's logits.
__device__ __forceinline__ uint64_t group_keep_mask(const float* lrow, int stride, int E,
                                                    int n_groups, int topk_groups) {
  const int gs = E / n_groups;
  uint64_t taken = 0;
  for (int r = 0; r < topk_groups; ++r) {
    int best = -1;
    float bv = -FLT_MAX;
    for (int gi = 0; gi < n_groups; ++gi) {
      if ((taken >> gi) & 1ull) continue;
      float gm = -FLT_MAX;
      for (int e = gi * gs; e < (gi + 1) * gs; ++e) gm = fmaxf(gm, lrow[e * stride]);
      if (best < 0 || gm > bv) {
        best = gi;
        bv = gm;
      }
    }
    taken |= 1ull << best;
  }
  uint64_t keep = 0;
  for (int e = 0; e < E; ++e)
    if ((taken >> (e / gs)) & 1ull) keep |= 1ull << e;
  return keep;
}

// W_g chunk permutation of the fused router at a 128-byte row pitch: the 8 rows that one
// transposed B read touches at one bank half (row bits 1 and 3-4 vary) get 8 different
// chunks.
__device__ __forceinline__ int wg_swz(int row) { return 2 * ((row >> 3) & 3) + ((row >> 1) & 1); }

static constexpr int kRfThreads = 256;
static constexpr int kRfLds = 160 * 1024;

// Slice depth: the largest power of two up to 256 whose slice (TB rows of x and SK
// rows of W_g) stays within 20 KB, but at least one 1 KB copy per wave of x; W_g's
// region is padded to whole copies per wave (the padding is never read).
template <int TB, int E8>
struct RouteFused {
  static constexpr int EP = 8 * E8;                               // experts, padded to 8
  static constexpr int NT = EP <= 16 ? 1 : EP / 16;               // 16-expert MFMA tiles
  static constexpr int SK0 = 20480 / (2 * (TB + EP));
  static constexpr int SKa = SK0 >= 256 ? 256 : SK0 >= 128 ? 128 : 64;
  static constexpr int SK = TB * SKa * 2 >= 4096 ? SKa : 4096 / (2 * TB);
  static constexpr int XB = TB * SK * 2;                          // x bytes per slice
  static constexpr int CX = XB / 4096;                            // x copies per wave
  static constexpr int CW = (SK * EP * 2 + 4095) / 4096;          // W_g copies per wave
  static constexpr int WB = CW * 4096;                            // W_g region per slice
  static constexpr int kSlot = XB + WB + 256;                     // + tr-read overrun slack
  static constexpr int NS = (kRfLds / kSlot) < 12 ? (kRfLds / kSlot) : 12;
  static constexpr int CPW = CX + CW;
  static constexpr int KS = SK / 32;                              // 32-deep steps per slice
  static constexpr int SWZ = (SK / 8 - 1) < 15 ? SK / 8 - 1 : 15;  // x chunk swizzle mask
  static_assert(CX >= 1 && XB % 4096 == 0, "x copy split");
  static_assert(NS >= 3 && (NS - 2) * CPW <= 63, "ring depth");
  static_assert(KS == 2 || KS == 4 || KS == 8, "steps per slice");
  static_assert(TB == 16 || TB == 32 || TB == 64, "16-token tiles over 4 waves");
  static_assert(4 * 64 * NT * 16 + 4 * 16 * 16 * NT * 4 <= NS * kSlot,
                "partial-logit and selection space");
  static_assert(E8 != 8 || SK * 128 <= CW * 4096, "swizzled W_g rows fit the region");
};

template <int TB, int E8>
__global__ void __launch_bounds__(kRfThreads, 1)
k_route_fused(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
              const float* __restrict__ bias, int T, int d, int E, int k, int n_groups,
              int topk_groups, int renormalize, float* __restrict__ logits_out,
              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  using C = RouteFused<TB, E8>;
  constexpr int SK = C::SK, NS = C::NS, CX = C::CX, CW = C::CW, KS = C::KS;
  constexpr int NT = C::NT;
  constexpr int kPitch = SK * 2;                  // bytes per staged x row
  __shared__ __align__(1024) unsigned char lds[NS * C::kSlot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int nsl = d / SK;
  const int wrow = E * 2;                          // bytes per W_g row

  // per-lane global offsets of this wave's copies (the same in every slice)
  uint32_t xoff[CX], woff[CW];
#pragma unroll
  for (int c = 0; c < CX; ++c) {
    const int p = (wave * CX + c) * 1024 + lane * 16;   // byte position in the x region
    const int row = p / kPitch, pc = (p % kPitch) / 16;
    const int lc = pc ^ (row & C::SWZ);                       // logical 16-byte chunk
    const int rowc = min(t0 + row, T - 1) - t0;
    xoff[c] = (uint32_t)(rowc * d * 2 + lc * 16);
  }
  const int wslice = SK * wrow;                    // real W_g bytes per slice
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    if constexpr (E8 == 8) {
      // 33..64 experts: W_g rows staged at a 128-byte pitch with their 16-byte chunks
      // permuted (physical chunk = logical ^ wg_swz(row)), so that the transposed B
      // reads spread over all banks; chunks past E's read chunk 0 (never used)
      const int P = ((wave * CW + c) * 64 + lane) * 16;
      const int row = P >> 7;
      const int lc = ((P >> 4) & 7) ^ wg_swz(row);
      woff[c] = (uint32_t)(min(row, SK - 1) * wrow + (lc * 8 < E ? lc : 0) * 16);
    } else {
      woff[c] = (uint32_t)min(((wave * CW + c) * 64 + lane) * 16, wslice - 16);
    }
  }

  // Blocks start at different slices (block b at slice b mod nsl, then wrapping round),
  // so that blocks running at the same time read different pieces of W_g rather than
  // all reading one piece from the same few L2 channels.  Each block's order is fixed.
  const int rot = blockIdx.x % nsl;
  auto issue = [&](int j) {                        // slice j of this block into slot j % NS
    int js = min(j, nsl - 1) + rot;
    if (js >= nsl) js -= nsl;
    unsigned char* slot = lds + (j % NS) * C::kSlot;
    const bf16_t* xb = uniform_ptr(x + (size_t)t0 * d + (size_t)js * SK);
    const bf16_t* wb = uniform_ptr(wg + (size_t)js * SK * E);
#pragma unroll
    for (int c = 0; c < CX; ++c) copy16_to_lds(xb, xoff[c], slot + (wave * CX + c) * 1024);
#pragma unroll
    for (int c = 0; c < CW; ++c) copy16_to_lds(wb, woff[c], slot + C::XB + (wave * CW + c) * 1024);
  };

  // Work split: 16-token MFMA tiles, NTT = TB / 16 of them; wave w owns tile w % NTT
  // and, when there are fewer tiles than waves, the k-phase w / NTT of KW = 4 / NTT:
  // the 32-deep steps kk = phase, phase + KW, ... of every slice.
  constexpr int NTT = TB / 16, KW = 4 / NTT;
  const int tw = wave % NTT, kw = wave / NTT;
  const int g = lane >> 4, r16 = lane & 15;
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3;
  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the bias of the lane's experts (16 nt + l % 16 in the MFMA output), loaded before
  // the ring fills so that its latency hides behind the loop (an extra older load only
  // makes the copy waits below wait longer, never shorter)
  float bv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = (lane & 15) + 16 * nt;
    bv[nt] = (bias && e < E) ? bias[e] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) issue(j);
  for (int j = 0; j < nsl; ++j) {
    MOE_WAIT_VMCNT((NS - 2) * (CX + CW));
    __syncthreads();
    issue(j + NS - 1);
    const unsigned char* slot = lds + (j % NS) * C::kSlot;
    const unsigned char* wl = slot + C::XB;
#pragma unroll
    for (int q = 0; q < (KS + KW - 1) / KW; ++q) {
      const int kk = kw + KW * q;                  // this wave's 32-deep step
      if (KS % KW != 0 && kk >= KS) break;
      bf16x8_t bop[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const unsigned char* bp;
        int bpitch;
        if constexpr (E8 == 8) {
          // row kk*32 + g*8 + tr_r: its swizzle is 2g + tr_r / 2 (rows +4 the same)
          bp = wl + (kk * 32 + g * 8 + tr_r) * 128 +
               (((2 * nt + (tr_c >> 1)) ^ (2 * g + (tr_r >> 1))) * 16) + (tr_c & 1) * 8;
          bpitch = 128;
        } else {
          bp = wl + (kk * 32 + g * 8 + tr_r) * wrow + nt * 32 + tr_c * 8;
          bpitch = wrow;
        }
        const i16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)bp);
        const i16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(bp + 4 * bpitch));
        bop[nt] = __builtin_bit_cast(bf16x8_t,
                                     __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      const int row = tw * 16 + r16;
      const int pc = (kk * 4 + g) ^ (row & C::SWZ);
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(slot + row * kPitch + pc * 16);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nt], acc[nt], 0, 0, 0);
    }
  }
  MOE_WAIT_VMCNT(0);                               // the copies past the last slice
  __syncthreads();

  // k-phases of one tile: phases 1.. leave their partial logits in LDS (each lane its
  // own 4 NT values), phase 0 adds them in phase order (deterministic)
  float* red = reinterpret_cast<float*>(lds);
  if constexpr (KW > 1) {
    if (kw > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4_t*>(red + ((wave * 64 + lane) * NT + nt) * 4) = acc[nt];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int ph = 1; ph < KW; ++ph)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x4_t o =
              *reinterpret_cast<const f32x4_t*>(red + (((ph * NTT + tw) * 64 + lane) * NT + nt) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nt][i] += o[i];
        }
    }
  }

  if (kw != 0) return;   // (no block-wide barrier follows)

  // The tile's logits are in registers (16x16 MFMA output: element i of lane l is
  // token (l / 16) * 4 + i of the tile, expert 16 nt + l % 16).  Bias, the optional
  // logits store, then the logits move through a wave-private LDS patch [16 NT][16]
  // (token-minor) to the selection layout: 4 lanes per token, lane lq holding experts
  // lq + 4 r (r < 4 NT), one token per lane quad, 16 tokens per wave at once.
  constexpr int EPT = 16 * NT;                     // expert columns of the tile
  constexpr int PER = EPT / 4;
  float* lgw = red + (KW > 1 ? 4 * 64 * NT * 4 : 0) + wave * 16 * EPT;
  {
    const int lt = lane & 15;
    const int tt0 = tw * 16 + g * 4;               // the lane's first token in the block
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = lt + 16 * nt;
      const bool he = e < E;
      const float b = bv[nt];
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = acc[nt][i] + b;
        if (logits_out && he && t0 + tt0 + i < T) logits_out[(size_t)(t0 + tt0 + i) * E + e] = v[i];
      }
      *reinterpret_cast<f32x4_t*>(lgw + e * 16 + g * 4) = v;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int tk = lane >> 2, lq = lane & 3;
  const int t = t0 + tw * 16 + tk;
  float l[PER], z[PER];
  bool has[PER];
  float m = -FLT_MAX;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = lq + 4 * r;
    has[r] = e < E;
    l[r] = has[r] ? lgw[e * 16 + tk] : -FLT_MAX;
    m = fmaxf(m, l[r]);
  }
  m = fmaxf(m, dpp_f32<kDppXor1>(m));
  m = fmaxf(m, dpp_f32<kDppXor2>(m));
  float zs = 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    z[r] = has[r] ? expf(l[r] - m) : 0.f;
    zs += z[r];
  }
  zs += dpp_f32<kDppXor1>(zs);
  const float S = zs + dpp_f32<kDppXor2>(zs);
  // group-limited eligibility: each of the token's lanes forms the same mask
  const uint64_t keep = n_groups > 0 ? group_keep_mask(lgw + tk, 16, E, n_groups, topk_groups) : ~0ull;
  // k rounds of "largest remaining eligible logit, ties to the lower id": the quad's
  // largest value (a local tree, then two DPP steps), the lowest id holding it (the
  // same), and that entry taken out (-inf).  -0 and +0 compare equal, as in the keys
  // of the other selection paths.
  float lv[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) lv[r] = (has[r] && ((keep >> (lq + 4 * r)) & 1ull)) ? l[r] : -INFINITY;
  // the round's weights wait in the wave's patch (its logits are all read by now)
  // until the renormalisation scale is known: slot j of the token at lgw[tk * EPT + j]
  float* pw = lgw + tk * EPT;
  float wsum = 0.f;
  for (int j = 0; j < k; ++j) {
    float c[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) c[r] = lv[r];
#pragma unroll
    for (int w = PER / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) c[r] = fmaxf(c[r], c[r + w]);
    float mq = fmaxf(c[0], dpp_f32<kDppXor1>(c[0]));
    mq = fmaxf(mq, dpp_f32<kDppXor2>(mq));
    int id = 1 << 30;
#pragma unroll
    for (int r = PER - 1; r >= 0; --r)
      if (lv[r] == mq) id = lq + 4 * r;
    id = min(id, (int)dpp_u32<kDppXor1>((uint32_t)id));
    id = min(id, (int)dpp_u32<kDppXor2>((uint32_t)id));
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (lq + 4 * r == id) lv[r] = -INFINITY;
    // the winner's weight: exactly the owner's exp(l - m), computed by every lane
    const float p = expf(mq - m) / S;
    wsum += p;
    if (lq == (j & 3)) {
      if (t < T && (id < 0 || id >= E)) MOE_DEBUG_REPORT(MOE_DBG_EXPERT_ID);
      if (t < T) topk_idx[(size_t)t * k + j] = id;
      pw[j] = p;
    }
  }
  if (t < T) {
    const float scale = 1.0f / wsum;
    for (int j = lq; j < k; j += 4) topk_w[(size_t)t * k + j] = renormalize ? pw[j] * scale : pw[j];
  }
}

// The fused router applies to bf16, E a multiple of 8 up to 64 and T >= 4096 (at least
// 256 blocks of 16 tokens), with d a multiple of the slice depth; 16, 32 or 64 tokens
// per block as T grows.
static int e8_of(int E) { return E <= 8 ? 1 : E <= 16 ? 2 : E <= 32 ? 4 : 8; }

static int route_fused_sk(int tb, int E) {
  switch (tb * 16 + e8_of(E)) {
#define MOE_RF_SK(TBV, E8V) case TBV * 16 + E8V: return RouteFused<TBV, E8V>::SK;
    MOE_RF_SK(16, 1) MOE_RF_SK(16, 2) MOE_RF_SK(16, 4) MOE_RF_SK(16, 8)
    MOE_RF_SK(32, 1) MOE_RF_SK(32, 2) MOE_RF_SK(32, 4) MOE_RF_SK(32, 8)
    MOE_RF_SK(64, 1) MOE_RF_SK(64, 2) MOE_RF_SK(64, 4) MOE_RF_SK(64, 8)
#undef MOE_RF_SK
    default: return 1 << 30;
  }
}

static int route_fused_tb(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16 || s.E % 8 || s.E > 64 || s.T < 4096) return 0;
  const int tb = s.T >= 16384 ? 64 : (s.T >= 8192 ? 32 : 16);
  // per-lane copy offsets reach tb rows of x: 32-bit byte offsets
  if ((int64_t)tb * s.d * 2 >= ((int64_t)1 << 31)) return 0;
  return s.d % route_fused_sk(tb, s.E) == 0 ? tb : 0;
}

bool route_is_fused(const moe_shape& s) { return route_fused_tb(s) > 0; }

template <int TB, int E8>
static void launch_route_fused_tb(const moe_shape& s, const bf16_t* x, const bf16_t* wg,
                                  const float* bias, float* logits, int32_t* topk_idx,
                                  float* topk_w, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(s.T, TB));
  hipLaunchKernelGGL((k_route_fused<TB, E8>), grid, dim3(kRfThreads), 0, st, x, wg, bias, s.T, s.d,
                     s.E, s.k, s.n_groups, s.topk_groups, s.renormalize, logits, topk_idx, topk_w);
}

moe_status launch_route(const moe_shape& s, const void* x, const void* w_gate, const float* bias,
                        float* logits, int32_t* topk_idx, float* topk_w, float* partial,
                        hipStream_t st) {
  if (const int tb = route_fused_tb(s)) {
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_gate);
    const int e8 = e8_of(s.E);
#define MOE_RF_TB(TBV)                                                                      \
  do {                                                                                      \
    if (e8 == 1) launch_route_fused_tb<TBV, 1>(s, xb, wb, bias, logits, topk_idx, topk_w, st); \
    else if (e8 == 2) launch_route_fused_tb<TBV, 2>(s, xb, wb, bias, logits, topk_idx, topk_w, st); \
    else if (e8 == 4) launch_route_fused_tb<TBV, 4>(s, xb, wb, bias, logits, topk_idx, topk_w, st); \
    else launch_route_fused_tb<TBV, 8>(s, xb, wb, bias, logits, topk_idx, topk_w, st);     \
  } while (0)
    if (tb == 16) MOE_RF_TB(16);
    else if (tb == 32) MOE_RF_TB(32);
    else MOE_RF_TB(64);
#undef MOE_RF_TB
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  const int nsplit = router_nsplit(s);
  if (s.dtype == MOE_DTYPE_BF16) {
    const int ntb = route_ntb(s);
    const int64_t pairs = ceil_div(s.d, kRoutePair);
    const int k_per_split = (int)(ceil_div(pairs, nsplit) * kRoutePair);
    dim3 grid((unsigned)ceil_div(s.T, kRouteTok), (unsigned)nsplit,
              (unsigned)ceil_div(s.E, 16 * ntb));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_gate);
    const int wg_vec = (s.E % 8 == 0) && (reinterpret_cast<uintptr_t>(w_gate) & 15u) == 0;
#define MOE_ROUTER_LAUNCH(NTBV)                                                               \
  hipLaunchKernelGGL(k_router_bf16<NTBV>, grid, dim3(kRouteThreads), 0, st, xb, wb, s.T, s.d, \
                     s.E, k_per_split, wg_vec, partial)
    switch (ntb) {
      case 1: MOE_ROUTER_LAUNCH(1); break;
      case 2: MOE_ROUTER_LAUNCH(2); break;
      default: MOE_ROUTER_LAUNCH(4); break;
    }
#undef MOE_ROUTER_LAUNCH
  } else {
    int64_t n = (int64_t)s.T * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_gate), s.T, s.d,
                       s.E, partial);
  }
  if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  const int G = select_lanes(s.E);
  int per = 1;
  while (per * G < s.E) per *= 2;
  const dim3 sgrid((unsigned)ceil_div(s.T, kSelThreads / G));
#define MOE_SELECT_LAUNCH(GV, PV)                                                              \
  hipLaunchKernelGGL((k_select<GV, PV>), sgrid, dim3(kSelThreads), 0, st, partial, nsplit, bias, \
                     s.T, s.E, s.k, s.n_groups, s.topk_groups, s.renormalize, logits, topk_idx, \
                     topk_w)
  if (G == 8) MOE_SELECT_LAUNCH(8, 1);
  else if (G == 16) MOE_SELECT_LAUNCH(16, 1);
  else if (G == 32) MOE_SELECT_LAUNCH(32, 1);
  else if (per == 1) MOE_SELECT_LAUNCH(64, 1);
  else if (per == 2) MOE_SELECT_LAUNCH(64, 2);
  else if (per == 4) MOE_SELECT_LAUNCH(64, 4);
  else if (per == 8) MOE_SELECT_LAUNCH(64, 8);
  else MOE_SELECT_LAUNCH(64, 16);
#undef MOE_SELECT_LAUNCH
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
