// Router GEMM and expert selection.
//
// logits = x[T, d] @ W_g[d, E] (+ bias) is a GEMM with M = T, N = E, K = d; it does
// no heavy arithmetic and is bound by reading x once (TileLang chapter "MoE, MLA and
// sparse-attention operators", section 2.2).  Selection is k rounds of "largest
// remaining logit" over the eligible experts (same section; group-limited routing
// from section 2.2 and the dropless notes, section 4 step 4).
//
// bf16 path: each wave owns 16 tokens and computes a 16 x E tile with
// v_mfma_f32_16x16x32_bf16.  x streams from HBM straight into the A operand (its rows
// are K-contiguous, so no LDS round trip); the block stages W_g^T for its K slice in
// LDS, shared by the 4 waves.  K is split over blockIdx.y so small-T shapes (decode)
// still spread over the chip; each split writes fp32 partial logits and the
// selection kernel adds them in split order, so the result is deterministic.
#include "moe_internal.h"

#include <float.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

static constexpr int kRouteThreads = 256;   // 4 waves
static constexpr int kRouteTok = 64;        // tokens per block (16 per wave)
static constexpr int kRouteLdsElems = 32768;  // W_g^T chunk: 64 KB of bf16

// Expert tiles (of 16) per block: enough to cover E up to 256 in one block.
static inline int route_ntb(int E) {
  int nt = (E + 15) / 16;
  int b = 1;
  while (b < nt && b < 16) b *= 2;
  return b;
}

static inline int route_kc(int ntb) {
  // K chunk staged in LDS: 16*ntb * (KC + 8) bf16 <= 32768 elements, KC % 32 == 0.
  int kc = (kRouteLdsElems / (16 * ntb) - 8) / 32 * 32;
  if (kc > 2048) kc = 2048;
  if (kc < 32) kc = 32;
  return kc;
}

int router_nsplit(const moe_shape& s) {
  if (s.dtype != MOE_DTYPE_BF16) return 1;
  int64_t tok_blocks = ceil_div(s.T, kRouteTok);
  int64_t ksteps = ceil_div(s.d, 32);
  int64_t want = ceil_div(2 * 256, tok_blocks > 0 ? tok_blocks : 1);  // ~2 blocks per CU
  if (want > ksteps) want = ksteps;
  if (want > 64) want = 64;
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
template <int NTB>
__global__ void __launch_bounds__(kRouteThreads)
k_router_bf16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, int T, int d, int E,
              int k_per_split, int kc, float* __restrict__ partial) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* wsT = reinterpret_cast<bf16_t*>(smem_raw);  // [16*NTB][kc + 8]
  constexpr int EB = 16 * NTB;
  const int ldw = kc + 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTok + wave * 16;
  const int e0 = blockIdx.z * EB;
  const int kbeg = blockIdx.y * k_per_split;
  const int kend = min(d, kbeg + k_per_split);

  // A operand: row t0 + lane%16, 8 k values at (lane/16)*8 within each 32-wide step.
  const int arow = t0 + (lane & 15);
  const int akoff = (lane >> 4) * 8;
  const bool arow_ok = arow < T;
  const bf16_t* xrow = x + (size_t)(arow_ok ? arow : 0) * d;

  f32x4_t acc[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kc0 = kbeg; kc0 < kend; kc0 += kc) {
    const int klen = min(kc, kend - kc0);
    const int kpad = (klen + 31) / 32 * 32;
    __syncthreads();
    // Stage W_g[kc0 .. kc0+klen)[e0 .. e0+EB) transposed into wsT[e][k]; zeros outside.
    for (int i = tid; i < kpad * EB; i += kRouteThreads) {
      const int e = i % EB;
      const int kk = i / EB;
      bf16_t v = 0;
      if (e0 + e < E && kk < klen) v = wg[(size_t)(kc0 + kk) * E + e0 + e];
      wsT[e * ldw + kk] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int ks = 0; ks < kpad; ks += 32) {
      const int kg = kc0 + ks + akoff;
      bf16x8_t a;
      if (arow_ok && kg < kend) {
        a = *reinterpret_cast<const bf16x8_t*>(xrow + kg);
      } else {
        a = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        const bf16x8_t b =
            *reinterpret_cast<const bf16x8_t*>(wsT + (nt * 16 + (lane & 15)) * ldw + ks + akoff);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nt], 0, 0, 0);
      }
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
// Selection: one wave per token.
// ---------------------------------------------------------------------------
struct Cand {
  float v;
  int e;
  int ok;  // 1 = a real candidate
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  if (a.ok != b.ok) return a.ok > b.ok;
  if (a.v != b.v) return a.v > b.v;
  return a.e < b.e;
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Cand o;
    o.v = __shfl_xor(c.v, off, 64);
    o.e = __shfl_xor(c.e, off, 64);
    o.ok = __shfl_xor(c.ok, off, 64);
    if (better(o, c)) c = o;
  }
  return c;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

static constexpr int kSelMaxPerLane = 16;   // E <= 1024
static constexpr int kSelWaves = 4;

__global__ void __launch_bounds__(64 * kSelWaves)
k_select(const float* __restrict__ partial, int nsplit, const float* __restrict__ bias, int T, int E,
         int k, int n_groups, int topk_groups, int renormalize, float* __restrict__ logits_out,
         int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float gl[kSelWaves][1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kSelWaves + wave;
  if (t >= T) return;  // wave-uniform
  const int per = (E + 63) / 64;

  float l[kSelMaxPerLane];
#pragma unroll
  for (int r = 0; r < kSelMaxPerLane; ++r) {
    const int e = lane + 64 * r;
    float v = -FLT_MAX;
    if (r < per && e < E) {
      float acc = 0.f;
      for (int sidx = 0; sidx < nsplit; ++sidx) acc += partial[((size_t)sidx * T + t) * E + e];
      if (bias) acc += bias[e];
      v = acc;
      if (logits_out) logits_out[(size_t)t * E + e] = v;
    }
    l[r] = v;
  }
  // softmax over all E in fp32 (max-subtracted)
  float m = -FLT_MAX;
#pragma unroll
  for (int r = 0; r < kSelMaxPerLane; ++r)
    if (r < per && lane + 64 * r < E) m = fmaxf(m, l[r]);
  m = wave_max(m);
  float z[kSelMaxPerLane];
  float zs = 0.f;
#pragma unroll
  for (int r = 0; r < kSelMaxPerLane; ++r) {
    z[r] = 0.f;
    if (r < per && lane + 64 * r < E) {
      z[r] = expf(l[r] - m);
      zs += z[r];
    }
  }
  const float S = wave_sum(zs);

  // eligibility (group-limited routing)
  unsigned elig = 0;  // bit r: expert lane + 64r eligible
#pragma unroll
  for (int r = 0; r < kSelMaxPerLane; ++r)
    if (r < per && lane + 64 * r < E) elig |= 1u << r;
  if (n_groups > 0) {
    const int gs = E / n_groups;
#pragma unroll
    for (int r = 0; r < kSelMaxPerLane; ++r)
      if (r < per && lane + 64 * r < E) gl[wave][lane + 64 * r] = l[r];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    Cand g{-FLT_MAX, 0x7fffffff, 0};
    if (lane < n_groups) {
      float gm = -FLT_MAX;
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) gm = fmaxf(gm, gl[wave][e]);
      g = Cand{gm, lane, 1};
    }
    uint64_t keep = 0;
    for (int r = 0; r < topk_groups; ++r) {
      const Cand b = wave_best(g);
      keep |= 1ull << b.e;
      if (lane == b.e) g.ok = 0;
    }
    unsigned el = 0;
#pragma unroll
    for (int r = 0; r < kSelMaxPerLane; ++r) {
      const int e = lane + 64 * r;
      if (r < per && e < E && ((keep >> (e / gs)) & 1ull)) el |= 1u << r;
    }
    elig = el;
  }

  // k rounds of "largest remaining eligible logit", ties to the lower id
  int my_idx[kSelMaxPerLane];
  float my_w[kSelMaxPerLane];
  float wsum = 0.f;
  for (int j = 0; j < k; ++j) {
    Cand c{-FLT_MAX, 0x7fffffff, 0};
#pragma unroll
    for (int r = 0; r < kSelMaxPerLane; ++r) {
      if ((elig >> r) & 1u) {
        Cand o{l[r], lane + 64 * r, 1};
        if (better(o, c)) c = o;
      }
    }
    const Cand b = wave_best(c);
    const int owner = b.e & 63, rr = b.e >> 6;
    float p = 0.f;
#pragma unroll
    for (int r = 0; r < kSelMaxPerLane; ++r)
      if (r == rr) p = z[r];
    p = __shfl(p, owner, 64) / S;
    if (lane == owner) elig &= ~(1u << rr);
    wsum += p;
    if (lane == (j & 63)) {
#pragma unroll
      for (int q = 0; q < kSelMaxPerLane; ++q)
        if (q == (j >> 6)) { my_idx[q] = b.e; my_w[q] = p; }
    }
  }
  const float scale = renormalize ? 1.0f / wsum : 1.0f;
#pragma unroll
  for (int q = 0; q < kSelMaxPerLane; ++q) {
    const int j = lane + 64 * q;
    if (j < k) {
      topk_idx[(size_t)t * k + j] = my_idx[q];
      topk_w[(size_t)t * k + j] = renormalize ? my_w[q] * scale : my_w[q];
    }
  }
}

moe_status launch_route(const moe_shape& s, const void* x, const void* w_gate, const float* bias,
                        float* logits, int32_t* topk_idx, float* topk_w, float* partial,
                        hipStream_t st) {
  const int nsplit = router_nsplit(s);
  if (s.dtype == MOE_DTYPE_BF16) {
    const int ntb = route_ntb(s.E);
    const int kc = route_kc(ntb);
    int64_t ksteps = ceil_div(s.d, 32);
    int k_per_split = (int)(ceil_div(ksteps, nsplit) * 32);
    dim3 grid((unsigned)ceil_div(s.T, kRouteTok), (unsigned)nsplit,
              (unsigned)ceil_div(s.E, 16 * ntb));
    size_t lds = (size_t)16 * ntb * (kc + 8) * sizeof(bf16_t);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_gate);
    switch (ntb) {
      case 1: hipLaunchKernelGGL(k_router_bf16<1>, grid, dim3(kRouteThreads), lds, st, xb, wb, s.T, s.d, s.E, k_per_split, kc, partial); break;
      case 2: hipLaunchKernelGGL(k_router_bf16<2>, grid, dim3(kRouteThreads), lds, st, xb, wb, s.T, s.d, s.E, k_per_split, kc, partial); break;
      case 4: hipLaunchKernelGGL(k_router_bf16<4>, grid, dim3(kRouteThreads), lds, st, xb, wb, s.T, s.d, s.E, k_per_split, kc, partial); break;
      case 8: hipLaunchKernelGGL(k_router_bf16<8>, grid, dim3(kRouteThreads), lds, st, xb, wb, s.T, s.d, s.E, k_per_split, kc, partial); break;
      default: hipLaunchKernelGGL(k_router_bf16<16>, grid, dim3(kRouteThreads), lds, st, xb, wb, s.T, s.d, s.E, k_per_split, kc, partial); break;
    }
  } else {
    int64_t n = (int64_t)s.T * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_gate), s.T, s.d,
                       s.E, partial);
  }
  if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  hipLaunchKernelGGL(k_select, dim3((unsigned)ceil_div(s.T, kSelWaves)), dim3(64 * kSelWaves), 0, st,
                     partial, nsplit, bias, s.T, s.E, s.k, s.n_groups, s.topk_groups, s.renormalize,
                     logits, topk_idx, topk_w);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
