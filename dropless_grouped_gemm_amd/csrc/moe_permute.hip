// Permute (in-card dispatch) and combine: the two stages of the MoE layer that do no
// matrix multiply and only move rows (TileLang chapter "MoE, MLA and sparse-attention
// operators", sections 2.3 and 2.5; dropless notes section 4, steps 5-6 and 10-11).
//
// Both are HBM-bound.  Work is split into (token, column chunk) items, one wave per
// item, with 16-byte vector loads and stores along the row, so every row is read or
// written as contiguous, fully coalesced pieces and even a few tokens (decode) spread
// over many waves.  A token's k destination (or source) rows and weights are loaded
// once per item, one slot per lane, and handed out with lane shuffles.
//   permute: read a chunk of x[t] once, write it to its k rows pos[t*k + j].
//   combine: read the chunk of the token's k expert rows (and the shared-expert
//            row), several slots' loads in flight at once, weight them in fp32 in
//            slot order j = 0..k-1, round once, write out[t].
// No atomics: every output row has exactly one writer, so results are reproducible.
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

static constexpr int kTokWaves = 4;    // waves per block
static constexpr int kPermVec = 8;     // permute: 16-byte vectors per lane per item
static constexpr int kCombVec = 4;     // combine: 16-byte vectors per lane per item
static constexpr int kCombSlots = 4;   // combine: slots whose loads are in flight together

__global__ void __launch_bounds__(64 * kTokWaves)
k_permute(const u32x4_t* __restrict__ x, const int32_t* __restrict__ pos, int T, int k,
          int nvec /* 16-byte vectors per row */, int64_t max_rows, u32x4_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (nvec + 64 * kPermVec - 1) / (64 * kPermVec);
  const int64_t items = (int64_t)T * nchunk;
  for (int64_t it = (int64_t)blockIdx.x * kTokWaves + wave; it < items;
       it += (int64_t)gridDim.x * kTokWaves) {
    const int t = (int)(it / nchunk);
    const int v0 = (int)(it % nchunk) * 64 * kPermVec;
    const u32x4_t* src = x + (size_t)t * nvec;
    u32x4_t r[kPermVec];
#pragma unroll
    for (int i = 0; i < kPermVec; ++i) {
      const int v = v0 + i * 64 + lane;
      if (v < nvec) r[i] = __builtin_nontemporal_load(src + v);
    }
    for (int j0 = 0; j0 < k; j0 += 64) {
      const int nj = min(64, k - j0);
      const int pl = lane < nj ? pos[(size_t)t * k + j0 + lane] : -1;
      for (int jj = 0; jj < nj; ++jj) {
        const int p = __shfl(pl, jj, 64);
        if (p < -1 || p >= max_rows) MOE_DEBUG_REPORT(MOE_DBG_POSITION);
        if (p < 0 || p >= max_rows) continue;
        u32x4_t* dst = x_perm + (size_t)p * nvec;
#pragma unroll
        for (int i = 0; i < kPermVec; ++i) {
          const int v = v0 + i * 64 + lane;
          if (v < nvec) dst[v] = r[i];
        }
      }
    }
  }
}

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int kN = 8;
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4_t pack(const float* f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};
template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4_t pack(const float* f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

template <typename T>
__global__ void __launch_bounds__(64 * kTokWaves)
k_combine(const u32x4_t* __restrict__ y, const int32_t* __restrict__ pos,
          const float* __restrict__ w, const u32x4_t* __restrict__ shared, int Tn, int k,
          int nvec, int64_t max_rows, u32x4_t* __restrict__ out) {
  constexpr int N = Vec16<T>::kN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = (nvec + 64 * kCombVec - 1) / (64 * kCombVec);
  const int64_t items = (int64_t)Tn * nchunk;
  for (int64_t it = (int64_t)blockIdx.x * kTokWaves + wave; it < items;
       it += (int64_t)gridDim.x * kTokWaves) {
    const int t = (int)(it / nchunk);
    const int v0 = (int)(it % nchunk) * 64 * kCombVec;
    float acc[kCombVec][N];
#pragma unroll
    for (int i = 0; i < kCombVec; ++i)
#pragma unroll
      for (int q = 0; q < N; ++q) acc[i][q] = 0.f;
    u32x4_t sh[kCombVec];
    if (shared) {
      const u32x4_t* src = shared + (size_t)t * nvec;
#pragma unroll
      for (int i = 0; i < kCombVec; ++i) {
        const int v = v0 + i * 64 + lane;
        if (v < nvec) sh[i] = __builtin_nontemporal_load(src + v);
      }
    }
    for (int j0 = 0; j0 < k; j0 += 64) {
      const int nj = min(64, k - j0);
      const int pl = lane < nj ? pos[(size_t)t * k + j0 + lane] : -1;
      const float wl = lane < nj ? (w ? w[(size_t)t * k + j0 + lane] : 1.f) : 0.f;
      for (int jj = 0; jj < nj; jj += kCombSlots) {
        // issue every load of kCombSlots slots, then accumulate them in slot order
        u32x4_t r[kCombSlots][kCombVec];
        bool ok[kCombSlots];
#pragma unroll
        for (int u = 0; u < kCombSlots; ++u) {
          const int p = __shfl(pl, min(jj + u, 63), 64);
          ok[u] = jj + u < nj && p >= 0 && p < max_rows;
          if (jj + u < nj && (p < -1 || p >= max_rows)) MOE_DEBUG_REPORT(MOE_DBG_POSITION);
          const u32x4_t* src = y + (size_t)(ok[u] ? p : 0) * nvec;
#pragma unroll
          for (int i = 0; i < kCombVec; ++i) {
            const int v = v0 + i * 64 + lane;
            if (ok[u] && v < nvec) r[u][i] = __builtin_nontemporal_load(src + v);
          }
        }
#pragma unroll
        for (int u = 0; u < kCombSlots; ++u) {
          const float wj = __shfl(wl, min(jj + u, 63), 64);
          if (!ok[u]) continue;
#pragma unroll
          for (int i = 0; i < kCombVec; ++i) {
            const int v = v0 + i * 64 + lane;
            if (v < nvec) {
              float f[N];
              Vec16<T>::unpack(r[u][i], f);
#pragma unroll
              for (int q = 0; q < N; ++q) acc[i][q] = fmaf(wj, f[q], acc[i][q]);
            }
          }
        }
      }
    }
    if (shared) {
#pragma unroll
      for (int i = 0; i < kCombVec; ++i) {
        const int v = v0 + i * 64 + lane;
        if (v < nvec) {
          float f[N];
          Vec16<T>::unpack(sh[i], f);
#pragma unroll
          for (int q = 0; q < N; ++q) acc[i][q] += f[q];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kCombVec; ++i) {
      const int v = v0 + i * 64 + lane;
      if (v < nvec) out[(size_t)t * nvec + v] = Vec16<T>::pack(acc[i]);
    }
  }
}

static unsigned item_grid(int64_t items) {
  int64_t blocks = ceil_div(items, kTokWaves);
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

moe_status launch_permute(const moe_shape& s, const void* x, const int32_t* pos, void* x_perm,
                          hipStream_t st) {
  const int eb = s.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int nvec = (int)((int64_t)s.d * eb / 16);
  const int64_t items = (int64_t)s.T * ceil_div(nvec, 64 * kPermVec);
  hipLaunchKernelGGL(k_permute, dim3(item_grid(items)), dim3(64 * kTokWaves), 0, st,
                     static_cast<const u32x4_t*>(x), pos, s.T, s.k, nvec, (int64_t)moe_max_rows(&s),
                     static_cast<u32x4_t*>(x_perm));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status launch_combine(const moe_shape& s, const void* y, const int32_t* pos, const float* topk_w,
                          const void* shared_out, void* out, hipStream_t st) {
  const int eb = s.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int nvec = (int)((int64_t)s.d * eb / 16);
  const unsigned grid = item_grid((int64_t)s.T * ceil_div(nvec, 64 * kCombVec));
  if (s.dtype == MOE_DTYPE_BF16) {
    hipLaunchKernelGGL(k_combine<bf16_t>, dim3(grid), dim3(64 * kTokWaves), 0, st,
                       static_cast<const u32x4_t*>(y), pos, topk_w,
                       static_cast<const u32x4_t*>(shared_out), s.T, s.k, nvec,
                       (int64_t)moe_max_rows(&s), static_cast<u32x4_t*>(out));
  } else {
    hipLaunchKernelGGL(k_combine<float>, dim3(grid), dim3(64 * kTokWaves), 0, st,
                       static_cast<const u32x4_t*>(y), pos, topk_w,
                       static_cast<const u32x4_t*>(shared_out), s.T, s.k, nvec,
                       (int64_t)moe_max_rows(&s), static_cast<u32x4_t*>(out));
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
