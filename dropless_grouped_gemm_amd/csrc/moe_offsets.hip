// Per-expert counts -> offsets -> padded offsets -> block metadata -> permutation,
// entirely on the device, with no host synchronisation and no atomics.
//
// The host never learns how many rows an expert received: the padded layout, the
// block table [expert, m_start, valid_m] and the block count all stay in device
// memory and the grouped GEMM reads them (TileLang chapter "MoE, MLA and
// sparse-attention operators", sections 2.2 item 2 and 2.3 item 2; dropless notes
// sections 3, 5 and 7).  Segments are padded to ceil(c / block_m) * block_m rows, or,
// in the unpadded layout (dropless notes section 11), keep their c rows: the row space
// is cut into block_m-row tiles and a tile holding rows of several experts gets one
// table entry per expert.
//
// Three kernels:
//   k_count     one block per chunk of assignments: per-wave counters in LDS give
//               every assignment its stable rank inside the chunk (wave ballots find
//               the lanes holding the same expert), plus the chunk's histogram.
//   k_scan_meta one block: per-expert exclusive scan over chunks, counts, offsets,
//               padded offsets, block table, block count, error flag.
//   k_scatter   pos[a] = padded offset + chunk base + rank; row_src is its inverse
//               with -1 on every pad row.
// Because each expert's rows are handed out in ascending assignment order, the
// result equals a stable sort of the assignments by expert id.
#include "moe_internal.h"

#include <mutex>

namespace moe {

static constexpr int kCountThreads = 256;      // 4 waves
static constexpr int kChunkRound = 1024;       // assignments per round of a chunk
static constexpr int kScanThreads = 1024;

int offsets_chunk(const moe_shape& s) {
  int64_t M = (int64_t)s.T * s.k;
  int64_t rounds = ceil_div(M, (int64_t)kChunkRound * 1024);  // keep nchunks <= 1024
  if (rounds < 1) rounds = 1;
  return (int)(rounds * kChunkRound);
}

int64_t offsets_nchunks(const moe_shape& s) {
  int64_t M = (int64_t)s.T * s.k;
  return ceil_div(M, offsets_chunk(s));
}

// hist [nchunks][E+1] + local rank [M]
size_t offsets_scratch_bytes(const moe_shape& s) {
  int64_t M = (int64_t)s.T * s.k;
  return align_up((size_t)offsets_nchunks(s) * (s.E + 1) * 4, 256) + align_up((size_t)M * 4, 256);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ void __launch_bounds__(kCountThreads)
k_count(const int32_t* __restrict__ idx, int64_t M, int E, int nbits, int chunk,
        int32_t* __restrict__ hist, int32_t* __restrict__ lrank) {
  extern __shared__ int32_t cnt[];  // [4][E]
  __shared__ int32_t bad_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += kCountThreads) cnt[i] = 0;
  __syncthreads();

  const int64_t cbase = (int64_t)blockIdx.x * chunk;
  int bad = 0;
  // Wave w owns the quarter [w*chunk/4, (w+1)*chunk/4) of the chunk, walked in
  // ascending order, 64 assignments at a time.
  const int quarter = chunk / 4;
  for (int off = 0; off < quarter; off += 64) {
    const int64_t a = cbase + (int64_t)wave * quarter + off + lane;
    const bool in = a < M;
    const int e = in ? idx[a] : 0;
    const bool okv = in && e >= 0 && e < E;
    bad += __popcll(__ballot(in && !okv));
    uint64_t peers = __ballot(okv);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(okv && bit);
      peers &= bit ? bal : ~bal;
    }
    int r = -1;
    if (okv) {
      const int base = cnt[wave * E + e];
      r = base + __popcll(peers & lanemask_lt(lane));
      // the highest peer publishes the new running count (after every peer read it)
      if (lane == 63 - __clzll(peers)) cnt[wave * E + e] = base + __popcll(peers);
    }
    if (in) lrank[a] = r;
  }
  if (lane == 0) bad_s[wave] = bad;
  __syncthreads();
  // per expert: exclusive scan over the 4 waves (wave bases), chunk total to hist
  for (int e = tid; e < E; e += kCountThreads) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    hist[(int64_t)blockIdx.x * (E + 1) + e] = run;
  }
  if (tid == 0) hist[(int64_t)blockIdx.x * (E + 1) + E] = bad_s[0] + bad_s[1] + bad_s[2] + bad_s[3];
  __syncthreads();
  // add the wave base: rank inside the chunk
  for (int off = 0; off < quarter; off += 64) {
    const int64_t a = cbase + (int64_t)wave * quarter + off + lane;
    if (a < M) {
      const int e = idx[a];
      if (e >= 0 && e < E) lrank[a] += cnt[wave * E + e];
    }
  }
}

// Inclusive scan of one int per thread across a block of kScanThreads threads.
__device__ int block_inclusive_scan(int v, int* sh_wave /*[16]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) sh_wave[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += sh_wave[w];
  __syncthreads();
  return v + add;
}

__global__ void __launch_bounds__(kScanThreads)
k_scan_meta(int32_t* __restrict__ hist, int64_t nchunks, int E, int block_m, int unpadded,
            int max_blocks, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
            int32_t* __restrict__ padded, int32_t* __restrict__ meta,
            int32_t* __restrict__ num_blocks, int32_t* __restrict__ err_flag) {
  __shared__ int sh_wave[16];
  __shared__ int s_cnt[1025], s_pad[1025], s_boff[1025];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  // Per column (expert, or E = out-of-range ids): exclusive scan over chunks (chunk
  // bases, in place) -> total.  Loads go out 16 at a time so the walk down the
  // chunks is not a chain of load latencies.
  int c = 0;
  for (int col = tid; col <= E; col += kScanThreads) {
    int run = 0;
    for (int64_t ch0 = 0; ch0 < nchunks; ch0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = ch0 + u < nchunks ? hist[(ch0 + u) * (E + 1) + col] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (ch0 + u < nchunks) {
          if (col < E) hist[(ch0 + u) * (E + 1) + col] = run;
          run += v[u];
        }
      }
    }
    if (col < E) {
      c = run;
      counts[col] = c;
    } else {
      s_bad = run;
    }
  }
  const int inc_c = block_inclusive_scan(c, sh_wave);
  // entries of expert e: padded, ceil(c / block_m) blocks; unpadded, the tiles its rows
  // [o, o + c) touch, floor((o + c - 1) / block_m) - floor(o / block_m) + 1
  const int o = inc_c - c;
  const int nb = unpadded ? (c > 0 ? (o + c - 1) / block_m - o / block_m + 1 : 0)
                          : (c + block_m - 1) / block_m;
  const int seg = unpadded ? c : nb * block_m;   // rows of the expert's segment
  const int inc_p = block_inclusive_scan(seg, sh_wave);
  const int inc_b = block_inclusive_scan(nb, sh_wave);
  if (tid < E) {
    s_cnt[tid] = c;
    s_pad[tid] = inc_p - seg;
    s_boff[tid] = inc_b - nb;
    offsets[tid] = inc_c - c;
    padded[tid] = inc_p - seg;
  }
  if (tid == E - 1) {
    s_pad[E] = inc_p;
    s_boff[E] = inc_b;
    offsets[E] = inc_c;
    padded[E] = inc_p;
    num_blocks[0] = inc_b;
  }
  __syncthreads();
  if (tid == 0) err_flag[0] = s_bad > 0 ? 1 : 0;
  // at most moe_max_blocks entries by construction (the bound the buffers are sized at)
  if (tid == 0 && s_boff[E] > max_blocks) MOE_DEBUG_REPORT(MOE_DBG_BLOCK_COUNT);
  const int total_blocks = min(s_boff[E], max_blocks);
  for (int b = tid; b < total_blocks; b += kScanThreads) {
    // the last expert whose first block index is <= b (empty experts never match last)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_boff[mid] <= b) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int i = b - s_boff[e];
    meta[3 * b + 0] = e;
    if (unpadded) {
      // the expert's rows inside tile floor(o / block_m) + i
      const int o = s_pad[e], t0 = (o / block_m + i) * block_m;
      const int m0 = max(t0, o), m1 = min(t0 + block_m, o + s_cnt[e]);
      meta[3 * b + 1] = m0;
      meta[3 * b + 2] = m1 - m0;
    } else {
      meta[3 * b + 1] = s_pad[e] + i * block_m;
      meta[3 * b + 2] = min(block_m, s_cnt[e] - i * block_m);
    }
  }
}

__global__ void k_scatter(const int32_t* __restrict__ idx, int64_t M, int E, int chunk,
                          const int32_t* __restrict__ hist, const int32_t* __restrict__ lrank,
                          const int32_t* __restrict__ padded, const int32_t* __restrict__ meta,
                          const int32_t* __restrict__ num_blocks, int block_m, int unpadded,
                          int64_t max_rows, int32_t* __restrict__ pos,
                          int32_t* __restrict__ row_src) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t a = i0; a < M; a += stride) {
    const int e = idx[a];
    if (e >= 0 && e < E) {
      const int64_t ch = a / chunk;
      const int p = padded[e] + hist[ch * (E + 1) + e] + lrank[a];
      // in range by construction (the scan's segment bases and the chunk ranks)
      if (p < 0 || p >= max_rows) {
        MOE_DEBUG_REPORT(MOE_DBG_POSITION);
        pos[a] = -1;
        continue;
      }
      pos[a] = p;
      row_src[p] = (int32_t)a;
    } else {
      pos[a] = -1;
    }
  }
  if (unpadded) {
    // rows past the routed total (only when some ids were out of range) hold nothing
    const int total = padded[E];
    for (int64_t r = i0 + total; r < max_rows; r += stride) row_src[r] = -1;
    return;
  }
  const int nb = num_blocks[0];
  for (int64_t r = i0; r < max_rows; r += stride) {
    const int64_t b = r / block_m;
    if (b >= nb || (int)(r - b * block_m) >= meta[3 * b + 2]) row_src[r] = -1;
  }
}

moe_status launch_build_offsets(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                                int32_t* offsets, int32_t* padded, int32_t* block_meta,
                                int32_t* num_blocks, int32_t* pos, int32_t* row_src,
                                int32_t* err_flag, void* scratch, hipStream_t st) {
  const int64_t M = (int64_t)s.T * s.k;
  const int chunk = offsets_chunk(s);
  const int64_t nchunks = offsets_nchunks(s);
  int32_t* hist = static_cast<int32_t*>(scratch);
  int32_t* lrank = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) +
                                              align_up((size_t)nchunks * (s.E + 1) * 4, 256));
  int nbits = 1;
  while ((1 << nbits) < s.E) ++nbits;
  if (nchunks > 0) {
    hipLaunchKernelGGL(k_count, dim3((unsigned)nchunks), dim3(kCountThreads),
                       (size_t)4 * s.E * sizeof(int32_t), st, topk_idx, M, s.E, nbits, chunk, hist,
                       lrank);
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  }
  hipLaunchKernelGGL(k_scan_meta, dim3(1), dim3(kScanThreads), 0, st, hist, nchunks, s.E, s.block_m,
                     s.unpadded, (int)moe_max_blocks(&s), counts, offsets, padded, block_meta, num_blocks, err_flag);
  if (hipGetLastError() != hipSuccess) return MOE_EHIP;
  const int64_t max_rows = (int64_t)moe_max_rows(&s);
  const int64_t work = M > max_rows ? M : max_rows;
  int64_t blocks = ceil_div(work, 256);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)blocks), dim3(256), 0, st, topk_idx, M, s.E, chunk,
                     hist, lrank, padded, block_meta, num_blocks, s.block_m, s.unpadded, max_rows,
                     pos, row_src);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate (moe_build_offsets_noalloc): the per-chunk
// histograms and local ranks live in one file-scope device array instead of the caller's
// workspace.  Each device holds its own copy of the array, at its own address, from the
// library's first use on that device until the process ends.  In host code the array's
// name is not a device address, so the address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is passed on.
// Nothing in it must start at zero: k_count writes every histogram entry and every local
// rank that k_scan_meta and k_scatter later read.  Calls on one device share the array,
// so calls that overlap in time on one device race.
// ---------------------------------------------------------------------------
static constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char offsets_static_scratch[kStaticScratchBytes];

static constexpr int kStaticMaxDevices = 64;
static std::mutex g_static_mu;
static void* g_static_ptr[kStaticMaxDevices];

size_t static_scratch_capacity() { return kStaticScratchBytes; }

moe_status static_scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(offsets_static_scratch)) != hipSuccess || !p)
      return MOE_EHIP;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return MOE_OK;
}

}  // namespace moe
