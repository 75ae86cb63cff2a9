// Local routing permutation: a stable counting sort of (token, slot) entries
// by expert, with each expert's slot padded to the alignment (P2, review
// comments: routing prepared once and cached for dispatch and combine;
// padded expert slots.  P1, commit messages: top_k, alignment and the index
// dtype are arguments of the NVFP4 paths).
//
// Up to kSingleMax entries everything runs in ONE workgroup
// of 16 waves (k_route_single): per-wave histograms in LDS, the cross-wave
// scan and the padded offsets in LDS, then the stable scatter -- one launch.
// Larger inputs use three launches, no atomics on global memory except the
// error flag:
//   1. count   -- each wave counts its 256 consecutive entries per expert
//                 (LDS atomics: order does not matter for counts);
//   2. scan    -- one workgroup turns the per-wave histograms into per-wave
//                 starting ranks, the counts, the padded offsets, and writes
//                 -1 into every padding / unused row of src_row;
//   3. scatter -- each wave walks its entries in order, 64 at a time; lanes
//                 with equal expert ids are found with one ballot per id bit,
//                 so the rank inside a step is a popcount and the order is
//                 stable (token order, then slot order).
#include "common.h"
#include "launch.h"

namespace mtb {

constexpr int kRouteChunk = 256;  // entries per wave
constexpr int kMaxExperts = 1024;

template <typename IDX>
__global__ __launch_bounds__(256) void k_route_count(const IDX* __restrict__ idx, int64_t R, int E, int W,
                                                     int32_t* __restrict__ hist, int32_t* __restrict__ d_error) {
  __shared__ int32_t cnt[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
  const int w = blockIdx.x * 4 + wl;
  for (int e = lane; e < E; e += 64) cnt[wl][e] = 0;
  __syncthreads();
  if (w < W) {
    // the chunk's loads first (indices clamped into [0, R)), then the counts
    IDX v[kRouteChunk / 64];
#pragma unroll
    for (int s = 0; s < kRouteChunk / 64; ++s) v[s] = idx[min((int64_t)w * kRouteChunk + s * 64 + lane, R - 1)];
    bool any_bad = false;
#pragma unroll
    for (int s = 0; s < kRouteChunk / 64; ++s) {
      const bool in = (int64_t)w * kRouteChunk + s * 64 + lane < R;
      const int64_t q = in ? (int64_t)v[s] : -1;
      any_bad |= (q < -1) || (q >= E);
      if (q >= 0 && q < E) atomicAdd(&cnt[wl][(int)q], 1);
    }
    if (any_bad) atomicOr(d_error, EP_DEVERR_EXPERT_ID);
  }
  __syncthreads();
  if (w < W)
    for (int e = lane; e < E; e += 64) hist[(int64_t)w * E + e] = cnt[wl][e];
}

constexpr int kScanBatch = 16;  // histogram loads in flight per thread in the scan

// One workgroup of 1024 threads.  hist [W, E] -> per-wave starting rank
// (exclusive prefix over waves), counts, padded offsets, -1 padding rows.
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ hist, int W, int E, int A, int r_cap,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ src_row) {
  __shared__ int32_t part[1024];
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x;
  const int G = 1024 / E;           // wave groups per expert (E <= 1024)
  const int e = tid % E, g = tid / E;
  const bool active = g < G;
  const int wpg = (W + G - 1) / G;
  const int w0 = active ? g * wpg : 0, w1 = active ? min(W, w0 + wpg) : 0;
  // the thread's run of histogram entries, kScanBatch loads in flight at a
  // time (one dependent round trip per batch, not per entry); the batch stays
  // in registers for the rank pass below when the run fits in one
  int32_t local = 0;
  int32_t keep[kScanBatch];
  for (int wb = w0; wb < w1; wb += kScanBatch) {
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) keep[u] = wb + u < w1 ? hist[(int64_t)(wb + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) local += keep[u];
  }
  if (active) part[g * E + e] = local;
  __syncthreads();
  if (tid < E) {
    int32_t run = 0;
    for (int gg = 0; gg < G; ++gg) {
      int32_t c = part[gg * E + tid];
      part[gg * E + tid] = run;
      run += c;
    }
    counts[tid] = run;
    scan[tid] = (run + A - 1) / A * A;
  }
  __syncthreads();
  if (active) {
    int32_t run = part[g * E + e];
    if (w1 - w0 <= kScanBatch) {  // the run is still in registers
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        if (w0 + u < w1) {
          hist[(int64_t)(w0 + u) * E + e] = run;
          run += keep[u];
        }
    } else {
      for (int wb = w0; wb < w1; wb += kScanBatch) {
        int32_t c[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) c[u] = wb + u < w1 ? hist[(int64_t)(wb + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
          if (wb + u < w1) {
            hist[(int64_t)(wb + u) * E + e] = run;
            run += c[u];
          }
      }
    }
  }
  // inclusive scan of the padded sizes over experts (Hillis-Steele in LDS)
  for (int o = 1; o < E; o <<= 1) {
    int32_t v = 0;
    if (tid < E && tid >= o) v = scan[tid - o];
    __syncthreads();
    if (tid < E) scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = scan[tid];
  if (tid == 0) offsets[0] = 0;
  // padding rows of each expert, then everything from off_E to r_cap: -1
  if (tid < E) {
    int32_t end = scan[tid];
    int32_t c = (tid ? scan[tid - 1] : 0) + counts[tid];
    for (int32_t r = c; r < end; ++r) src_row[r] = -1;
  }
  const int32_t total = scan[E - 1];
  for (int32_t r = total + tid; r < r_cap; r += 1024) src_row[r] = -1;
}

template <typename IDX>
__global__ __launch_bounds__(256) void k_route_scatter(const IDX* __restrict__ idx, int64_t R, int k, int E, int W,
                                                       int ebits, const int32_t* __restrict__ hist,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row) {
  __shared__ int32_t base[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
  const int w = blockIdx.x * 4 + wl;
  if (w < W)
    for (int e = lane; e < E; e += 64) base[wl][e] = hist[(int64_t)w * E + e] + offsets[e];
  __syncthreads();
  if (w >= W) return;
  const uint64_t lt = (1ull << lane) - 1ull;
  IDX v[kRouteChunk / 64];
#pragma unroll
  for (int s = 0; s < kRouteChunk / 64; ++s) v[s] = idx[min((int64_t)w * kRouteChunk + s * 64 + lane, R - 1)];
#pragma unroll
  for (int s = 0; s < kRouteChunk / 64; ++s) {
    int64_t i = (int64_t)w * kRouteChunk + s * 64 + lane;
    const int64_t q = i < R ? (int64_t)v[s] : -1;
    const int x = (q >= 0 && q < E) ? (int)q : -1;
    const bool valid = x >= 0;
    uint64_t m = __ballot(valid);
    // lanes whose expert id agrees with this lane's on every id bit
#pragma unroll 1
    for (int b = 0; b < ebits; ++b) {
      uint64_t bb = __ballot(valid && ((x >> b) & 1));
      m &= ((x >> b) & 1) ? bb : ~bb;
    }
    if (valid) {
      int32_t b0 = base[wl][x];
      int32_t rank = __popcll(m & lt);
      int32_t d = b0 + rank;
      dst_row[i] = d;
      src_row[d] = (int32_t)(i / k);
      if ((m >> lane) == 1ull) base[wl][x] = b0 + __popcll(m);  // the group's last lane advances the base
    } else if (i < R) {
      dst_row[i] = -1;
    }
  }
}

// ------------------------------------------------------------------ single workgroup
constexpr int kSingleWaves = 16;
constexpr int64_t kSingleMax = 16384;  // beyond this one CU's scattered stores dominate
constexpr int kSingleSteps = (int)(kSingleMax / kSingleWaves / 64);  // 64-entry steps per wave, at most

// Each wave owns `chunk` consecutive entries and loads all of them into
// registers up front (one memory round trip instead of one per 64 entries:
// the kernel is latency-bound), counts them, and after the scan places them.
// (Building src_row in LDS and writing it out coalesced at the end was measured
// no faster than the scattered 4-byte stores.)
template <typename IDX>
__global__ __launch_bounds__(1024) void k_route_single(const IDX* __restrict__ idx, int R, int k, int E, int A,
                                                       int r_cap, int ebits, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ dst_row,
                                                       int32_t* __restrict__ src_row, int32_t* __restrict__ d_error) {
  __shared__ int32_t hist[kSingleWaves][kMaxExperts];  // per-wave counts, then per-wave starting rows
  __shared__ int32_t scan[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunk = ((R + kSingleWaves - 1) / kSingleWaves + 63) / 64 * 64;  // <= kSingleSteps * 64
  const int c0 = w * chunk, c1 = min(R, c0 + chunk);
  // all loads first, unconditional (indices clamped into [0, R)), so that they
  // are in flight together; entries outside the wave's range are dropped after
  IDX v[kSingleSteps];
  if (R > 0) {
#pragma unroll
    for (int st = 0; st < kSingleSteps; ++st) v[st] = idx[min(c0 + st * 64 + lane, R - 1)];
  }
  int xs[kSingleSteps];
  bool any_bad = false;
#pragma unroll
  for (int st = 0; st < kSingleSteps; ++st) {
    const int i = c0 + st * 64 + lane;
    const bool in = R > 0 && st * 64 < chunk && i < c1;
    const int64_t q = in ? (int64_t)v[st] : -1;
    any_bad |= (q < -1) || (q >= E);
    xs[st] = (q >= 0 && q < E) ? (int)q : -1;
  }
  for (int e = lane; e < E; e += 64) hist[w][e] = 0;
  __syncthreads();
  // Counting and ranking in one pass: per 64-entry step, the lanes holding
  // the same expert id (one ballot per id bit) elect their lowest lane, which
  // adds the group's size to the wave's count of that expert and receives the
  // count before it; every lane of the group takes that value plus its rank
  // among the group's lanes.  One LDS atomic per distinct id and step, not
  // one per entry, and the scatter below needs no further ranking.  A wave's
  // LDS operations complete in order, so ranks follow the entries' order.
  const uint64_t lt = (1ull << lane) - 1ull;
  int loc[kSingleSteps];
#pragma unroll
  for (int st = 0; st < kSingleSteps; ++st) {
    loc[st] = 0;
    if (st * 64 >= chunk) continue;  // wave-uniform
    const int x = xs[st];
    const bool valid = x >= 0;
    uint64_t m = __ballot(valid);
#pragma unroll 1
    for (int b = 0; b < ebits; ++b) {
      const uint64_t bb = __ballot(valid && ((x >> b) & 1));
      m &= ((x >> b) & 1) ? bb : ~bb;
    }
    const int leader = valid ? __ffsll((unsigned long long)m) - 1 : lane;
    int base = 0;
    if (valid && leader == lane) base = atomicAdd(&hist[w][x], __popcll(m));
    base = __shfl(base, leader, kWave);
    loc[st] = base + __popcll(m & lt);
  }
  if (any_bad) atomicOr(d_error, EP_DEVERR_EXPERT_ID);
  __syncthreads();
  int32_t cnt = 0;
  if (tid < E) {
    for (int ww = 0; ww < kSingleWaves; ++ww) {
      int32_t c = hist[ww][tid];
      hist[ww][tid] = cnt;
      cnt += c;
    }
    counts[tid] = cnt;
    scan[tid] = (cnt + A - 1) / A * A;
  }
  __syncthreads();
  for (int o = 1; o < E; o <<= 1) {
    int32_t v = (tid < E && tid >= o) ? scan[tid - o] : 0;
    __syncthreads();
    if (tid < E) scan[tid] += v;
    __syncthreads();
  }
  // exclusive offset of each expert -> add it to every wave's starting rank
  if (tid < E) {
    const int32_t start = tid ? scan[tid - 1] : 0;
    offsets[tid + 1] = scan[tid];
    for (int ww = 0; ww < kSingleWaves; ++ww) hist[ww][tid] += start;
    for (int32_t r = start + cnt; r < scan[tid]; ++r) src_row[r] = -1;  // padding rows
  }
  if (tid == 0) offsets[0] = 0;
  const int32_t total = scan[E - 1];
  for (int32_t r = total + tid; r < r_cap; r += 1024) src_row[r] = -1;
  __syncthreads();
  // hist[w][e] is now the wave's first row of expert e: place the entries
#pragma unroll
  for (int st = 0; st < kSingleSteps; ++st) {
    if (st * 64 >= chunk) break;  // wave-uniform
    const int i = c0 + st * 64 + lane;
    const int x = xs[st];
    if (x >= 0) {
      const int32_t d = hist[w][x] + loc[st];
      dst_row[i] = d;
      src_row[d] = i / k;
    } else if (i < c1) {
      dst_row[i] = -1;
    }
  }
}

}  // namespace mtb

using namespace mtb;

static int64_t route_waves(int64_t tokens, int64_t top_k) { return (tokens * top_k + kRouteChunk - 1) / kRouteChunk; }

MTB_EXPORT int64_t ep_route_capacity(int64_t tokens, int64_t top_k, int64_t num_experts, int64_t alignment) {
  if (tokens < 0 || top_k < 1 || num_experts < 1) return EP_ERR_SHAPE;
  if (alignment < 16 || alignment % 16 != 0) return EP_ERR_ALIGN;
  if (tokens >= kSizeLimit || top_k >= kSizeLimit || num_experts >= kSizeLimit || alignment >= kSizeLimit)
    return EP_ERR_RANGE;
  return tokens * top_k + num_experts * (alignment - 1);
}

MTB_EXPORT size_t ep_route_workspace_bytes(int64_t tokens, int64_t top_k, int64_t num_experts) {
  if (tokens < 0 || top_k < 1 || num_experts < 1) return 0;
  if (tokens >= kSizeLimit || top_k >= kSizeLimit || num_experts >= kSizeLimit) return 0;
  int64_t w = route_waves(tokens, top_k);
  int64_t bytes = 0;
  if (__builtin_mul_overflow((w > 0 ? w : 1) * (int64_t)sizeof(int32_t), num_experts, &bytes)) return 0;
  return (size_t)bytes;
}

MTB_EXPORT int32_t ep_route_plan(const void* topk_idx, int32_t idx_dtype, int64_t tokens, int64_t top_k,
                                 int64_t num_experts, int64_t alignment, int64_t r_cap, int32_t* counts,
                                 int32_t* offsets, int32_t* dst_row, int32_t* src_row, void* workspace,
                                 size_t workspace_bytes, int32_t* d_error, void* stream) {
  if (tokens < 0 || top_k < 1 || num_experts < 1 || r_cap < 0) return EP_ERR_SHAPE;
  if (num_experts > kMaxExperts) return EP_ERR_SHAPE;
  if (alignment < 16 || alignment % 16 != 0) return EP_ERR_ALIGN;
  if (idx_dtype != EP_IDX_INT32 && idx_dtype != EP_IDX_INT64) return EP_ERR_DTYPE;
  if (tokens >= INT32_MAX || top_k >= INT32_MAX || alignment >= INT32_MAX || r_cap >= INT32_MAX ||
      tokens * top_k + num_experts * alignment >= (int64_t)INT32_MAX)
    return EP_ERR_RANGE;
  if (r_cap < ep_route_capacity(tokens, top_k, num_experts, alignment)) return EP_ERR_CAPACITY;
  if (!counts || !offsets || !src_row || !d_error || (tokens > 0 && (!topk_idx || !dst_row))) return EP_ERR_NULL;
  if (!workspace || workspace_bytes < ep_route_workspace_bytes(tokens, top_k, num_experts)) return EP_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int64_t R = tokens * top_k;
  const int W = (int)route_waves(tokens, top_k);
  const int E = (int)num_experts;
  int32_t* hist = (int32_t*)workspace;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  if (R <= kSingleMax) {
    if (idx_dtype == EP_IDX_INT32)
      hipLaunchKernelGGL(k_route_single<int32_t>, dim3(1), dim3(1024), 0, s, (const int32_t*)topk_idx, (int)R,
                         (int)top_k, E, (int)alignment, (int)r_cap, ebits, counts, offsets, dst_row, src_row, d_error);
    else
      hipLaunchKernelGGL(k_route_single<int64_t>, dim3(1), dim3(1024), 0, s, (const int64_t*)topk_idx, (int)R,
                         (int)top_k, E, (int)alignment, (int)r_cap, ebits, counts, offsets, dst_row, src_row, d_error);
    return launch_status();
  }
  if (W > 0) {
    dim3 grid((unsigned)((W + 3) / 4)), block(256);
    if (idx_dtype == EP_IDX_INT32)
      hipLaunchKernelGGL(k_route_count<int32_t>, grid, block, 0, s, (const int32_t*)topk_idx, R, E, W, hist, d_error);
    else
      hipLaunchKernelGGL(k_route_count<int64_t>, grid, block, 0, s, (const int64_t*)topk_idx, R, E, W, hist, d_error);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, hist, W, E, (int)alignment, (int)r_cap, counts,
                     offsets, src_row);
  if (W > 0) {
    dim3 grid((unsigned)((W + 3) / 4)), block(256);
    if (idx_dtype == EP_IDX_INT32)
      hipLaunchKernelGGL(k_route_scatter<int32_t>, grid, block, 0, s, (const int32_t*)topk_idx, R, (int)top_k, E, W,
                         ebits, hist, offsets, dst_row, src_row);
    else
      hipLaunchKernelGGL(k_route_scatter<int64_t>, grid, block, 0, s, (const int64_t*)topk_idx, R, (int)top_k, E, W,
                         ebits, hist, offsets, dst_row, src_row);
  }
  return launch_status();
}
