// Stable counting sort of (token, slot) pairs into 2E buckets, one 1024-pair
// chunk per 1024-thread workgroup: the body shared by the permutation kernel
// and the router's top-k kernel, whose last workgroup permutes a batch of at
// most 1024 pairs in the same launch.  Exactly computed pairs are bucketed
// by expert, pairs left to the LoRE surrogate by E + expert.
#pragma once

#include "common.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr int PERM_WAVES = PERM_THREADS / MOE_WAVE;
constexpr int PERM_BUCKETS = 2 * MOE_MAX_EXPERTS;

// Bucket of pair f: expert for exact pairs, E + expert for the others, -1
// for out-of-range ids (never placed).  exact == nullptr: every pair exact.
__device__ __forceinline__ int bucket_of(int f, int E, const int32_t* __restrict__ ids,
                                         const uint8_t* __restrict__ exact) {
  const int e = ids[f];
  if ((unsigned)e >= (unsigned)E) return -1;
  return (!exact || exact[f]) ? e : E + e;
}

// Places chunk `chunk` of `nchunks`; every thread of a 1024-thread block
// calls it.  counts == nullptr: the block histograms every pair itself.
// A pair's rank among equal buckets in the chunk is the popcount of
// its wave's peer mask (eight ballots over the bits of bucket+1) below its
// lane, plus that bucket's counts in earlier waves, so the order is stable
// and deterministic with no order-dependent atomics.
__device__ __forceinline__ void permute_chunk(int chunk, int nchunks, int n_pairs, int E,
                                              const int32_t* __restrict__ ids,
                                              const uint8_t* __restrict__ exact,
                                              const int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* __restrict__ row_of,
                                              int32_t* __restrict__ miss_offsets) {
  __shared__ int tot[PERM_BUCKETS];     // pairs per bucket over all chunks
  __shared__ int before[PERM_BUCKETS];  // pairs per bucket in earlier chunks
  __shared__ int cursor[PERM_BUCKETS];
  __shared__ int wcnt[PERM_WAVES][PERM_BUCKETS];
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wv = tid >> 6;
  const int NB = 2 * E;
  const int f = chunk * PERM_THREADS + tid;
  const int b = f < n_pairs ? bucket_of(f, E, ids, exact) : -1;
  if (counts) {
    // bucket sums over the chunks' histograms: thread (g, bucket) adds
    // chunks g, g + 8, ... with its loads in flight together, then the
    // eight partial sums of a bucket are added (integers: any order is exact)
    constexpr int NG = PERM_THREADS / PERM_BUCKETS;
    __shared__ int ptot[NG][PERM_BUCKETS], pbef[NG][PERM_BUCKETS];
    const int bk = tid % PERM_BUCKETS, g = tid / PERM_BUCKETS;
    int t = 0, bf = 0;
    if (bk < NB) {
#pragma unroll 4
      for (int c = g; c < nchunks; c += NG) {
        const int v = counts[(int64_t)c * NB + bk];
        t += v;
        bf += c < chunk ? v : 0;
      }
    }
    ptot[g][bk] = t;
    pbef[g][bk] = bf;
    __syncthreads();
    if (tid < NB) {
      int st = 0, sb = 0;
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        st += ptot[q][tid];
        sb += pbef[q][tid];
      }
      tot[tid] = st;
      before[tid] = sb;
    }
  } else {
    // no per-chunk histograms: the block counts every pair itself (one
    // chunk, or a few), all of them for the bucket totals and those of the
    // chunks before its own for its starts
    if (tid < PERM_BUCKETS) {
      tot[tid] = 0;
      before[tid] = 0;
    }
    __syncthreads();
    const int lo = chunk * PERM_THREADS;
    for (int g = tid; g < n_pairs; g += PERM_THREADS) {
      const int bg = g == f ? b : bucket_of(g, E, ids, exact);
      if (bg >= 0) {
        atomicAdd(&tot[bg], 1);
        if (g < lo) atomicAdd(&before[bg], 1);
      }
    }
  }
  __syncthreads();
  if (tid < MOE_WAVE) {
    // two buckets per lane: 2*lane, 2*lane+1 (NB <= 128)
    const int c0 = 2 * lane < NB ? tot[2 * lane] : 0;
    const int c1 = 2 * lane + 1 < NB ? tot[2 * lane + 1] : 0;
    const int c = c0 + c1;
    const int s = wave_incl_scan_i(c);
    cursor[2 * lane] = s - c + (2 * lane < NB ? before[2 * lane] : 0);
    cursor[2 * lane + 1] = s - c + c0 + (2 * lane + 1 < NB ? before[2 * lane + 1] : 0);
    if (lane == MOE_WAVE - 1) s_total = s;
    if (chunk == 0) {
      // bucket bases (chunk 0 has nothing before it)
      if (2 * lane <= E) offsets[2 * lane] = s - c;
      if (2 * lane + 1 <= E) offsets[2 * lane + 1] = s - c + c0;
    }
  }
  __syncthreads();
  if (chunk == 0 && miss_offsets && tid <= E) miss_offsets[tid] = tid < E ? cursor[E + tid] : s_total;
  const uint64_t below = (1ull << lane) - 1ull;
  const int v = b + 1;  // 0..128
  uint64_t peers = __ballot(1);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = (v >> bit) & 1;
    const uint64_t bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  const int rank = __popcll(peers & below);
  wcnt[wv][lane] = 0;
  wcnt[wv][lane + MOE_WAVE] = 0;
  __builtin_amdgcn_wave_barrier();
  if (b >= 0 && rank == 0) wcnt[wv][b] = __popcll(peers);
  __syncthreads();
  if (b >= 0) {
    int pos = cursor[b] + rank;
    for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][b];
    perm[pos] = f;
    inv[f] = b < E ? pos : -1;
    if (row_of) row_of[f] = pos;
  } else if (f < n_pairs) {
    inv[f] = -1;
    if (row_of) row_of[f] = -1;
  }
}

}  // namespace moe
