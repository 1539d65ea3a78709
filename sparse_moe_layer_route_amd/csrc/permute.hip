// Token -> expert permutation: a stable counting sort of all (token, slot)
// pairs f = t*k + j into 2E buckets -- exactly computed pairs by expert
// first, then pairs left to the LoRE surrogate by expert.
//
// Pairs are taken in chunks of 1024 (one 1024-thread workgroup per chunk).
// A count kernel writes each chunk's bucket histogram (LDS atomics on
// counts, whose order does not matter); the scatter kernel's block c then
// sums the histograms -- all chunks for the bucket bases, chunks before c for
// its own start in each bucket -- and places its chunk.  Inside a chunk a
// pair's rank among equal buckets is the popcount of its wave's peer mask
// (eight ballots over the bits of bucket+1) below its lane, plus the counts
// of the same bucket in the waves before it, so the order is stable and
// deterministic with no order-dependent atomics.  Up to a few chunks each
// scatter block takes the histogram of all pairs itself (one launch).
#include <algorithm>

#include "permute_block.h"

namespace moe {

// Histogram of chunk blockIdx.x into counts[blockIdx.x][2E].
__global__ void __launch_bounds__(PERM_THREADS)
permute_count_kernel(int n_pairs, int E, const int32_t* __restrict__ ids,
                     const uint8_t* __restrict__ exact, int32_t* __restrict__ counts) {
  __shared__ int cnt[PERM_BUCKETS];
  const int tid = threadIdx.x, NB = 2 * E;
  if (tid < PERM_BUCKETS) cnt[tid] = 0;
  __syncthreads();
  const int f = blockIdx.x * PERM_THREADS + tid;
  if (f < n_pairs) {
    const int b = bucket_of(f, E, ids, exact);
    if (b >= 0) atomicAdd(&cnt[b], 1);
  }
  __syncthreads();
  if (tid < NB) counts[(int64_t)blockIdx.x * NB + tid] = cnt[tid];
}

// Block c places chunk c.  counts == nullptr: a single block histograms the
// (at most one) chunk itself.
__global__ void __launch_bounds__(PERM_THREADS)
permute_kernel(int n_pairs, int E, const int32_t* __restrict__ ids, const uint8_t* __restrict__ exact,
               const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
               int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ row_of,
               int32_t* __restrict__ miss_offsets) {
  permute_chunk(blockIdx.x, gridDim.x, n_pairs, E, ids, exact, counts, offsets, perm, inv, row_of,
                miss_offsets);
}

int permute_scratch_bytes(int n_pairs, int E) {
  const int nchunks = (n_pairs + PERM_THREADS - 1) / PERM_THREADS;
  return nchunks > 1 ? nchunks * 2 * E * 4 : 0;
}

// Up to this many chunks every scatter block histograms all pairs itself (a
// few thousand pairs: one launch instead of the count and scatter launches).
#ifndef PERM_SELF_HIST_CHUNKS
#define PERM_SELF_HIST_CHUNKS 4
#endif

hipError_t launch_permute(int n_pairs, int E, const int32_t* ids, const uint8_t* exact,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* row_of,
                          int32_t* miss_offsets, int32_t* scratch, hipStream_t s) {
  const int nchunks = (n_pairs + PERM_THREADS - 1) / PERM_THREADS;
  if (nchunks <= PERM_SELF_HIST_CHUNKS) {
    permute_kernel<<<std::max(nchunks, 1), PERM_THREADS, 0, s>>>(n_pairs, E, ids, exact, nullptr,
                                                                offsets, perm, inv, row_of,
                                                                miss_offsets);
  } else {
    permute_count_kernel<<<nchunks, PERM_THREADS, 0, s>>>(n_pairs, E, ids, exact, scratch);
    permute_kernel<<<nchunks, PERM_THREADS, 0, s>>>(n_pairs, E, ids, exact, scratch, offsets, perm,
                                                    inv, row_of, miss_offsets);
  }
  return hipGetLastError();
}

}  // namespace moe
