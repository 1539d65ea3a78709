// Token -> expert permutation: a stable counting sort of the exactly computed
// (token, slot) pairs f = t*k + j by expert.
//
// One 1024-thread workgroup: LDS histogram (order-free atomics on counts),
// one wave's shuffle scan for the expert offsets, then a stable scatter in
// chunks of 1024 pairs.  Inside a chunk a pair's rank among equal experts is
// the popcount of its wave's peer mask (seven ballots over the bits of
// expert+1) below its lane, plus the counts of the same expert in the waves
// before it -- no order-dependent atomics, so perm is deterministic.
#include "common.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr int PERM_WAVES = PERM_THREADS / MOE_WAVE;

__global__ void __launch_bounds__(PERM_THREADS)
permute_kernel(int n_pairs, int E, const int32_t* __restrict__ ids, const uint8_t* __restrict__ exact,
               int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int cnt[MOE_WAVE];
  __shared__ int cursor[MOE_WAVE];
  __shared__ int wcnt[PERM_WAVES][MOE_WAVE];
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wv = tid >> 6;
  if (tid < MOE_WAVE) cnt[tid] = 0;
  __syncthreads();
  for (int f = tid; f < n_pairs; f += PERM_THREADS) {
    const int e = ids[f];
    if (exact[f] && (unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < MOE_WAVE) {
    const int c = lane < E ? cnt[lane] : 0;
    int s = c;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
      const int v = __shfl_up(s, o, MOE_WAVE);
      if (lane >= o) s += v;
    }
    cursor[lane] = s - c;
    if (lane < E) offsets[lane] = s - c;
    if (lane == MOE_WAVE - 1) offsets[E] = s;
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = 0; base < n_pairs; base += PERM_THREADS) {
    const int f = base + tid;
    int e = -1;
    if (f < n_pairs && exact[f]) {
      const int ee = ids[f];
      if ((unsigned)ee < (unsigned)E) e = ee;  // out-of-range ids count as not exact
    }
    const int v = e + 1;  // 0..64
    uint64_t peers = __ballot(1);
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const bool bit = (v >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & below);
    wcnt[wv][lane] = 0;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && rank == 0) wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int pos = cursor[e] + rank;
      for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
      perm[pos] = f;
      inv[f] = pos;
    } else if (f < n_pairs) {
      inv[f] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w2 = 0; w2 < PERM_WAVES; ++w2) s += wcnt[w2][tid];
      cursor[tid] += s;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(int n_pairs, int E, const int32_t* ids, const uint8_t* exact,
                          int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t s) {
  permute_kernel<<<1, PERM_THREADS, 0, s>>>(n_pairs, E, ids, exact, offsets, perm, inv);
  return hipGetLastError();
}

}  // namespace moe
