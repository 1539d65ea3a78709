// Router: logits -> softmax -> top-k, residency split, stall-free
// substitution, and the APEX prefetch mask.
//
// One 256-thread block per token.  The four waves each sum a quarter of the
// hidden dimension with lane = expert (E <= 64), the partial logits meet in
// LDS, and wave 0 does everything else with wave-wide shuffles:
//   softmax            max / sum of exp over the 64 lanes;
//   top-k              k rounds of a 64-bit arg-max whose key is
//                      (order-preserving logit bits, 0xFFFFFFFF - id), so
//                      equal logits go to the lower id;
//   near-tie flag      one extra round reads the first rejected logit.
// Stall-free substitution [APEX page, Sec. 4.3, Algorithm 1]: every routed
// expert outranks every non-routed one, so "keep the prefetched routed experts
// and fill each miss with the best remaining prefetched expert" is the top-k
// of the router restricted to the prefetched set; the kernel takes that
// masked top-k.
#include "common.h"

namespace moe {

__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  return ((uint64_t)float_order_key(l) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// Logits of token t for lanes 0..E-1, returned to every lane of wave 0 (-inf
// beyond E).  Call from all 256 threads.
template <typename Tin>
__device__ __forceinline__ float block_logits(const Tin* __restrict__ xr, const Tin* __restrict__ w,
                                              int H, int E, float (*part)[MOE_WAVE]) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  float acc = 0.f;
  if (lane < E) {
    const int hq = H >> 2;
    const int h0 = wv * hq;
    for (int h = h0; h < h0 + hq; ++h)
      acc = fmaf(elem<Tin>::load(xr, h), elem<Tin>::load(w, (int64_t)h * E + lane), acc);
  }
  part[wv][lane] = acc;
  __syncthreads();
  float l = -INFINITY;
  if (lane < E) l = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  return l;
}

template <typename Tin>
__global__ void __launch_bounds__(256)
route_kernel(const Tin* __restrict__ x, const Tin* __restrict__ w_router, int H, int E, int k,
             int renorm, float margin, int mode, const uint64_t* __restrict__ resident,
             int64_t res_stride, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
             uint8_t* __restrict__ exact, uint32_t* __restrict__ flags,
             float* __restrict__ logits_out, float* __restrict__ mass_out) {
  __shared__ float part[4][MOE_WAVE];
  const int t = blockIdx.x;
  const float l = block_logits<Tin>(x + (int64_t)t * H, w_router, H, E, part);
  if (threadIdx.x >= MOE_WAVE) return;
  const int lane = threadIdx.x;
  if (logits_out && lane < E) logits_out[(int64_t)t * E + lane] = l;

  // softmax numerator / denominator
  const float mx = wave_max(l);
  const float ex = lane < E ? __expf(l - mx) : 0.f;
  const float denom = wave_sum(ex);

  // routed top-k over all experts
  uint64_t key = lane < E ? topk_key(l, lane) : 0ull;
  uint64_t routed = 0ull;
  float l_last = 0.f;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(key);
    const int e = key_id(m);
    routed |= 1ull << e;
    if (r == k - 1) l_last = __shfl(l, e, MOE_WAVE);
    if (lane == e) key = 0ull;
  }
  uint32_t flag = 0;
  if (k < E) {
    const int e = key_id(wave_max_u64(key));
    if (l_last - __shfl(l, e, MOE_WAVE) < margin) flag |= 1u;
  }
  const bool in_routed = lane < E && ((routed >> lane) & 1ull);
  const float mass = wave_sum(in_routed ? ex : 0.f) / denom;

  uint64_t res_mask = ~0ull;
  if (mode == MOE_MODE_LORE || mode == MOE_MODE_STALL_FREE) res_mask = resident[res_stride * t];

  // final set: routed, or the top-k inside the prefetched set (stall-free)
  uint64_t final_set = routed;
  if (mode == MOE_MODE_STALL_FREE && (routed & ~res_mask) != 0ull) {
    uint64_t allowed = res_mask;
    // fewer than k prefetched experts: the remaining slots take the best
    // experts outside the set (callers pass sets of at least k experts)
    if (__popcll(allowed & ((E == 64) ? ~0ull : ((1ull << E) - 1ull))) < k) allowed = ~0ull;
    key = (lane < E && ((allowed >> lane) & 1ull)) ? topk_key(l, lane) : 0ull;
    final_set = 0ull;
    for (int r = 0; r < k; ++r) {
      const uint64_t m = wave_max_u64(key);
      const int e = key_id(m);
      final_set |= 1ull << e;
      if (r == k - 1) l_last = __shfl(l, e, MOE_WAVE);
      if (lane == e) key = 0ull;
    }
    const uint64_t m = wave_max_u64(key);
    if (m != 0ull && l_last - __shfl(l, key_id(m), MOE_WAVE) < margin) flag |= 4u;
  }

  // slots in (-logit, id) order, weights p_e (renormalised over the set)
  const bool in_final = lane < E && ((final_set >> lane) & 1ull);
  const float fsum = wave_sum(in_final ? ex : 0.f);
  key = in_final ? topk_key(l, lane) : 0ull;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(key);
    const int e = key_id(m);
    if (lane == e) {
      key = 0ull;
      const int64_t o = (int64_t)t * k + r;
      topk_ids[o] = e;
      topk_w[o] = renorm ? ex / fsum : ex / denom;
      exact[o] = (mode == MOE_MODE_LORE) ? (uint8_t)((res_mask >> e) & 1ull) : (uint8_t)1;
    }
  }
  if (lane == 0) {
    flags[t] = flag;
    if (mass_out) mass_out[t] = mass;
  }
}

// APEX prefetch set: top-(k + delta_t) of x W_p as a bit mask.
template <typename Tin>
__global__ void __launch_bounds__(256)
prefetch_kernel(const Tin* __restrict__ x, const Tin* __restrict__ w_p, int H, int E, int k,
                float margin, const int32_t* __restrict__ delta, uint64_t* __restrict__ mask_out,
                uint32_t* __restrict__ flags) {
  __shared__ float part[4][MOE_WAVE];
  const int t = blockIdx.x;
  const float l = block_logits<Tin>(x + (int64_t)t * H, w_p, H, E, part);
  if (threadIdx.x >= MOE_WAVE) return;
  const int lane = threadIdx.x;
  int n = k + delta[t];
  n = n < 1 ? 1 : (n > E ? E : n);
  uint64_t key = lane < E ? topk_key(l, lane) : 0ull;
  uint64_t mask = 0ull;
  float l_last = 0.f;
  for (int r = 0; r < n; ++r) {
    const uint64_t m = wave_max_u64(key);
    const int e = key_id(m);
    mask |= 1ull << e;
    if (r == n - 1) l_last = __shfl(l, e, MOE_WAVE);
    if (lane == e) key = 0ull;
  }
  uint32_t flag = 0;
  if (n < E) {
    const int e = key_id(wave_max_u64(key));
    if (l_last - __shfl(l, e, MOE_WAVE) < margin) flag = 2u;
  }
  if (lane == 0) {
    mask_out[t] = mask;
    flags[t] = flag;
  }
}

hipError_t launch_route(const moe_dims_t& d, int T, const void* x, const void* w_router,
                        const uint64_t* resident, int64_t res_stride, int mode, int32_t* ids,
                        float* w, uint8_t* exact, uint32_t* flags, float* logits, float* mass,
                        hipStream_t s) {
  if (d.dtype == MOE_BF16)
    route_kernel<bf16><<<T, 256, 0, s>>>((const bf16*)x, (const bf16*)w_router, d.hidden,
                                         d.n_experts, d.top_k, d.renormalize, d.tie_margin, mode,
                                         resident, res_stride, ids, w, exact, flags, logits, mass);
  else
    route_kernel<float><<<T, 256, 0, s>>>((const float*)x, (const float*)w_router, d.hidden,
                                          d.n_experts, d.top_k, d.renormalize, d.tie_margin, mode,
                                          resident, res_stride, ids, w, exact, flags, logits, mass);
  return hipGetLastError();
}

hipError_t launch_prefetch(const moe_dims_t& d, int T, const void* x, const void* w_p,
                           const int32_t* delta, uint64_t* mask_out, uint32_t* flags,
                           hipStream_t s) {
  if (d.dtype == MOE_BF16)
    prefetch_kernel<bf16><<<T, 256, 0, s>>>((const bf16*)x, (const bf16*)w_p, d.hidden,
                                            d.n_experts, d.top_k, d.tie_margin, delta, mask_out,
                                            flags);
  else
    prefetch_kernel<float><<<T, 256, 0, s>>>((const float*)x, (const float*)w_p, d.hidden,
                                             d.n_experts, d.top_k, d.tie_margin, delta, mask_out,
                                             flags);
  return hipGetLastError();
}

}  // namespace moe
