// Router: logits -> softmax -> top-k, residency split, stall-free
// substitution, shared-expert gate, and the APEX prefetch mask.
//
// Routing is two launches (batches of at most four tokens rank and permute
// in one small block: route_topk_small_kernel).
//   logits  one 512-thread block per (16-token tile, 16-expert tile): bf16
//           l = X W_r^T on the matrix cores (v_mfma_f32_16x16x32_bf16),
//           A = 16 token rows, B = 16 expert rows of W_r [E][H] (both k
//           contiguous); the 8 waves take contiguous eighths of K and their
//           partial tiles meet in LDS, summed in a fixed order, so logits are
//           bitwise reproducible.  Spreading the expert tiles over blocks
//           keeps each CU's share of W_r small.  fp32: one thread per
//           (token, expert) dot product.
//   top-k   one wave per token, lane = expert: softmax by wave max / sum of
//           exp; each lane's rank is the number of lanes whose key
//           (order-preserving logit bits, 0xFFFFFFFF - id) is larger, read
//           with E scalar lane reads, so equal logits go to the lower id; the
//           expert of rank j fills slot j, and the logits at ranks k-1 and k
//           give the near-tie flag.
// The prefetch mask runs as one 1024-thread block per 16-token tile (logits
// and ranking in one launch).
// Stall-free substitution [APEX page, Sec. 4.3, Algorithm 1]: every routed
// expert outranks every non-routed one, so keeping the prefetched routed
// experts and filling each miss with the best remaining prefetched expert is
// the top-k of the router restricted to the prefetched set; the kernel takes
// that masked top-k.
#include "permute_block.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int ROUTE_TOK = 16;
constexpr int ROUTE_WAVES = 16;

__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  return ((uint64_t)float_order_key(l) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
// Rank of this lane's key among lanes 0..E-1 (0 = largest).  Keys of valid
// lanes are distinct (the id is part of the key), so ranks are a permutation.
__device__ __forceinline__ int key_rank(uint64_t key, int E) {
  const int lo = (int)(uint32_t)key, hi = (int)(uint32_t)(key >> 32);
  int rank = 0;
  for (int j = 0; j < E; ++j) {
    const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, j) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(lo, j);
    rank += kj > key;
  }
  return rank;
}

// Logit of the lane holding rank r (lanes pass their own rank; r < E).
__device__ __forceinline__ float lane_logit_at_rank(float l, int rank, int r, int E) {
  const uint64_t hit = __ballot(lane_id() < E && rank == r);
  const int src = __ffsll((unsigned long long)hit) - 1;
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), src));
}

struct RouteLds {
  float part[ROUTE_WAVES][ROUTE_TOK][MOE_MAX_EXPERTS];
  float logits[ROUTE_TOK][MOE_MAX_EXPERTS];
};

#ifndef ROUTE_TILE_U
#define ROUTE_TILE_U 4
#endif
// Logits of tokens t0..t0+15 (rows past T are clamped, results unused) into
// lds.logits.  Called by all 1024 threads.
__device__ __forceinline__ void tile_logits(const bf16* __restrict__ x, const bf16* __restrict__ w,
                                            int T, int H, int E, int t0, RouteLds& lds) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int n_et = (E + 15) >> 4;
  const int n_sp = ROUTE_WAVES / n_et;
  const int et = wv % n_et, sp = wv / n_et;
  const int r16 = lane & 15, kg = lane >> 4;
  if (sp < n_sp) {
    const int t = min(t0 + r16, T - 1);
    const int e = et * 16 + r16;
    const bf16* xr = x + (int64_t)t * H + 8 * kg;
    const bf16* wr = w + (int64_t)min(e, E - 1) * H + 8 * kg;
    const bool live = e < E;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int ksteps = H >> 5;
    // a contiguous range of k steps per wave, in batches of ROUTE_TILE_U
    // loads in flight, so consecutive steps of a row (the two 64-byte halves
    // of one 128-byte line) are read by the same wave close together (the
    // 4096-token Granite-shaped launch 15.7 -> 15.0 us against steps strided
    // over the waves); steps past the range load its last step again and
    // multiply zeros.  Over a full grid batches of 8 or 12 measured slower
    // than 4 (4096 tokens, strided steps: 15.3 us at 4, 18.3 at 8, 15.7 at
    // 12; contiguous: 15.0 at 4, 17.4 at 8).
    const int per = (ksteps + n_sp - 1) / n_sp;
    const int kb = sp * per, ke = min(ksteps, kb + per);
    constexpr int U = ROUTE_TILE_U;
    for (int ks = kb; ks < ke; ks += U) {
      bf16x8_t a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = min(ks + u, ke - 1) << 5;
        a[u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xr + kk));
        b[u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wr + kk));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!live || ks + u >= ke) b[u] = __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
      }
    }
    // accumulator: rows (tokens) 4*kg+i, column (expert) r16
#pragma unroll
    for (int i = 0; i < 4; ++i) lds.part[sp][4 * kg + i][et * 16 + r16] = acc[i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ROUTE_TOK * MOE_MAX_EXPERTS; idx += ROUTE_TOK * MOE_WAVE) {
    const int tt = idx / MOE_MAX_EXPERTS, e = idx % MOE_MAX_EXPERTS;
    float s = 0.f;
    for (int p = 0; p < n_sp; ++p) s += lds.part[p][tt][e];
    lds.logits[tt][e] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ void tile_logits(const float* __restrict__ x, const float* __restrict__ w,
                                            int T, int H, int E, int t0, RouteLds& lds) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int t = t0 + wv;
  if (t < T) {
    for (int e = 0; e < E; ++e) {
      float acc = 0.f;
      for (int h = lane * 8; h < H; h += 8 * MOE_WAVE) {
        float a8[8], b8[8];
        elem<float>::load8(x + (int64_t)t * H + h, a8);
        elem<float>::load8(w + (int64_t)e * H + h, b8);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(a8[j], b8[j], acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) lds.logits[wv][e] = acc;
    }
  }
  __syncthreads();
}

#ifndef ROUTE_LOGIT_WAVES
#define ROUTE_LOGIT_WAVES 8
#endif
constexpr int LOGIT_WAVES = ROUTE_LOGIT_WAVES;

// Logits of tokens 16*blockIdx.x.. and experts 16*blockIdx.y.. into
// logits [T][E].
__global__ void __launch_bounds__(LOGIT_WAVES * MOE_WAVE)
route_logits_kernel(const bf16* __restrict__ x, const bf16* __restrict__ w, int T, int H, int E,
                    float* __restrict__ logits, int32_t* __restrict__ zero_me) {
  // the top-k kernel that follows counts its finished blocks here
  if (zero_me && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *zero_me = 0;
  __shared__ f32x4_t part[LOGIT_WAVES - 1][MOE_WAVE];
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const bf16* xr = x + (int64_t)min(t0 + r16, T - 1) * H + 8 * kg;
  const bf16* wr = w + (int64_t)min(e0 + r16, E - 1) * H + 8 * kg;
  const bool live = e0 + r16 < E;
#ifndef ROUTE_LOGIT_U
#define ROUTE_LOGIT_U 4
#endif
  constexpr int U = ROUTE_LOGIT_U;
  const int ksteps = H >> 5;
  const int per = (ksteps + LOGIT_WAVES - 1) / LOGIT_WAVES;
  const int kb = wv * per, ke = min(ksteps, kb + per);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = kb; k0 < ke; k0 += U) {
    bf16x8_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ko = min(k0 + u, ke - 1) << 5;
      a[u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xr + ko));
      b[u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wr + ko));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool on = live && k0 + u < ke;
      const bf16x8_t bv = on ? b[u] : __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bv, acc, 0, 0, 0);
    }
  }
  if (wv > 0) part[wv - 1][lane] = acc;
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int p = 0; p < LOGIT_WAVES - 1; ++p) acc += part[p][lane];
    // accumulator: rows (tokens) 4*kg+i, column (expert) r16
    const int e = e0 + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * kg + i;
      if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i];
    }
  }
}

__global__ void __launch_bounds__(LOGIT_WAVES * MOE_WAVE)
route_logits_kernel(const float* __restrict__ x, const float* __restrict__ w, int T, int H, int E,
                    float* __restrict__ logits, int32_t* __restrict__ zero_me) {
  const int tid = threadIdx.x;
  if (zero_me && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *zero_me = 0;
  if (tid >= 256) return;
  const int t = blockIdx.x * 16 + (tid >> 4), e = blockIdx.y * 16 + (tid & 15);
  if (t >= T || e >= E) return;
  const float* xr = x + (int64_t)t * H;
  const float* wr = w + (int64_t)e * H;
  float acc = 0.f;
  for (int h = 0; h < H; h += 4) {
    const float4 a = *reinterpret_cast<const float4*>(xr + h);
    const float4 b = *reinterpret_cast<const float4*>(wr + h);
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  logits[(int64_t)t * E + e] = acc;
}

template <typename Tin>
__device__ __forceinline__ float wave_dot(const Tin* __restrict__ a, const Tin* __restrict__ b, int H) {
  // a lane's 8-element chunks in ascending order, four loads in flight at a
  // time (chunks past H are neither loaded nor added)
  constexpr int STEP = 8 * MOE_WAVE;
  float acc = 0.f;
  for (int h0 = lane_id() * 8; h0 < H; h0 += 4 * STEP) {
    float a8[4][8], b8[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (h0 + u * STEP < H) {
        elem<Tin>::load8(a + h0 + u * STEP, a8[u]);
        elem<Tin>::load8(b + h0 + u * STEP, b8[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (h0 + u * STEP < H) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(a8[u][j], b8[u][j], acc);
      }
    }
  }
  return wave_sum(acc);
}

// Everything after the logits for token t, one wave, lane = expert: shared
// gate, softmax, routed top-k, near-tie flag, mass, residency split or
// stall-free substitution, weights.  l is this lane's logit (-inf past E).
template <typename Tin>
__device__ __forceinline__ void route_topk_token(
    int t, float l, const Tin* __restrict__ x, int H, int E, int k, int renorm, float margin,
    int mode, const uint64_t* __restrict__ resident, int64_t res_stride,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, uint8_t* __restrict__ exact,
    uint32_t* __restrict__ flags, float* __restrict__ mass_out, const Tin* __restrict__ w_sg,
    float* __restrict__ g_s) {
  const int lane = lane_id();
  if (g_s) {
    const float gd = w_sg ? wave_dot<Tin>(x + (int64_t)t * H, w_sg, H) : 0.f;
    if (lane == 0) g_s[t] = w_sg ? sigmoid_f(gd) : 1.f;
  }

  // softmax numerator / denominator
  const float mx = wave_max(l);
  const float ex = lane < E ? __expf(l - mx) : 0.f;
  const float denom = wave_sum(ex);

  // routed top-k: rank of each expert's key among all experts
  const uint64_t key = lane < E ? topk_key(l, lane) : 0ull;
  const int rank = key_rank(key, E);
  const uint64_t routed = __ballot(lane < E && rank < k);
  uint32_t flag = 0;
  if (k < E && lane_logit_at_rank(l, rank, k - 1, E) - lane_logit_at_rank(l, rank, k, E) < margin)
    flag |= 1u;
  const bool in_routed = lane < E && rank < k;
  const float mass = wave_sum(in_routed ? ex : 0.f) / denom;

  uint64_t res_mask = ~0ull;
  if (mode == MOE_MODE_LORE || mode == MOE_MODE_STALL_FREE) res_mask = resident[res_stride * t];
  const uint64_t all_e = (E == 64) ? ~0ull : ((1ull << E) - 1ull);

  // final set: routed, or the top-k inside the prefetched set (stall-free)
  bool in_final = in_routed;
  int slot = rank;
  if (mode == MOE_MODE_STALL_FREE && (routed & ~res_mask) != 0ull) {
    const uint64_t allowed = res_mask & all_e;
    const int na = __popcll(allowed);
    const bool ok = (allowed >> lane) & 1ull;
    if (na >= k) {
      const int mrank = key_rank(ok ? key : 0ull, E);
      in_final = ok && mrank < k;
      slot = mrank;
      if (na > k) {
        const int mr = ok ? mrank : E;
        if (lane_logit_at_rank(l, mr, k - 1, E) - lane_logit_at_rank(l, mr, k, E) < margin) flag |= 4u;
      }
    } else {
      // fewer than k prefetched experts (lists of k + delta >= k never are):
      // all of them are kept and the remaining k - na slots take the best
      // experts outside the set by router score (flag 32)
      const bool out = lane < E && !ok;
      const int nrank = key_rank(out ? key : 0ull, E);  // rank among the experts outside
      const int need = k - na;
      in_final = lane < E && (ok || nrank < need);
      flag |= 32u;
      if (E > k) {
        const int nr = out ? nrank : E;
        if (lane_logit_at_rank(l, nr, need - 1, E) - lane_logit_at_rank(l, nr, need, E) < margin) flag |= 4u;
      }
      slot = key_rank(in_final ? key : 0ull, E);
    }
  }

  // slots in (-logit, id) order, weights p_e (renormalised over the set)
  const float fsum = wave_sum(in_final ? ex : 0.f);
  if (in_final) {
    const int64_t o = (int64_t)t * k + slot;
    topk_ids[o] = lane;
    topk_w[o] = renorm ? ex / fsum : ex / denom;
    exact[o] = (mode == MOE_MODE_LORE) ? (uint8_t)((res_mask >> lane) & 1ull) : (uint8_t)1;
  }
  if (lane == 0) {
    flags[t] = flag;
    if (mass_out) mass_out[t] = mass;
  }
}

// On logits [T][E] from route_logits_kernel: top-k of TPB tokens per block (one wave each).  TPB == PERM_WAVES (1024
// threads): the batch's (token, slot) pairs are also permuted in this launch.
template <typename Tin, int TPB>
__global__ void __launch_bounds__(TPB * MOE_WAVE)
route_topk_kernel(const Tin* __restrict__ x, const float* __restrict__ logits, int T, int H, int E,
                  int k, int renorm, float margin, int mode, const uint64_t* __restrict__ resident,
                  int64_t res_stride, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                  uint8_t* __restrict__ exact, uint32_t* __restrict__ flags,
                  float* __restrict__ mass_out, const Tin* __restrict__ w_sg,
                  float* __restrict__ g_s, PermOut po) {
  const int lane = lane_id();
  const int t = blockIdx.x * TPB + (threadIdx.x >> 6);
  if (t < T) {
    const float l = lane < E ? logits[(int64_t)t * E + lane] : -INFINITY;
    route_topk_token<Tin>(t, l, x, H, E, k, renorm, margin, mode, resident, res_stride, topk_ids,
                          topk_w, exact, flags, mass_out, w_sg, g_s);
  }
  if constexpr (TPB == PERM_WAVES) {
    // fused permutation (at most one 1024-pair chunk): the last block to
    // finish its tokens sorts every pair; the logits kernel zeroed the count
    // (one wave fences: the barrier has put every wave's stores in L2, and
    // a device-scope fence writes back / invalidates whole caches)
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
      __threadfence();
      s_last = atomicAdd(po.counter, 1) == (int)gridDim.x - 1;
      if (s_last) __threadfence();
    }
    __syncthreads();
    if (s_last)
      permute_chunk(0, 1, T * k, E, topk_ids, exact, nullptr, po.offsets, po.perm, po.inv,
                    po.row_of, po.miss_offsets);
  }
}

// Places the P <= 64 (token, slot) pairs of a small batch: the stable
// counting sort of permute_chunk done by one wave (lane = pair) with no
// barrier.  Bucket counts in LDS (a wave's LDS operations complete in
// order), one wave scan over the 2E buckets (two per lane), and a pair's
// rank among equal buckets from the ballots of its bucket bits.  Called by
// the 64 lanes of one wave after ids / exact are visible to it.
__device__ __forceinline__ void permute_one_wave(int P, int E, const int32_t* __restrict__ ids,
                                                 const uint8_t* __restrict__ exact, int* cnt,
                                                 const PermOut& po) {
  const int lane = lane_id(), NB = 2 * E;
  const int b = lane < P ? bucket_of(lane, E, ids, exact) : -1;
  cnt[2 * lane] = 0;
  cnt[2 * lane + 1] = 0;
  __builtin_amdgcn_wave_barrier();
  if (b >= 0) atomicAdd(&cnt[b], 1);
  __builtin_amdgcn_wave_barrier();
  const int c0 = cnt[2 * lane], c1 = cnt[2 * lane + 1];
  const int sc = wave_incl_scan_i(c0 + c1);
  const int base0 = sc - c0 - c1, base1 = sc - c1;  // first positions of buckets 2l, 2l+1
  const int total = __builtin_amdgcn_readlane(sc, MOE_WAVE - 1);
  if (2 * lane <= E) po.offsets[2 * lane] = base0;
  if (2 * lane + 1 <= E) po.offsets[2 * lane + 1] = base1;
  if (po.miss_offsets) {
    if (2 * lane >= E && 2 * lane < NB) po.miss_offsets[2 * lane - E] = base0;
    if (2 * lane + 1 >= E && 2 * lane + 1 < NB) po.miss_offsets[2 * lane + 1 - E] = base1;
    if (lane == 0) po.miss_offsets[E] = total;
  }
  const int v = b + 1;  // 0..128
  uint64_t peers = __ballot(1);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = (v >> bit) & 1;
    const uint64_t bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  const int bl = b >= 0 ? b >> 1 : 0;
  const int bb0 = __shfl(base0, bl, MOE_WAVE), bb1 = __shfl(base1, bl, MOE_WAVE);
  if (b >= 0) {
    const int pos = ((b & 1) ? bb1 : bb0) + rank;
    po.perm[pos] = lane;
    po.inv[lane] = b < E ? pos : -1;
    if (po.row_of) po.row_of[lane] = pos;
  } else if (lane < P) {
    po.inv[lane] = -1;
    if (po.row_of) po.row_of[lane] = -1;
  }
}

// Top-k of a batch of at most ROUTE_TOPK_SMALL_T tokens (one wave each) and
// its permutation by wave 0, in one small block: the 1024-thread top-k block
// with the chunk permutation took about 7 us at one token.
constexpr int ROUTE_TOPK_SMALL_T = 4;
template <typename Tin>
__global__ void __launch_bounds__(ROUTE_TOPK_SMALL_T * MOE_WAVE)
route_topk_small_kernel(const Tin* __restrict__ x, const float* __restrict__ logits, int T, int H,
                        int E, int k, int renorm, float margin, int mode,
                        const uint64_t* __restrict__ resident, int64_t res_stride,
                        int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                        uint8_t* __restrict__ exact, uint32_t* __restrict__ flags,
                        float* __restrict__ mass_out, const Tin* __restrict__ w_sg,
                        float* __restrict__ g_s, PermOut po) {
  __shared__ int cnt[PERM_BUCKETS];
  const int lane = lane_id(), t = threadIdx.x >> 6;
  if (t < T) {
    const float l = lane < E ? logits[(int64_t)t * E + lane] : -INFINITY;
    route_topk_token<Tin>(t, l, x, H, E, k, renorm, margin, mode, resident, res_stride, topk_ids,
                          topk_w, exact, flags, mass_out, w_sg, g_s);
  }
  __syncthreads();  // the waves' ids / exact stores before wave 0 reads them
  if (t == 0) permute_one_wave(T * k, E, topk_ids, exact, cnt, po);
}

// Small batches: logits and top-k in one launch.  A 1024-thread block takes
// tpb tokens (<= 16): its 16 waves form the logits of a 16-row token tile on
// the matrix cores (rows past tpb belong to the next block and go unused),
// then wave j ranks token t0 + j.  po.perm != nullptr (a single block and at
// most 1024 pairs): the block then permutes the batch's pairs itself.
#ifndef ROUTE_FUSED_WAVE_PERM
#define ROUTE_FUSED_WAVE_PERM 1
#endif
template <typename Tin>
__global__ void __launch_bounds__(1024)
route_fused_kernel(const Tin* __restrict__ x, const Tin* __restrict__ w_router, int T, int H,
                   int E, int tpb, int k, int renorm, float margin, int mode,
                   const uint64_t* __restrict__ resident, int64_t res_stride,
                   int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                   uint8_t* __restrict__ exact, uint32_t* __restrict__ flags,
                   float* __restrict__ logits_out, float* __restrict__ mass_out,
                   const Tin* __restrict__ w_sg, float* __restrict__ g_s, PermOut po) {
  __shared__ RouteLds lds;
  const int t0 = blockIdx.x * tpb;
  tile_logits(x, w_router, T, H, E, t0, lds);
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int t = t0 + wv;
  if (wv < tpb && t < T) {
    const float l = lane < E ? lds.logits[wv][lane] : -INFINITY;
    if (lane < E) logits_out[(int64_t)t * E + lane] = l;
    route_topk_token<Tin>(t, l, x, H, E, k, renorm, margin, mode, resident, res_stride, topk_ids,
                          topk_w, exact, flags, mass_out, w_sg, g_s);
  }
  if (po.perm) {  // block-uniform; the barrier orders the waves' writes within the workgroup
    __syncthreads();
#if ROUTE_FUSED_WAVE_PERM
    if (T * k <= MOE_WAVE) {   // a few pairs: one wave sorts them, no block barriers
      __shared__ int cnt[PERM_BUCKETS];
      if (wv == 0) permute_one_wave(T * k, E, topk_ids, exact, cnt, po);
      return;
    }
#endif
    permute_chunk(0, 1, T * k, E, topk_ids, exact, nullptr, po.offsets, po.perm, po.inv,
                  po.row_of, po.miss_offsets);
  }
}

// APEX prefetch set: top-(k + delta_t) of x W_p^T as a bit mask.  ADAPT:
// delta_t is the adaptive budget [APEX page, Sec. 4.2]: with s = w . x_t,
// p_d = sigmoid(theta_d - s) >= tau  <=>  theta_d - s >= logit(tau) (lt), so
// lane d tests its own budget and the least qualifying lane is the budget
// (N - k when none qualifies).  Given the router's choices, the kernel also
// reports delta* (the least budget covering them: the largest prefetch rank
// among them, minus k - 1) and how many of them the list covers.
template <typename Tin, bool ADAPT>
__global__ void __launch_bounds__(1024)
prefetch_kernel(const Tin* __restrict__ x, const Tin* __restrict__ w_p, int T, int H, int E, int k,
                float margin, const int32_t* __restrict__ delta, uint64_t* __restrict__ mask_out,
                uint32_t* __restrict__ flags, const Tin* __restrict__ w_delta,
                const float* __restrict__ theta, float lt, const int32_t* __restrict__ routed,
                int32_t* __restrict__ delta_out, int32_t* __restrict__ delta_star_out,
                int32_t* __restrict__ overlap_out) {
  __shared__ RouteLds lds;
  const int t0 = blockIdx.x * ROUTE_TOK;
  tile_logits(x, w_p, T, H, E, t0, lds);
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int t = t0 + wv;
  if (t >= T) return;
  const float l = lane < E ? lds.logits[wv][lane] : -INFINITY;
  uint32_t flag = 0;
  int n;
  if constexpr (ADAPT) {
    const float sc = wave_dot<Tin>(x + (int64_t)t * H, w_delta, H);
    const int nd = E - k + 1;  // budgets 0..N-k
    const float g = lane < nd ? theta[lane] - sc - lt : -INFINITY;
    const uint64_t ok = __ballot(lane < nd && g >= 0.f);
    const int d = ok ? __ffsll((unsigned long long)ok) - 1 : nd - 1;
    if (__ballot((lane == d || lane == d - 1) && fabsf(g) < margin)) flag |= 16u;
    if (lane == 0) delta_out[t] = d;
    n = k + d;
  } else {
    n = k + delta[t];
  }
  n = n < 1 ? 1 : (n > E ? E : n);
  const int rank = key_rank(lane < E ? topk_key(l, lane) : 0ull, E);
  const uint64_t mask = __ballot(lane < E && rank < n);
  if (n < E && lane_logit_at_rank(l, rank, n - 1, E) - lane_logit_at_rank(l, rank, n, E) < margin)
    flag |= 2u;
  if constexpr (ADAPT) {
    if (routed) {
      int top = -1, cover = 0;
      for (int j = 0; j < k; ++j) {
        const int e = __builtin_amdgcn_readfirstlane(routed[(int64_t)t * k + j]);
        if (e < 0 || e >= E) continue;
        const int re = __builtin_amdgcn_readlane(rank, e);
        top = re > top ? re : top;
        cover += re < n ? 1 : 0;
      }
      if (lane == 0) {
        delta_star_out[t] = top + 1 - k > 0 ? top + 1 - k : 0;
        overlap_out[t] = cover;
      }
    }
  }
  if (lane == 0) {
    mask_out[t] = mask;
    flags[t] = flag;
  }
}

// Batches up to ROUTE_FUSED_MAX_T tokens with at most ROUTE_FUSED_MAX_E
// experts route in one launch (logits and top-k per block); so do batches of
// ROUTE_FUSED_BIG_T tokens or more, whose many blocks share the cost of
// streaming W_r through each CU.  The rest spread the logits over (token,
// expert) tiles first.  Tiny batches put fewer tokens in a block so more CUs
// share W_r.
#ifndef ROUTE_FUSED_MAX_T
#define ROUTE_FUSED_MAX_T 256
#endif
#ifndef ROUTE_FUSED_MAX_E
#define ROUTE_FUSED_MAX_E 16
#endif
#ifndef ROUTE_FUSED_BIG_T
#define ROUTE_FUSED_BIG_T 2048
#endif
#ifndef ROUTE_FUSED_SMALL_T
#define ROUTE_FUSED_SMALL_T 64
#endif
#ifndef ROUTE_FUSED_SMALL_TPB
#define ROUTE_FUSED_SMALL_TPB 4
#endif

hipError_t launch_route(const moe_dims_t& d, int T, const void* x, const void* w_router,
                        const uint64_t* resident, int64_t res_stride, int mode, int32_t* ids,
                        float* w, uint8_t* exact, uint32_t* flags, float* logits, float* mass,
                        const void* w_sg, float* g_s, hipStream_t s, const PermOut* po,
                        bool* permuted) {
  if (permuted) *permuted = false;
  if ((T <= ROUTE_FUSED_MAX_T && d.n_experts <= ROUTE_FUSED_MAX_E) || T >= ROUTE_FUSED_BIG_T) {
    const int tpb = T <= ROUTE_FUSED_SMALL_T ? ROUTE_FUSED_SMALL_TPB : ROUTE_TOK;
    const int blocks = (T + tpb - 1) / tpb;
    // one block holding every token also permutes the (<= 1024) pairs
    const bool fuse = po != nullptr && blocks == 1 && (int64_t)T * d.top_k <= PERM_THREADS;
    PermOut pp{};
    if (fuse) pp = *po;
    if (d.dtype == MOE_BF16)
      route_fused_kernel<bf16><<<blocks, 1024, 0, s>>>(
          (const bf16*)x, (const bf16*)w_router, T, d.hidden, d.n_experts, tpb, d.top_k,
          d.renormalize, d.tie_margin, mode, resident, res_stride, ids, w, exact, flags, logits,
          mass, (const bf16*)w_sg, g_s, pp);
    else
      route_fused_kernel<float><<<blocks, 1024, 0, s>>>(
          (const float*)x, (const float*)w_router, T, d.hidden, d.n_experts, tpb, d.top_k,
          d.renormalize, d.tie_margin, mode, resident, res_stride, ids, w, exact, flags, logits,
          mass, (const float*)w_sg, g_s, pp);
    if (permuted) *permuted = fuse;
    return hipGetLastError();
  }
  // a batch of at most one permutation chunk is sorted by the top-k launch
  const bool fuse = po != nullptr && (int64_t)T * d.top_k <= PERM_THREADS;
  const dim3 lgrid((T + 15) / 16, (d.n_experts + 15) / 16);
  // at most four tokens: one small top-k block whose first wave permutes
  // (DeepSeek-V2-Lite shape, one token: the step 40.1 -> 38.5 us)
  const bool small = fuse && T <= ROUTE_TOPK_SMALL_T;
  int32_t* zero_me = (fuse && !small) ? po->counter : nullptr;
  const PermOut none{};
  if (d.dtype == MOE_BF16) {
    route_logits_kernel<<<lgrid, LOGIT_WAVES * MOE_WAVE, 0, s>>>(
        (const bf16*)x, (const bf16*)w_router, T, d.hidden, d.n_experts, logits, zero_me);
    if (small)
      route_topk_small_kernel<bf16><<<1, T * MOE_WAVE, 0, s>>>(
          (const bf16*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const bf16*)w_sg, g_s, *po);
    else if (fuse)
      route_topk_kernel<bf16, PERM_WAVES><<<(T + PERM_WAVES - 1) / PERM_WAVES, PERM_THREADS, 0, s>>>(
          (const bf16*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const bf16*)w_sg, g_s, *po);
    else
      route_topk_kernel<bf16, 4><<<(T + 3) / 4, 256, 0, s>>>(
          (const bf16*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const bf16*)w_sg, g_s, none);
  } else {
    route_logits_kernel<<<lgrid, LOGIT_WAVES * MOE_WAVE, 0, s>>>(
        (const float*)x, (const float*)w_router, T, d.hidden, d.n_experts, logits, zero_me);
    if (small)
      route_topk_small_kernel<float><<<1, T * MOE_WAVE, 0, s>>>(
          (const float*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const float*)w_sg, g_s, *po);
    else if (fuse)
      route_topk_kernel<float, PERM_WAVES><<<(T + PERM_WAVES - 1) / PERM_WAVES, PERM_THREADS, 0, s>>>(
          (const float*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const float*)w_sg, g_s, *po);
    else
      route_topk_kernel<float, 4><<<(T + 3) / 4, 256, 0, s>>>(
          (const float*)x, logits, T, d.hidden, d.n_experts, d.top_k, d.renormalize, d.tie_margin,
          mode, resident, res_stride, ids, w, exact, flags, mass, (const float*)w_sg, g_s, none);
  }
  if (permuted) *permuted = fuse;
  return hipGetLastError();
}

hipError_t launch_prefetch(const moe_dims_t& d, int T, const void* x, const void* w_p,
                           const int32_t* delta, uint64_t* mask_out, uint32_t* flags,
                           hipStream_t s) {
  const int blocks = (T + ROUTE_TOK - 1) / ROUTE_TOK;
  if (d.dtype == MOE_BF16)
    prefetch_kernel<bf16, false><<<blocks, 1024, 0, s>>>(
        (const bf16*)x, (const bf16*)w_p, T, d.hidden, d.n_experts, d.top_k, d.tie_margin, delta,
        mask_out, flags, nullptr, nullptr, 0.f, nullptr, nullptr, nullptr, nullptr);
  else
    prefetch_kernel<float, false><<<blocks, 1024, 0, s>>>(
        (const float*)x, (const float*)w_p, T, d.hidden, d.n_experts, d.top_k, d.tie_margin, delta,
        mask_out, flags, nullptr, nullptr, 0.f, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefetch_adaptive(const moe_dims_t& d, int T, const void* x, const void* w_p,
                                    const void* w_delta, const float* theta, float logit_tau,
                                    const int32_t* routed, int32_t* delta_out,
                                    uint64_t* mask_out, uint32_t* flags, int32_t* delta_star,
                                    int32_t* overlap, hipStream_t s) {
  const int blocks = (T + ROUTE_TOK - 1) / ROUTE_TOK;
  if (d.dtype == MOE_BF16)
    prefetch_kernel<bf16, true><<<blocks, 1024, 0, s>>>(
        (const bf16*)x, (const bf16*)w_p, T, d.hidden, d.n_experts, d.top_k, d.tie_margin,
        nullptr, mask_out, flags, (const bf16*)w_delta, theta, logit_tau, routed, delta_out,
        delta_star, overlap);
  else
    prefetch_kernel<float, true><<<blocks, 1024, 0, s>>>(
        (const float*)x, (const float*)w_p, T, d.hidden, d.n_experts, d.top_k, d.tie_margin,
        nullptr, mask_out, flags, (const float*)w_delta, theta, logit_tau, routed, delta_out,
        delta_star, overlap);
  return hipGetLastError();
}

}  // namespace moe
