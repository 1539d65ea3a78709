// Weighted combine with the LoRE surrogate fused in [SPICE page, "LoRE
// low-rank surrogate"]:
//   out[t] = g_s(t) y_s(t) + sum_j w_tj yhat_tj,
//   yhat_tj = y_perm[inv[t*k+j]]            (exact slot)
//           = y_s(t) + B_e (A_e x_t)        (non-resident slot).
// One 256-thread block per token.  The rank-r projections z_j = A_e x_t of
// the token's non-exact slots are wave dot products over H into LDS; each
// thread then owns output columns and adds B_e[h, :] . z_j (r contiguous
// values, 16-byte loads) for those slots.
#include "common.h"

namespace moe {

constexpr int COMBINE_THREADS = 256;

template <typename Tin>
__device__ __forceinline__ void lore_project(const Tin* __restrict__ xr, const Tin* __restrict__ lore_A,
                                             int H, int k, int r, const int* s_ids, const int* s_ex,
                                             float (*z)[MOE_MAX_LORE_RANK]) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  for (int idx = wv; idx < k * r; idx += COMBINE_THREADS / MOE_WAVE) {
    const int j = idx / r, q = idx - j * r;
    if (s_ex[j]) continue;
    const Tin* arow = lore_A + ((int64_t)s_ids[j] * r + q) * H;
    float acc = 0.f;
    for (int h = lane * 8; h < H; h += 8 * MOE_WAVE) {
      float a8[8], x8[8];
      elem<Tin>::load8(arow + h, a8);
      elem<Tin>::load8(xr + h, x8);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = fmaf(a8[c], x8[c], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) z[j][q] = acc;
  }
}

template <typename Tin>
__device__ __forceinline__ float lore_apply(const Tin* __restrict__ brow, int r, const float* zj) {
  float acc = 0.f;
  for (int q = 0; q < r; q += 8) {
    float b8[8];
    elem<Tin>::load8(brow + q, b8);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc = fmaf(b8[c], zj[q + c], acc);
  }
  return acc;
}

// lore_A / lore_B non-null: LoRE computed here.  Else lore_out (may be null)
// supplies the residuals.
template <typename Tin>
__global__ void __launch_bounds__(COMBINE_THREADS)
combine_kernel(int H, int k, int r, const float* __restrict__ y_perm, const int32_t* __restrict__ inv,
               const float* __restrict__ topk_w, const uint8_t* __restrict__ exact,
               const int32_t* __restrict__ ids, const float* __restrict__ y_s,
               const float* __restrict__ g_s, const float* __restrict__ lore_out,
               const Tin* __restrict__ x, const Tin* __restrict__ lore_A,
               const Tin* __restrict__ lore_B, Tin* __restrict__ out) {
  __shared__ float z[MOE_MAX_TOPK][MOE_MAX_LORE_RANK];
  __shared__ int s_ids[MOE_MAX_TOPK], s_ex[MOE_MAX_TOPK], s_row[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    const int64_t o = (int64_t)t * k + tid;
    s_ids[tid] = ids ? ids[o] : 0;
    s_ex[tid] = exact ? exact[o] : 1;
    s_row[tid] = inv[o];
    s_w[tid] = topk_w[o];
  }
  __syncthreads();
  const bool fused = lore_A != nullptr;
  if (fused) {
    lore_project<Tin>(x + (int64_t)t * H, lore_A, H, k, r, s_ids, s_ex, z);
    __syncthreads();
  }
  const float gs = g_s ? g_s[t] : 1.f;
  for (int h = tid; h < H; h += COMBINE_THREADS) {
    const float ys = y_s ? y_s[(int64_t)t * H + h] : 0.f;
    float acc = gs * ys;
    for (int j = 0; j < k; ++j) {
      float yj;
      if (s_ex[j] && s_row[j] >= 0) {
        yj = y_perm[(int64_t)s_row[j] * H + h];
      } else {
        float lr = 0.f;
        if (fused)
          lr = lore_apply<Tin>(lore_B + ((int64_t)s_ids[j] * H + h) * r, r, z[j]);
        else if (lore_out)
          lr = lore_out[((int64_t)t * k + j) * H + h];
        yj = ys + lr;
      }
      acc = fmaf(s_w[j], yj, acc);
    }
    elem<Tin>::store(out, (int64_t)t * H + h, acc);
  }
}

// Standalone LoRE residuals: lore_out[t][j] = B_e (A_e x_t) for non-exact
// slots, 0 for exact ones.
template <typename Tin>
__global__ void __launch_bounds__(COMBINE_THREADS)
lore_kernel(int H, int k, int r, const Tin* __restrict__ x, const int32_t* __restrict__ ids,
            const uint8_t* __restrict__ exact, const Tin* __restrict__ lore_A,
            const Tin* __restrict__ lore_B, float* __restrict__ lore_out) {
  __shared__ float z[MOE_MAX_TOPK][MOE_MAX_LORE_RANK];
  __shared__ int s_ids[MOE_MAX_TOPK], s_ex[MOE_MAX_TOPK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    s_ids[tid] = ids[(int64_t)t * k + tid];
    s_ex[tid] = exact[(int64_t)t * k + tid];
  }
  __syncthreads();
  lore_project<Tin>(x + (int64_t)t * H, lore_A, H, k, r, s_ids, s_ex, z);
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    float* o = lore_out + ((int64_t)t * k + j) * H;
    for (int h = tid; h < H; h += COMBINE_THREADS)
      o[h] = s_ex[j] ? 0.f : lore_apply<Tin>(lore_B + ((int64_t)s_ids[j] * H + h) * r, r, z[j]);
  }
}

// Combine over y_perm rows: out[t] = g_s y_s + sum_j w_j (y_perm[row_of[f]] +
// (exact ? 0 : y_s)), f = t*k + j.  Non-exact rows already hold B_e A_e x_t,
// so a surrogate slot contributes w_j (y_s + B_e A_e x_t).  Each thread owns
// four consecutive columns; y_perm rows are fp32 or bf16 (Ty), the sums fp32.
template <typename Ty>
__device__ __forceinline__ float4 load4(const Ty* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16>(const bf16* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return float4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
}

template <typename Tin>
__device__ __forceinline__ void store4(Tin* p, float a0, float a1, float a2, float a3);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a0, float a1, float a2, float a3) {
  *reinterpret_cast<float4*>(p) = float4{a0, a1, a2, a3};
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a0, float a1, float a2, float a3) {
  *reinterpret_cast<uint2*>(p) = make_uint2(f2_to_bf16x2(a0, a1), f2_to_bf16x2(a2, a3));
}

// grid (T tokens, H / (4 * COMBINE_THREADS) column blocks): a thread owns four
// consecutive columns of one token and issues the loads of all k slots
// before summing them; the token's slot table is read with scalar loads.
template <typename Tin, typename Ty>
__global__ void __launch_bounds__(COMBINE_THREADS)
combine_rows_kernel(int H, int k, const Ty* __restrict__ y_perm, const int32_t* __restrict__ row_of,
                    const float* __restrict__ topk_w, const uint8_t* __restrict__ exact,
                    const float* __restrict__ y_s, const float* __restrict__ g_s,
                    Tin* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * COMBINE_THREADS + threadIdx.x) * 4;
  if (h >= H) return;
  const float gs = g_s ? g_s[t] : 1.f;
  float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
  if (y_s) ys = *reinterpret_cast<const float4*>(y_s + (int64_t)t * H + h);
  int row[MOE_MAX_TOPK];
  float4 v[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    row[j] = j < k ? row_of[(int64_t)t * k + j] : -1;
    v[j] = row[j] >= 0 ? load4<Ty>(y_perm + (int64_t)row[j] * H + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float a0 = gs * ys.x, a1 = gs * ys.y, a2 = gs * ys.z, a3 = gs * ys.w;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (row[j] < 0) continue;
    const int64_t o = (int64_t)t * k + j;
    float4 vj = v[j];
    if (!exact[o]) {
      vj.x += ys.x; vj.y += ys.y; vj.z += ys.z; vj.w += ys.w;
    }
    const float wj = topk_w[o];
    a0 = fmaf(wj, vj.x, a0);
    a1 = fmaf(wj, vj.y, a1);
    a2 = fmaf(wj, vj.z, a2);
    a3 = fmaf(wj, vj.w, a3);
  }
  store4<Tin>(out + (int64_t)t * H + h, a0, a1, a2, a3);
}

// The same sums over bf16 rows with eight columns per thread (one 16-byte
// load per slot row, one 16-byte store), in the same order and rounding as
// combine_rows_kernel.
template <typename Tin>
__global__ void __launch_bounds__(COMBINE_THREADS)
combine_rows8_kernel(int H, int k, const bf16* __restrict__ y_perm, const int32_t* __restrict__ row_of,
                     const float* __restrict__ topk_w, const uint8_t* __restrict__ exact,
                     const float* __restrict__ y_s, const float* __restrict__ g_s,
                     Tin* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (h >= H) return;
  const float gs = g_s ? g_s[t] : 1.f;
  float ys[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (y_s) elem<float>::load8(y_s + (int64_t)t * H + h, ys);
  int row[MOE_MAX_TOPK];
  uint4 v[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    row[j] = j < k ? row_of[(int64_t)t * k + j] : -1;
    v[j] = row[j] >= 0 ? *reinterpret_cast<const uint4*>(y_perm + (int64_t)row[j] * H + h)
                       : make_uint4(0u, 0u, 0u, 0u);
  }
  float a[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) a[c] = gs * ys[c];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (row[j] < 0) continue;
    const int64_t o = (int64_t)t * k + j;
    const float wj = topk_w[o];
    const float sj = exact[o] ? 0.f : 1.f;
    const float f[8] = {bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y), bf16_hi(v[j].y),
                        bf16_lo(v[j].z), bf16_hi(v[j].z), bf16_lo(v[j].w), bf16_hi(v[j].w)};
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = fmaf(wj, fmaf(sj, ys[c], f[c]), a[c]);
  }
  store4<Tin>(out + (int64_t)t * H + h, a[0], a[1], a[2], a[3]);
  store4<Tin>(out + (int64_t)t * H + h + 4, a[4], a[5], a[6], a[7]);
}

// y_bf16: y_perm holds bf16 rows.
hipError_t launch_combine_rows(const moe_dims_t& d, int T, const void* y_perm, bool y_bf16,
                               const int32_t* row_of, const float* topk_w, const uint8_t* exact,
                               const float* y_s, const float* g_s, void* out, hipStream_t s) {
  const dim3 grid(T, (d.hidden + 4 * COMBINE_THREADS - 1) / (4 * COMBINE_THREADS));
  if (d.dtype == MOE_BF16) {
    if (y_bf16) {
      // eight columns per thread; blocks sized to the row (H % 64 == 0)
      const int need = d.hidden / 8;
      const int thr = need >= COMBINE_THREADS ? COMBINE_THREADS : ((need + 63) / 64) * 64;
      const dim3 grid8(T, (need + thr - 1) / thr);
      combine_rows8_kernel<bf16><<<grid8, thr, 0, s>>>(
          d.hidden, d.top_k, (const bf16*)y_perm, row_of, topk_w, exact, y_s, g_s, (bf16*)out);
    } else
      combine_rows_kernel<bf16, float><<<grid, COMBINE_THREADS, 0, s>>>(
          d.hidden, d.top_k, (const float*)y_perm, row_of, topk_w, exact, y_s, g_s, (bf16*)out);
  } else {
    combine_rows_kernel<float, float><<<grid, COMBINE_THREADS, 0, s>>>(
        d.hidden, d.top_k, (const float*)y_perm, row_of, topk_w, exact, y_s, g_s, (float*)out);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const moe_dims_t& d, int T, const float* y_perm, const int32_t* inv,
                          const float* topk_w, const uint8_t* exact, const int32_t* ids,
                          const float* y_s, const float* g_s, const float* lore_out, const void* x,
                          const void* lore_A, const void* lore_B, void* out, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    combine_kernel<bf16><<<T, COMBINE_THREADS, 0, s>>>(
        d.hidden, d.top_k, d.lore_rank, y_perm, inv, topk_w, exact, ids, y_s, g_s, lore_out,
        (const bf16*)x, (const bf16*)lore_A, (const bf16*)lore_B, (bf16*)out);
  else
    combine_kernel<float><<<T, COMBINE_THREADS, 0, s>>>(
        d.hidden, d.top_k, d.lore_rank, y_perm, inv, topk_w, exact, ids, y_s, g_s, lore_out,
        (const float*)x, (const float*)lore_A, (const float*)lore_B, (float*)out);
  return hipGetLastError();
}

hipError_t launch_lore(const moe_dims_t& d, int T, const void* x, const int32_t* ids,
                       const uint8_t* exact, const void* lore_A, const void* lore_B,
                       float* lore_out, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    lore_kernel<bf16><<<T, COMBINE_THREADS, 0, s>>>(d.hidden, d.top_k, d.lore_rank, (const bf16*)x,
                                                    ids, exact, (const bf16*)lore_A,
                                                    (const bf16*)lore_B, lore_out);
  else
    lore_kernel<float><<<T, COMBINE_THREADS, 0, s>>>(d.hidden, d.top_k, d.lore_rank,
                                                     (const float*)x, ids, exact,
                                                     (const float*)lore_A, (const float*)lore_B,
                                                     lore_out);
  return hipGetLastError();
}

}  // namespace moe
