// FloE expert [FloE page, Sec. 1 "Hybrid compression"; Sec. 3 sparse GEMV]:
//   u = x W_up with 2-bit group-quantised W_up, decoded in registers;
//   S_t keeps the floe_keep channels of largest |u| (ties -> lower channel);
//   g_i = x . W_gate[i] and a_i = SiLU(g_i) u_i only for kept channels;
//   y = sum over kept i of a_i W_down[i, :]  (down stored channel-major).
//
// up:     one wave per up row; lane l owns the 64 inputs of quantisation
//         group l (16 bytes of codes = one 16-byte load), keeps its 64 x values
//         and their sum in registers across rows, and forms
//         s * (sum_h q_h x_h - z * sum_h x_h) -- the group's (q - z) * s dot
//         product -- before one wave reduction.  Codes are unpacked four at a
//         time: (word >> 2j) & 0x03030303 leaves code j of every byte in that
//         byte, which converts to float with a single byte-to-float op.
// select: one 1024-thread workgroup per pair, |u| bit patterns (monotone for
//         non-negative floats) in LDS, MSB-first 8-bit radix select for the
//         keep-th largest, then two block scans to list kept channels in
//         ascending order, equal keys resolved toward lower channels.
// gate:   one wave per kept channel row (contiguous H-vector).
// down:   each thread owns 8 output columns and sweeps a slice of the kept
//         channel rows; slices are summed by a small reduction kernel.
#include "common.h"

namespace moe {

constexpr int FLOE_ROWS_PER_BLOCK = 16;
constexpr int FLOE_SELECT_THREADS = 1024;
constexpr int FLOE_MAX_INTER = 16384;
constexpr int FLOE_DOWN_SLICE = 32;

// Pair position p -> (pair f, token t, expert e).  e is the segment of the
// permutation holding p: the largest e with offsets[e] <= p.
__device__ __forceinline__ bool pair_of(int p, int E, int k, const int32_t* __restrict__ offsets,
                                        const int32_t* __restrict__ perm, int& f, int& t, int& e) {
  if (p >= offsets[E]) return false;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  e = lo;
  f = perm[p];
  t = f / k;
  return true;
}

template <typename Tin>
__global__ void __launch_bounds__(256)
floe_up_kernel(const Tin* __restrict__ x, const uint8_t* __restrict__ up_q,
               const uint16_t* __restrict__ up_s, const uint16_t* __restrict__ up_z, int H, int I,
               int E, int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
               float* __restrict__ u_out) {
  int f, t, e;
  if (!pair_of(blockIdx.y, E, k, offsets, perm, f, t, e)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int G = H >> 6;  // groups per row
  const Tin* xr = x + (int64_t)t * H;
  for (int g0 = 0; g0 < G; g0 += MOE_WAVE) {
    const int g = g0 + lane;
    const bool act = g < G;
    float xv[64];
    float xs = 0.f;
    if (act) {
#pragma unroll
      for (int c = 0; c < 64; c += 8) {
        float v8[8];
        elem<Tin>::load8(xr + (int64_t)g * 64 + c, v8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[c + j] = v8[j];
          xs += v8[j];
        }
      }
    }
    for (int q = 0; q < FLOE_ROWS_PER_BLOCK / 4; ++q) {
      const int i = blockIdx.x * FLOE_ROWS_PER_BLOCK + wv * (FLOE_ROWS_PER_BLOCK / 4) + q;
      const int64_t row = (int64_t)e * I + i;
      float part = 0.f;
      if (act) {
        const uint4 cw = *reinterpret_cast<const uint4*>(up_q + row * (H >> 2) + (int64_t)g * 16);
        const float s = half_bits_to_f(up_s[row * G + g]);
        const float z = half_bits_to_f(up_z[row * G + g]);
        const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t m = (words[w] >> (2 * j)) & 0x03030303u;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              acc = fmaf((float)((m >> (8 * b)) & 0xFFu), xv[w * 16 + 4 * b + j], acc);
          }
        }
        part = s * (acc - z * xs);
      }
      const float uval = wave_sum(part);
      if (lane == 0) {
        if (g0 == 0)
          u_out[(int64_t)blockIdx.y * I + i] = uval;
        else
          u_out[(int64_t)blockIdx.y * I + i] += uval;
      }
    }
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int s = v;
#pragma unroll
  for (int o = 1; o < MOE_WAVE; o <<= 1) {
    const int n = __shfl_up(s, o, MOE_WAVE);
    if (lane >= o) s += n;
  }
  if (lane == MOE_WAVE - 1) wsum[wv] = s;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < FLOE_SELECT_THREADS / MOE_WAVE; ++w) {
    const int c = wsum[w];
    if (w < wv) base += c;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + s - v;
}

__global__ void __launch_bounds__(FLOE_SELECT_THREADS)
floe_select_kernel(const float* __restrict__ u, int I, int n_keep, float margin, int E, int k,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                   int32_t* __restrict__ keep_out,
                   uint32_t* __restrict__ flags) {
  __shared__ uint32_t keys[FLOE_MAX_INTER];
  __shared__ int hist[256];
  __shared__ int wsum[FLOE_SELECT_THREADS / MOE_WAVE];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ uint32_t s_next;
  int f, t, e;
  if (!pair_of(blockIdx.x, E, k, offsets, perm, f, t, e)) return;
  const int tid = threadIdx.x, lane = lane_id();
  const float* ur = u + (int64_t)blockIdx.x * I;
  for (int i = tid; i < I; i += FLOE_SELECT_THREADS) keys[i] = __float_as_uint(fabsf(ur[i]));
  if (tid == 0) {
    s_prefix = 0u;
    s_need = n_keep;
    s_next = 0u;
  }
  __syncthreads();
  uint32_t pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int i = tid; i < I; i += FLOE_SELECT_THREADS) {
      const uint32_t kk = keys[i];
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    if (tid < MOE_WAVE) {
      const int need = s_need;
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                h3 = hist[4 * lane + 3];
      const int c4 = h0 + h1 + h2 + h3;
      int suf = c4;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < MOE_WAVE; o <<= 1) {
        const int n = __shfl_down(suf, o, MOE_WAVE);
        if (lane + o < MOE_WAVE) suf += n;
      }
      const uint64_t bal = __ballot(suf >= need);
      const int L = 63 - __clzll(bal);  // highest lane whose suffix reaches need
      if (lane == L) {
        int gt = suf - c4;
        const int hb[4] = {h0, h1, h2, h3};
        int b = 3;
        for (; b > 0; --b) {
          if (gt + hb[b] >= need) break;
          gt += hb[b];
        }
        s_prefix = prefix | ((uint32_t)(4 * L + b) << shift);
        s_need = need - gt;
      }
    }
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int need_eq = s_need;
  // chunk of consecutive channels per thread
  const int ch = (I + FLOE_SELECT_THREADS - 1) / FLOE_SELECT_THREADS;
  const int i0 = tid * ch, i1 = min(I, i0 + ch);
  int n_eq = 0;
  uint32_t below_max = 0u;
  for (int i = i0; i < i1; ++i) {
    const uint32_t kk = keys[i];
    n_eq += kk == thr;
    if (kk < thr && kk > below_max) below_max = kk;
  }
  int eq_total;
  int eq_rank = block_excl_scan(n_eq, wsum, eq_total);
  int n_kept = 0;
  {
    int r = eq_rank;
    for (int i = i0; i < i1; ++i) {
      const uint32_t kk = keys[i];
      if (kk > thr) ++n_kept;
      else if (kk == thr) { if (r < need_eq) ++n_kept; ++r; }
    }
  }
  int kept_total;
  int pos = block_excl_scan(n_kept, wsum, kept_total);
  {
    int r = eq_rank;
    int32_t* ko = keep_out + (int64_t)f * n_keep;
    for (int i = i0; i < i1; ++i) {
      const uint32_t kk = keys[i];
      bool kp = kk > thr;
      if (kk == thr) { kp = r < need_eq; ++r; }
      if (kp) ko[pos++] = i;
    }
  }
  // near-tie at the edge: next value below the threshold, or a tie at it
  if (n_keep < I) {
    uint32_t m = below_max;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t v = __shfl_xor(m, o, MOE_WAVE);
      m = v > m ? v : m;
    }
    if (lane == 0) atomicMax(&s_next, m);
    __syncthreads();
    if (tid == 0) {
      const bool tie = eq_total > need_eq || (__uint_as_float(thr) - __uint_as_float(s_next)) < margin;
      if (tie) atomicOr(&flags[t], 8u);
    }
  }
}

template <typename Tin>
__global__ void __launch_bounds__(256)
floe_gate_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wg, const float* __restrict__ u,
                 int H, int I, int n_keep, int E, int k, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, const int32_t* __restrict__ keep,
                 float* __restrict__ a_out) {
  int f, t, e;
  if (!pair_of(blockIdx.y, E, k, offsets, perm, f, t, e)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const Tin* xr = x + (int64_t)t * H;
  for (int q = 0; q < FLOE_ROWS_PER_BLOCK / 4; ++q) {
    const int c = blockIdx.x * FLOE_ROWS_PER_BLOCK + wv * (FLOE_ROWS_PER_BLOCK / 4) + q;
    if (c >= n_keep) break;
    const int i = keep[(int64_t)f * n_keep + c];
    const Tin* row = wg + ((int64_t)e * I + i) * H;
    float acc = 0.f;
    for (int h = lane * 8; h < H; h += 8 * MOE_WAVE) {
      float w8[8], x8[8];
      elem<Tin>::load8(row + h, w8);
      elem<Tin>::load8(xr + h, x8);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(w8[j], x8[j], acc);
    }
    const float g = wave_sum(acc);
    if (lane == 0) a_out[(int64_t)blockIdx.y * n_keep + c] = silu_f(g) * u[(int64_t)blockIdx.y * I + i];
  }
}

template <typename Tin>
__global__ void __launch_bounds__(256)
floe_down_kernel(const Tin* __restrict__ wd, const float* __restrict__ a, int H, int I, int n_keep,
                 int P_max, int E, int k, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, const int32_t* __restrict__ keep,
                 float* __restrict__ part) {
  int f, t, e;
  if (!pair_of(blockIdx.z, E, k, offsets, perm, f, t, e)) return;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (h >= H) return;
  const int c0 = blockIdx.y * FLOE_DOWN_SLICE, c1 = min(n_keep, c0 + FLOE_DOWN_SLICE);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* ar = a + (int64_t)blockIdx.z * n_keep;
  const int32_t* kr = keep + (int64_t)f * n_keep;
  for (int c = c0; c < c1; ++c) {
    const float av = ar[c];
    float w8[8];
    elem<Tin>::load8(wd + ((int64_t)e * I + kr[c]) * H + h, w8);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(av, w8[j], acc[j]);
  }
  float* o = part + ((int64_t)blockIdx.y * P_max + blockIdx.z) * H + h;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = acc[j];
}

__global__ void __launch_bounds__(256)
floe_reduce_kernel(const float* __restrict__ part, int H, int n_slices, int P_max, int E,
                   const int32_t* __restrict__ offsets, float* __restrict__ y) {
  const int p = blockIdx.y;
  if (p >= offsets[E]) return;
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  float s = 0.f;
  for (int sl = 0; sl < n_slices; ++sl) s += part[((int64_t)sl * P_max + p) * H + h];
  y[(int64_t)p * H + h] = s;
}

int floe_slices(int n_keep) { return (n_keep + FLOE_DOWN_SLICE - 1) / FLOE_DOWN_SLICE; }
int floe_max_inter() { return FLOE_MAX_INTER; }

template <typename Tin>
static hipError_t launch_floe_t(const moe_dims_t& d, int T, const Tin* x, const moe_weights_t& w,
                                const int32_t* offsets, const int32_t* perm, float* u,
                                int32_t* keep, float* a, float* part, float* y_perm,
                                uint32_t* flags, const Prof& pf, hipStream_t s) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k, nk = d.floe_keep;
  const int P = T * k;
  if (P == 0) return hipSuccess;
  hipError_t e = pf.begin(MOE_KERNEL_FLOE_UP, s);
  floe_up_kernel<Tin><<<dim3(I / FLOE_ROWS_PER_BLOCK, P), 256, 0, s>>>(
      x, w.up_q, w.up_scale, w.up_zero, H, I, E, k, offsets, perm, u);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_UP, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_SELECT, s);
  floe_select_kernel<<<P, FLOE_SELECT_THREADS, 0, s>>>(u, I, nk, d.tie_margin, E, k, offsets, perm,
                                                        keep, flags);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_SELECT, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_GATE, s);
  floe_gate_kernel<Tin><<<dim3((nk + FLOE_ROWS_PER_BLOCK - 1) / FLOE_ROWS_PER_BLOCK, P), 256, 0, s>>>(
      x, (const Tin*)w.w_gate, u, H, I, nk, E, k, offsets, perm, keep, a);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_GATE, s);
  const int ns = floe_slices(nk);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_DOWN, s);
  floe_down_kernel<Tin><<<dim3((H + 2047) / 2048, ns, P), 256, 0, s>>>(
      (const Tin*)w.w_down, a, H, I, nk, P, E, k, offsets, perm, keep, part);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_DOWN, s);
  floe_reduce_kernel<<<dim3((H + 255) / 256, P), 256, 0, s>>>(part, H, ns, P, E, offsets, y_perm);
  return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_floe(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                       const int32_t* offsets, const int32_t* perm, float* u,
                       int32_t* keep, float* a, float* part, float* y_perm, uint32_t* flags,
                       const Prof& pf, hipStream_t s) {
  if (d.dtype == MOE_BF16)
    return launch_floe_t<bf16>(d, T, (const bf16*)x, w, offsets, perm, u, keep, a, part, y_perm,
                               flags, pf, s);
  return launch_floe_t<float>(d, T, (const float*)x, w, offsets, perm, u, keep, a, part, y_perm,
                              flags, pf, s);
}

}  // namespace moe
