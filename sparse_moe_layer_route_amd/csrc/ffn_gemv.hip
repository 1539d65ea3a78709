// Expert SwiGLU FFN as a multi-token GEMV: y = (SiLU(x W_g) * (x W_u)) W_d
// [FloE page, Sec. 1, forward a^S(x) with S_t = identity].
//
// Every weight matrix is stored with the contraction index contiguous
// (gate/up [I][H], down [H][I]), so each output channel is one coalesced
// 16-byte-per-lane sweep of a weight row by a wave64, dotted with several
// token rows at once, then a wave reduction.  One launch per projection covers the routed and the shared experts: each
// wave owns one output row and dots it with up to eight token rows per pass,
// so a small layer puts many short, independent row sweeps in flight instead
// of a few long chains.  Grid.y walks the experts that received pairs: block
// y finds the y-th non-empty segment from the offsets with one ballot, so no
// host round trip is needed; the shared experts follow with the identity
// token map.
#include "common.h"

namespace moe {

constexpr int GEMV_WAVES = 4;   // rows per block: one output row per wave
constexpr int GEMV_NT = 8;      // token rows dotted per pass over a weight row

// Routed segment blockIdx.y of the pair permutation: the blockIdx.y-th
// expert with a non-empty segment (e < 0: none).  Called by every thread.
struct SegInfo {
  int e;      // expert
  int seg0;   // first pair position of the segment
  int n;      // pairs in the segment
};
__device__ __forceinline__ SegInfo find_segment(int E, const int32_t* __restrict__ offsets) {
  __shared__ int s_e, s_seg0, s_n;
  if (threadIdx.x < MOE_WAVE) {
    const int lane = threadIdx.x;
    int o0 = 0, n = 0;
    if (lane < E) {
      o0 = offsets[lane];
      n = offsets[lane + 1] - o0;
    }
    const uint64_t bal = __ballot(n > 0);
    const int target = blockIdx.y;
    if (n > 0 && __popcll(bal & ((1ull << lane) - 1ull)) == target) {
      s_e = lane;
      s_seg0 = o0;
      s_n = n;
    }
    if (lane == 0 && __popcll(bal) <= target) s_e = -1;
  }
  __syncthreads();
  return SegInfo{s_e, s_seg0, s_n};
}

// One launch for the gate/up projections of the routed experts and the
// shared experts.  Grid.y: the first n_routed rows walk the experts that
// received pairs (act[pos][i]); the next n_shared rows are shared expert s
// over all T tokens (act_s[t][s * Is + i]).  Each wave owns one channel row
// i and sweeps it once per pass of GEMV_NT tokens:
//   act = SiLU(x_t . W_g[i]) * (x_t . W_u[i]).
template <typename Tin>
__global__ void __launch_bounds__(GEMV_WAVES * MOE_WAVE)
gemv_gate_up_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wg,
                    const Tin* __restrict__ wu, const Tin* __restrict__ wsg,
                    const Tin* __restrict__ wsu, int H, int I, int Is, int n_routed, int n_shared,
                    int E, int k, int T, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ perm, float* __restrict__ act,
                    float* __restrict__ act_s) {
  const bool routed = (int)blockIdx.y < n_routed;
  SegInfo sg{(int)blockIdx.y - n_routed, 0, T};
  if (routed) sg = find_segment(E, offsets);   // block-uniform branch
  if (sg.e < 0) return;
  const int rows = routed ? I : Is;
  const int i = blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6);
  if (i >= rows) return;
  const int lane = lane_id();
  const Tin* grow = (routed ? wg : wsg) + ((int64_t)sg.e * rows + i) * H;
  const Tin* urow = (routed ? wu : wsu) + ((int64_t)sg.e * rows + i) * H;
  for (int tk = 0; tk < sg.n; tk += GEMV_NT) {
    const int nv = min(GEMV_NT, sg.n - tk);
    const Tin* xr[GEMV_NT];
#pragma unroll
    for (int n = 0; n < GEMV_NT; ++n) {
      const int r = tk + (n < nv ? n : 0);
      const int tok = routed ? perm[sg.seg0 + r] / k : r;
      xr[n] = x + (int64_t)tok * H;
    }
    float ag[GEMV_NT], au[GEMV_NT];
#pragma unroll
    for (int n = 0; n < GEMV_NT; ++n) ag[n] = au[n] = 0.f;
    for (int c = lane * 8; c < H; c += 8 * MOE_WAVE) {
      float g8[8], u8[8];
      elem<Tin>::load8(grow + c, g8);
      elem<Tin>::load8(urow + c, u8);
#pragma unroll
      for (int n = 0; n < GEMV_NT; ++n) {
        if (n < nv) {
          float x8[8];
          elem<Tin>::load8(xr[n] + c, x8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            ag[n] = fmaf(g8[j], x8[j], ag[n]);
            au[n] = fmaf(u8[j], x8[j], au[n]);
          }
        }
      }
    }
#pragma unroll
    for (int n = 0; n < GEMV_NT; ++n) {
      if (n < nv) {
        const float g = wave_sum(ag[n]);
        const float u = wave_sum(au[n]);
        if (lane == 0) {
          const float v = silu_f(g) * u;
          if (routed) act[((int64_t)sg.seg0 + tk + n) * I + i] = v;
          else act_s[((int64_t)tk + n) * ((int64_t)n_shared * Is) + (int64_t)sg.e * Is + i] = v;
        }
      }
    }
  }
}

// One launch for the down projections: grid.y rows below n_routed walk the
// routed segments (y_perm[pos][h] = W_d[e][h] . act[pos]); row n_routed is
// the shared experts, summed over the n_shared sub-matrices in order
// (y_s[t][h] = sum_s W_ds[s][h] . act_s[t][s * Is ..]).  One output row h
// per wave, GEMV_NT tokens per pass.
template <typename Tin>
__global__ void __launch_bounds__(GEMV_WAVES * MOE_WAVE)
gemv_down_kernel(const Tin* __restrict__ wd, const Tin* __restrict__ wsd, int H, int I, int Is,
                 int n_routed, int n_shared, int E, int T, const int32_t* __restrict__ offsets,
                 const float* __restrict__ act, const float* __restrict__ act_s,
                 float* __restrict__ y_perm, float* __restrict__ y_s) {
  const bool routed = (int)blockIdx.y < n_routed;
  SegInfo sg{0, 0, T};
  if (routed) sg = find_segment(E, offsets);   // block-uniform branch
  if (sg.e < 0) return;
  const int h = blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6);
  if (h >= H) return;
  const int lane = lane_id();
  const int K = routed ? I : Is, n_sub = routed ? 1 : n_shared;
  const int64_t ld = routed ? (int64_t)I : (int64_t)n_shared * Is;
  const Tin* wrow0 = routed ? wd + ((int64_t)sg.e * H + h) * I : wsd + (int64_t)h * Is;
  const float* a0 = routed ? act + (int64_t)sg.seg0 * ld : act_s;
  float* out = routed ? y_perm + (int64_t)sg.seg0 * H : y_s;
  for (int tk = 0; tk < sg.n; tk += GEMV_NT) {
    const int nv = min(GEMV_NT, sg.n - tk);
    float acc[GEMV_NT];
#pragma unroll
    for (int n = 0; n < GEMV_NT; ++n) acc[n] = 0.f;
    for (int sub = 0; sub < n_sub; ++sub) {
      const Tin* wrow = wrow0 + (int64_t)sub * H * Is;
      for (int c = lane * 8; c < K; c += 8 * MOE_WAVE) {
        float w8[8];
        elem<Tin>::load8(wrow + c, w8);
#pragma unroll
        for (int n = 0; n < GEMV_NT; ++n) {
          if (n < nv) {
            float a8[8];
            elem<float>::load8(a0 + (int64_t)(tk + n) * ld + (int64_t)sub * K + c, a8);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[n] = fmaf(w8[j], a8[j], acc[n]);
          }
        }
      }
    }
#pragma unroll
    for (int n = 0; n < GEMV_NT; ++n) {
      if (n < nv) {
        const float v = wave_sum(acc[n]);
        if (lane == 0) out[(int64_t)(tk + n) * H + h] = v;
      }
    }
  }
}

// Shared-expert scalar gate g_s = sigmoid(x . w_sg), one wave per token.
template <typename Tin>
__global__ void __launch_bounds__(64)
shared_gate_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wsg, int H, int use_gate,
                   float* __restrict__ g) {
  const int t = blockIdx.x, lane = threadIdx.x;
  if (!use_gate) {
    if (lane == 0) g[t] = 1.f;
    return;
  }
  float acc = 0.f;
  for (int c = lane * 8; c < H; c += 8 * MOE_WAVE) {
    float a8[8], b8[8];
    elem<Tin>::load8(x + (int64_t)t * H + c, a8);
    elem<Tin>::load8(wsg + c, b8);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(a8[j], b8[j], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) g[t] = sigmoid_f(acc);
}

template <typename Tin>
static hipError_t launch_dense_ffn_t(const moe_dims_t& d, int T, const Tin* x, const moe_weights_t& w,
                                     const int32_t* offsets, const int32_t* perm, int n_pairs_max,
                                     float* act, float* y_perm, float* act_s, float* y_s,
                                     const Prof& pf, hipStream_t s) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k;
  const int Is = d.shared_inter, ns = d.n_shared;
  const int n_routed = n_pairs_max < E ? n_pairs_max : E;
  if (n_routed + ns == 0) return hipSuccess;
  const int rows = I > Is ? I : Is;
  hipError_t e = pf.begin(MOE_KERNEL_EXPERT_GATE_UP, s);
  gemv_gate_up_kernel<Tin><<<dim3((rows + GEMV_WAVES - 1) / GEMV_WAVES, n_routed + ns),
                             GEMV_WAVES * MOE_WAVE, 0, s>>>(
      x, (const Tin*)w.w_gate, (const Tin*)w.w_up, (const Tin*)w.ws_gate, (const Tin*)w.ws_up, H, I,
      Is, n_routed, ns, E, k, T, offsets, perm, act, act_s);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_GATE_UP, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_EXPERT_DOWN, s);
  gemv_down_kernel<Tin><<<dim3((H + GEMV_WAVES - 1) / GEMV_WAVES, n_routed + (ns > 0 ? 1 : 0)),
                          GEMV_WAVES * MOE_WAVE, 0, s>>>(
      (const Tin*)w.w_down, (const Tin*)w.ws_down, H, I, Is, n_routed, ns, E, T, offsets, act, act_s,
      y_perm, y_s);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_DOWN, s);
  return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_shared_gate(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                              float* g_s, hipStream_t s) {
  if (d.n_shared == 0) return hipSuccess;
  if (d.dtype == MOE_BF16)
    shared_gate_kernel<bf16><<<T, 64, 0, s>>>((const bf16*)x, (const bf16*)w.w_shared_gate, d.hidden,
                                              d.shared_gate, g_s);
  else
    shared_gate_kernel<float><<<T, 64, 0, s>>>((const float*)x, (const float*)w.w_shared_gate,
                                               d.hidden, d.shared_gate, g_s);
  return hipGetLastError();
}

hipError_t launch_dense_ffn(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                            const int32_t* offsets, const int32_t* perm, int n_pairs_max,
                            float* act, float* y_perm, float* act_s, float* y_s, const Prof& pf,
                            hipStream_t s) {
  if (d.dtype == MOE_BF16)
    return launch_dense_ffn_t<bf16>(d, T, (const bf16*)x, w, offsets, perm, n_pairs_max, act, y_perm,
                                    act_s, y_s, pf, s);
  return launch_dense_ffn_t<float>(d, T, (const float*)x, w, offsets, perm, n_pairs_max, act, y_perm,
                                   act_s, y_s, pf, s);
}

}  // namespace moe
