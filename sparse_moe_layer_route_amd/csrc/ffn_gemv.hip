// Expert SwiGLU FFN as a multi-token GEMV: y = (SiLU(x W_g) * (x W_u)) W_d
// [FloE page, Sec. 1, forward a^S(x) with S_t = identity].
//
// Every weight matrix is stored with the contraction index contiguous
// (gate/up [I][H], down [H][I]), so each output channel is one coalesced
// 16-byte-per-lane sweep of a weight row by a wave64, dotted with up to NT
// token rows at once, then a wave reduction.  A 256-thread block owns 16
// consecutive rows of one expert (4 per wave).  Grid.y walks the experts
// that received pairs: block y finds the y-th non-empty segment from the
// offsets with one ballot, so no host round trip is needed.  Shared experts
// use the same kernels with the identity token map.
#include "common.h"

namespace moe {

constexpr int GEMV_ROWS_PER_BLOCK = 16;
constexpr int GEMV_ROWS_PER_WAVE = 4;

struct SegInfo {
  int e;      // expert (routed) or shared-expert index
  int seg0;   // first pair position of the segment (routed) or 0
  int n;      // rows of the segment
};

// Routed: the blockIdx.y-th expert with a non-empty segment.  Shared: expert
// blockIdx.y over all T tokens.
__device__ __forceinline__ SegInfo find_segment(int routed, int E, int T,
                                                const int32_t* __restrict__ offsets) {
  __shared__ int s_e, s_seg0, s_n;
  if (!routed) return SegInfo{(int)blockIdx.y, 0, T};
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

// gate+up: act[row(p)][col0 + i] = SiLU(x_t . W_g[i]) * (x_t . W_u[i])
template <typename Tin, int NT>
__global__ void __launch_bounds__(256)
gate_up_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wg, const Tin* __restrict__ wu,
               int H, int I, int64_t e_stride, int routed, int E, int k, int T,
               const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
               float* __restrict__ act, int64_t act_ld) {
  const SegInfo sg = find_segment(routed, E, T, offsets);
  if (sg.e < 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const Tin* wg_e = wg + (int64_t)sg.e * e_stride;
  const Tin* wu_e = wu + (int64_t)sg.e * e_stride;
  const int64_t col0 = routed ? 0 : (int64_t)sg.e * I;
  const int r0 = blockIdx.x * GEMV_ROWS_PER_BLOCK + wv * GEMV_ROWS_PER_WAVE;
  for (int tk = 0; tk < sg.n; tk += NT) {
    const int nv = min(NT, sg.n - tk);
    const Tin* xr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int r = tk + (n < nv ? n : 0);
      const int tok = routed ? perm[sg.seg0 + r] / k : r;
      xr[n] = x + (int64_t)tok * H;
    }
    for (int q = 0; q < GEMV_ROWS_PER_WAVE; ++q) {
      const int i = r0 + q;
      const Tin* grow = wg_e + (int64_t)i * H;
      const Tin* urow = wu_e + (int64_t)i * H;
      float ag[NT], au[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) ag[n] = au[n] = 0.f;
      for (int c = lane * 8; c < H; c += 8 * MOE_WAVE) {
        float g8[8], u8[8];
        elem<Tin>::load8(grow + c, g8);
        elem<Tin>::load8(urow + c, u8);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
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
      for (int n = 0; n < NT; ++n) {
        if (n < nv) {
          const float g = wave_sum(ag[n]);
          const float u = wave_sum(au[n]);
          if (lane == 0) {
            const int64_t row = routed ? (int64_t)sg.seg0 + tk + n : (int64_t)tk + n;
            act[row * act_ld + col0 + i] = silu_f(g) * u;
          }
        }
      }
    }
  }
}

// down: out[row(p)][h] = sum over sub-matrices s of W_d[s][h][:] . act[row][s*K..]
// (routed: one sub-matrix per expert; shared: all n_sub shared experts summed).
template <typename Tin, int NT>
__global__ void __launch_bounds__(256)
down_kernel(const Tin* __restrict__ wd, int H, int K, int64_t e_stride, int n_sub,
            int64_t sub_stride, int routed, int E, int T, const int32_t* __restrict__ offsets,
            const float* __restrict__ act, int64_t act_ld, float* __restrict__ out) {
  const SegInfo sg = find_segment(routed, E, T, offsets);
  if (sg.e < 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const Tin* wd_e = wd + (routed ? (int64_t)sg.e * e_stride : 0);
  const int r0 = blockIdx.x * GEMV_ROWS_PER_BLOCK + wv * GEMV_ROWS_PER_WAVE;
  for (int tk = 0; tk < sg.n; tk += NT) {
    const int nv = min(NT, sg.n - tk);
    for (int q = 0; q < GEMV_ROWS_PER_WAVE; ++q) {
      const int h = r0 + q;
      float acc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = 0.f;
      for (int s = 0; s < n_sub; ++s) {
        const Tin* wrow = wd_e + (int64_t)s * sub_stride + (int64_t)h * K;
        for (int c = lane * 8; c < K; c += 8 * MOE_WAVE) {
          float w8[8];
          elem<Tin>::load8(wrow + c, w8);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            if (n < nv) {
              const int64_t row = (routed ? (int64_t)sg.seg0 : 0) + tk + n;
              float a8[8];
              elem<float>::load8(act + row * act_ld + (int64_t)s * K + c, a8);
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[n] = fmaf(w8[j], a8[j], acc[n]);
            }
          }
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < nv) {
          const float v = wave_sum(acc[n]);
          if (lane == 0) {
            const int64_t row = (routed ? (int64_t)sg.seg0 : 0) + tk + n;
            out[row * H + h] = v;
          }
        }
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
  constexpr int NT = 4;
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k;
  const int max_active = n_pairs_max < E ? n_pairs_max : E;
  hipError_t e = hipSuccess;
  if (max_active > 0) {
    dim3 g1(I / GEMV_ROWS_PER_BLOCK, max_active);
    e = pf.begin(MOE_KERNEL_EXPERT_GATE_UP, s);
    gate_up_kernel<Tin, NT><<<g1, 256, 0, s>>>(x, (const Tin*)w.w_gate, (const Tin*)w.w_up, H, I,
                                               (int64_t)I * H, 1, E, k, T, offsets, perm, act, I);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_GATE_UP, s);
    dim3 g2(H / GEMV_ROWS_PER_BLOCK, max_active);
    if (e == hipSuccess) e = pf.begin(MOE_KERNEL_EXPERT_DOWN, s);
    down_kernel<Tin, NT><<<g2, 256, 0, s>>>((const Tin*)w.w_down, H, I, (int64_t)H * I, 1, 0, 1, E,
                                            T, offsets, act, I, y_perm);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_DOWN, s);
  }
  if (e != hipSuccess) return e;
  if (d.n_shared > 0) {
    const int Is = d.shared_inter, ns = d.n_shared;
    dim3 g1(Is / GEMV_ROWS_PER_BLOCK, ns);
    gate_up_kernel<Tin, NT><<<g1, 256, 0, s>>>(x, (const Tin*)w.ws_gate, (const Tin*)w.ws_up, H, Is,
                                               (int64_t)Is * H, 0, E, k, T, offsets, perm, act_s,
                                               (int64_t)ns * Is);
    dim3 g2(H / GEMV_ROWS_PER_BLOCK, 1);
    down_kernel<Tin, NT><<<g2, 256, 0, s>>>((const Tin*)w.ws_down, H, Is, 0, ns, (int64_t)H * Is, 0,
                                            E, T, offsets, act_s, (int64_t)ns * Is, y_s);
  }
  return hipGetLastError();
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
