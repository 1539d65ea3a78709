// Host side of the exact execution of missed experts [SPICE page, "CPU-GPU
// collaboration: handling prefetch misses"]: the per-expert cost rule that
// chooses between fetching a missed expert to the GPU and running it on the
// host, the host SwiGLU FFN on the weights already in host memory, and the
// kernel that puts the host rows into the GPU's expert-output rows.  The
// orchestration (copies, launches, the waits) is in api.hip.
//
// Host FFN.  Pairs are grouped by expert so that each weight row is read
// from host memory once per group and used for up to four tokens at a time
// from registers.  Work items are (group, block of 64 rows): first the gate/up
// rows (g = W_g x, u = W_u x, a = SiLU(g) u rounded to the layer dtype as the
// GPU kernels round it), then the down rows (y = W_d a).  Items are claimed
// in that order from one atomic counter; a down item waits, spinning, until
// every gate/up item of its group has finished, which cannot deadlock because
// all gate/up items have been claimed (and are running) before the first
// down item is.  Sums are fp32.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "common.h"

namespace moe {

// The host code below is compiled in the host pass only (the device pass
// has no x86 targets for its multiversioned dot products).
#ifndef __HIP_DEVICE_COMPILE__
// The two costs of one missed expert with `tokens` routed pairs: fetching,
// W_e / B + T_gpu, and running it on the host, T_cpu + 2 H / B per pair with
// T_cpu = cpu_expert_s + tokens * cpu_pair_s.
void offload_costs(double weight_bytes, double hidden_bytes, int tokens, double pcie_bytes_per_s,
                   double gpu_expert_s, double cpu_expert_s, double cpu_pair_s, double* fetch,
                   double* host) {
  *fetch = weight_bytes / pcie_bytes_per_s + gpu_expert_s;
  *host = cpu_expert_s + (double)tokens * cpu_pair_s +
          2.0 * (double)tokens * hidden_bytes / pcie_bytes_per_s;
}

namespace {

constexpr int HOST_ROWS = 64;  // weight rows per work item

inline float bf16_to_f(uint16_t b) {
  const uint32_t w = (uint32_t)b << 16;
  float f;
  memcpy(&f, &w, 4);
  return f;
}
// round to the nearest bf16, ties to even (finite values)
inline float round_bf16(float f) {
  uint32_t w;
  memcpy(&w, &f, 4);
  w = (w + 0x7FFFu + ((w >> 16) & 1u)) & 0xFFFF0000u;
  float r;
  memcpy(&r, &w, 4);
  return r;
}
inline float to_f(uint16_t v) { return bf16_to_f(v); }
inline float to_f(float v) { return v; }

// Dot products of one weight row with NT vectors x[0..NT): sixteen partial
// sums per vector (element i goes to sum i % 16), added in a fixed tree at
// the end, so a result does not depend on NT or on the thread that runs it
// (for one build of the row loop).  Converting a bf16 weight once for NT
// tokens and keeping 16 * NT independent sums in flight is what makes the
// row loop compute-bound rather than latency-bound.  n % 16 == 0
// (H % 64 == 0, I % 16 == 0).
template <int NT, typename Tw>
inline void dot_rows(const Tw* __restrict__ w, const float* const* x, int n, float* out) {
  float acc[NT][16];
  for (int t = 0; t < NT; ++t)
    for (int j = 0; j < 16; ++j) acc[t][j] = 0.f;
  for (int i = 0; i < n; i += 16) {
    float wf[16];
    for (int j = 0; j < 16; ++j) wf[j] = to_f(w[i + j]);
    for (int t = 0; t < NT; ++t)
      for (int j = 0; j < 16; ++j) acc[t][j] += wf[j] * x[t][i + j];
  }
  for (int t = 0; t < NT; ++t) {
    float r[8];
    for (int j = 0; j < 8; ++j) r[j] = acc[t][j] + acc[t][j + 8];
    out[t] = ((r[0] + r[4]) + (r[2] + r[6])) + ((r[1] + r[5]) + (r[3] + r[7]));
  }
}

// the row loops of every expert group, for each instruction set the host
// may have (x86-64-v4 = AVX-512, v3 = AVX2 + FMA), picked once at load time
#define HOST_CLONES __attribute__((target_clones("arch=x86-64-v4", "arch=x86-64-v3", "default")))

template <typename Tw>
inline void up_rows(const Tw* wg, const Tw* wu, int H, int I, int c0, int c1, const float* xf,
                    int q0, int q1, float* act, bool round) {
  for (int c = c0; c < c1; ++c) {
    const Tw* rg = wg + (int64_t)c * H;
    const Tw* ru = wu + (int64_t)c * H;
    int q = q0;
    for (; q + 4 <= q1; q += 4) {
      const float* xs[4] = {xf + (int64_t)q * H, xf + (int64_t)(q + 1) * H,
                            xf + (int64_t)(q + 2) * H, xf + (int64_t)(q + 3) * H};
      float g[4], u[4];
      dot_rows<4>(rg, xs, H, g);
      dot_rows<4>(ru, xs, H, u);
      for (int t = 0; t < 4; ++t) {
        const float av = g[t] / (1.f + expf(-g[t])) * u[t];
        act[(int64_t)(q + t) * I + c] = round ? round_bf16(av) : av;
      }
    }
    for (; q < q1; ++q) {
      const float* xs[1] = {xf + (int64_t)q * H};
      float g, u;
      dot_rows<1>(rg, xs, H, &g);
      dot_rows<1>(ru, xs, H, &u);
      const float av = g / (1.f + expf(-g)) * u;
      act[(int64_t)q * I + c] = round ? round_bf16(av) : av;
    }
  }
}

template <typename Tw>
inline void down_rows(const Tw* wd, int H, int I, int h0, int h1, const float* act, int q0,
                      int q1, float* y) {
  for (int h = h0; h < h1; ++h) {
    const Tw* rd = wd + (int64_t)h * I;
    int q = q0;
    for (; q + 4 <= q1; q += 4) {
      const float* as[4] = {act + (int64_t)q * I, act + (int64_t)(q + 1) * I,
                            act + (int64_t)(q + 2) * I, act + (int64_t)(q + 3) * I};
      float o[4];
      dot_rows<4>(rd, as, I, o);
      for (int t = 0; t < 4; ++t) y[(int64_t)(q + t) * H + h] = o[t];
    }
    for (; q < q1; ++q) {
      const float* as[1] = {act + (int64_t)q * I};
      dot_rows<1>(rd, as, I, y + (int64_t)q * H + h);
    }
  }
}

HOST_CLONES void up_rows_bf16(const uint16_t* wg, const uint16_t* wu, int H, int I, int c0,
                              int c1, const float* xf, int q0, int q1, float* act) {
  up_rows(wg, wu, H, I, c0, c1, xf, q0, q1, act, true);
}
HOST_CLONES void up_rows_f32(const float* wg, const float* wu, int H, int I, int c0, int c1,
                             const float* xf, int q0, int q1, float* act) {
  up_rows(wg, wu, H, I, c0, c1, xf, q0, q1, act, false);
}
HOST_CLONES void down_rows_bf16(const uint16_t* wd, int H, int I, int h0, int h1,
                                const float* act, int q0, int q1, float* y) {
  down_rows(wd, H, I, h0, h1, act, q0, q1, y);
}
HOST_CLONES void down_rows_f32(const float* wd, int H, int I, int h0, int h1, const float* act,
                               int q0, int q1, float* y) {
  down_rows(wd, H, I, h0, h1, act, q0, q1, y);
}
inline void up_any(const uint16_t* wg, const uint16_t* wu, int H, int I, int c0, int c1,
                   const float* xf, int q0, int q1, float* act) {
  up_rows_bf16(wg, wu, H, I, c0, c1, xf, q0, q1, act);
}
inline void up_any(const float* wg, const float* wu, int H, int I, int c0, int c1,
                   const float* xf, int q0, int q1, float* act) {
  up_rows_f32(wg, wu, H, I, c0, c1, xf, q0, q1, act);
}
inline void down_any(const uint16_t* wd, int H, int I, int h0, int h1, const float* act, int q0,
                     int q1, float* y) {
  down_rows_bf16(wd, H, I, h0, h1, act, q0, q1, y);
}
inline void down_any(const float* wd, int H, int I, int h0, int h1, const float* act, int q0,
                     int q1, float* y) {
  down_rows_f32(wd, H, I, h0, h1, act, q0, q1, y);
}

template <typename Tw>
void host_ffn_t(const HostFfnArgs& a, const Tw* x, const Tw* wg, const Tw* wu, const Tw* wd) {
  const int H = a.H, I = a.I;
  // fp32 token rows, in group order
  for (int q = 0; q < a.n_pairs; ++q)
    for (int h = 0; h < H; ++h) a.xf[(int64_t)q * H + h] = to_f(x[(int64_t)a.tok[q] * H + h]);
  const int ib = (I + HOST_ROWS - 1) / HOST_ROWS, hb = (H + HOST_ROWS - 1) / HOST_ROWS;
  const int n_up = a.n_groups * ib, n_items = n_up + a.n_groups * hb;
  for (int g = 0; g < a.n_groups; ++g) a.done[g] = 0;
  int next = 0;
  auto worker = [&]() {
    for (int it = __atomic_fetch_add(&next, 1, __ATOMIC_RELAXED); it < n_items;
         it = __atomic_fetch_add(&next, 1, __ATOMIC_RELAXED)) {
      if (it < n_up) {
        const int g = it / ib, c0 = (it % ib) * HOST_ROWS, c1 = std::min(I, c0 + HOST_ROWS);
        const int64_t e = a.gexp[g];
        up_any(wg + e * I * H, wu + e * I * H, H, I, c0, c1, a.xf, a.gstart[g], a.gstart[g + 1],
               a.act);
        __atomic_fetch_add(&a.done[g], 1, __ATOMIC_RELEASE);
      } else {
        const int j = it - n_up;
        const int g = j / hb, h0 = (j % hb) * HOST_ROWS, h1 = std::min(H, h0 + HOST_ROWS);
        while (__atomic_load_n(&a.done[g], __ATOMIC_ACQUIRE) < ib) std::this_thread::yield();
        const int64_t e = a.gexp[g];
        down_any(wd + e * H * I, H, I, h0, h1, a.act, a.gstart[g], a.gstart[g + 1], a.y);
      }
    }
  };
  const int nt = std::max(1, std::min(a.threads, n_items));
  std::vector<std::thread> pool;
  pool.reserve(nt - 1);
  for (int i = 1; i < nt; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

void host_expert_ffn(const HostFfnArgs& a, bool bf16_weights, const void* x, const void* wg,
                     const void* wu, const void* wd) {
  if (bf16_weights)
    host_ffn_t<uint16_t>(a, (const uint16_t*)x, (const uint16_t*)wg, (const uint16_t*)wu,
                         (const uint16_t*)wd);
  else
    host_ffn_t<float>(a, (const float*)x, (const float*)wg, (const float*)wu, (const float*)wd);
}
#endif  // __HIP_DEVICE_COMPILE__

// y_perm row of host pair i (pair index pairs[i]) <- y_host row i; the pair
// then counts as exactly computed, like the GPU's own rows.
__global__ void __launch_bounds__(256)
offload_scatter_kernel(int H, const int32_t* __restrict__ pairs, const float* __restrict__ y_host,
                       const int32_t* __restrict__ row_of, float* __restrict__ y_perm,
                       uint8_t* __restrict__ exact) {
  const int i = blockIdx.x;
  const int f = pairs[i];
  const int row = row_of[f];
  for (int h = threadIdx.x * 4; h < H; h += 256 * 4)
    *reinterpret_cast<float4*>(y_perm + (int64_t)row * H + h) =
        *reinterpret_cast<const float4*>(y_host + (int64_t)i * H + h);
  if (threadIdx.x == 0) exact[f] = 1;
}

hipError_t launch_offload_scatter(int n, int H, const int32_t* pairs, const float* y_host,
                                  const int32_t* row_of, float* y_perm, uint8_t* exact,
                                  hipStream_t s) {
  if (n > 0) offload_scatter_kernel<<<n, 256, 0, s>>>(H, pairs, y_host, row_of, y_perm, exact);
  return hipGetLastError();
}

}  // namespace moe
