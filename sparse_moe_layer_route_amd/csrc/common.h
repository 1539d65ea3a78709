// Device helpers shared by the gfx950 kernels: bf16 packing, 16-byte vector
// loads, wave64 reductions and the workspace plan.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_route.h"

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------- bf16 ----
struct bf16 {
  uint16_t b;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
// fp32 -> bf16, round to nearest even (NaN stays NaN): one hardware
// conversion (v_cvt_pk_bf16_f32), two values per instruction when packed.
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t f2_to_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
}

__device__ __forceinline__ float half_bits_to_f(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}

// Element type traits: F32 = float storage, BF16 = bf16 storage.
template <typename T> struct elem;
template <> struct elem<float> {
  static constexpr int bytes = 4;
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
  // 8 consecutive elements starting at p (p 16-byte aligned)
  __device__ __forceinline__ static void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct elem<bf16> {
  static constexpr int bytes = 2;
  __device__ __forceinline__ static float load(const bf16* p, int64_t i) { return bf16_to_f(p[i].b); }
  __device__ __forceinline__ static void store(bf16* p, int64_t i, float v) { p[i].b = f_to_bf16(v); }
  __device__ __forceinline__ static void load8(const bf16* p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
};

// --------------------------------------------------------- wave64 ops -----
// Reductions and scans run on the DPP lane network rather than through LDS
// permutes (each of which is an LDS round trip): values move by 1, 2, 4 and
// 8 lanes within each row of 16, then the rows take the totals of the rows
// before them (lane 15 of each row broadcast into rows 1 and 3, lane 31 into
// rows 2 and 3), so lane l ends with the result over lanes 0..l.  Called by
// whole waves.  dpp_move: lanes with no source lane get 0 (BOUND_ZERO) or
// `old`; lanes of rows outside ROWS get `old`.
template <int CTRL, int ROWS = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ int dpp_move(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, BOUND_ZERO);
}
// Inclusive prefix sum of one int per lane.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  x += dpp_move<0x111>(0, x);             // row_shr:1 (no source: 0)
  x += dpp_move<0x112>(0, x);             // row_shr:2
  x += dpp_move<0x114>(0, x);             // row_shr:4
  x += dpp_move<0x118>(0, x);             // row_shr:8
  x += dpp_move<0x142, 0xa, false>(0, x); // row_bcast:15 into rows 1, 3
  x += dpp_move<0x143, 0xc, false>(0, x); // row_bcast:31 into rows 2, 3
  return x;
}
// Sum over the wave, in every lane (a fixed order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x111>(0, x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x112>(0, x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x114>(0, x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x118>(0, x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x142, 0xa, false>(0, x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp_move<0x143, 0xc, false>(0, x)));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}
// Maximum over the wave, in every lane (lanes with no source keep their own).
__device__ __forceinline__ float wave_max(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x111, 0xf, false>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x112, 0xf, false>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x114, 0xf, false>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x118, 0xf, false>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x142, 0xa, false>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_move<0x143, 0xc, false>(x, x))));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

// Monotone map of a float to uint32: a < b  <=>  key(a) < key(b) (no NaN).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// SiLU and sigmoid with the hardware reciprocal (1 ulp) instead of an IEEE
// division: a division expands to about ten instructions, which dominates the
// epilogue of the matrix-core kernels.  Large |z| still ends in 0 or z:
// rcp(inf) = 0 and rcp(1) = 1.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Activation buffers of the matrix-core FFN (bf16 hi + optional lo parts).
struct FfnBuffers {
  bf16* act;   // routed   [T*k][I]
  bf16* acts;  // shared   [T][n_shared*I_s]
  bf16* z;     // LoRE A x [T*k][r]
  float *y, *ys;  // y_perm [T*k][H], y_shared [T][H]
};

// Events recorded around one named kernel launch (see moe_kernel_t).
struct Prof {
  int id = MOE_KERNEL_NONE;
  hipEvent_t start = nullptr, stop = nullptr;
  hipError_t begin(int k, hipStream_t s) const {
    return (id == k && start) ? hipEventRecord(start, s) : hipSuccess;
  }
  hipError_t end(int k, hipStream_t s) const {
    return (id == k && stop) ? hipEventRecord(stop, s) : hipSuccess;
  }
};

// Where the router's top-k launch writes the permutation when it also sorts
// the (token, slot) pairs; counter is a workspace word the logits launch
// zeroes and the top-k blocks count themselves in.
struct PermOut {
  int32_t* counter;
  int32_t *offsets, *perm, *inv, *row_of, *miss_offsets;
};

// Weighted combine fused into the last FloE launch: out [T][H] in the layer
// dtype, from the slot -> row map, the slot weights and exact flags, and the
// shared experts' output and gate (y_s / g_s may be null).
struct FloeCombine {
  const int32_t* row_of;
  const float* topk_w;
  const uint8_t* exact;
  const float* y_s;
  const float* g_s;
  void* out;
};

// Host FFN of the pairs run on the host (host memory throughout): n_groups
// experts gexp[g], whose pairs are q in [gstart[g], gstart[g+1]) with token
// tok[q]; xf [n_pairs][H] and act [n_pairs][I] are scratch, y [n_pairs][H]
// the fp32 expert outputs; done [n_groups] are work counters.
struct HostFfnArgs {
  int H, I, n_pairs, n_groups, threads;
  const int32_t *tok, *gexp, *gstart;
  int32_t* done;
  float *xf, *act, *y;
};

}  // namespace moe
