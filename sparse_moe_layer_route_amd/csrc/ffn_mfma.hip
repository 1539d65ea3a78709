// bf16 expert SwiGLU FFN on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16)
// for decode and small batches: routed experts, shared experts and the LoRE
// surrogate's two skinny products in one launch per projection.
//
// Expert weights dominate the bytes, so each weight element is read once from
// HBM and every token of its segment is multiplied against it while it sits
// in registers.  Tokens form the MFMA's N dimension in tiles of 16 (up to NTT
// tiles per pass); a one-token segment wastes 15/16 of each MFMA, which the
// matrix cores absorb easily: one 16x16x32 MFMA consumes 1 KiB of weights in
// 16 cycles, about 20x a CU's share of HBM bandwidth.
//
// Fragments (lane l, 16x16x32): A row l%16 and B column l%16, each with 8
// consecutive k starting at 8*(l/16); the accumulator holds rows 4*(l/16)..+3
// of column l%16.  Every weight matrix keeps k contiguous (gate/up/LoRE-A
// [rows][H], down/LoRE-B [H][rows]), so a fragment is one 16-byte load.
//
// Tile kinds (blockIdx.x enumerates them in this order):
//   0 routed   up:   act = SiLU(W_g x) * (W_u x)      down: y = W_d act
//   1 shared   up:   same on the shared experts       down: y_s = sum_s W_sd act_s
//   2 LoRE     up:   z = A_e x  (r rows)              down: y = B_e z
// SPICE's surrogate for a non-resident slot is y_shared + B_e A_e x [SPICE
// page, "LoRE low-rank surrogate"]; the B_e A_e x part lands in the pair's
// y_perm row and the combine adds y_shared.
//
// The up epilogue stores its fp32 result as bf16 hi + lo (hi + lo carries
// ~16 significant bits) so the down kernel loads B fragments directly; with
// use_lo = 0 only hi is kept (large token counts, where the second MFMA would
// make the kernel compute-bound).
//
// Work split: a block of 4 waves owns 16*WM rows of one segment and WK = 4/WM
// k-splits: the waves deal the k loop round-robin and reduce through LDS,
// which keeps the dependent k chain of each wave short.  Each block picks,
// per chunk of tokens, the smallest instantiation covering its live token
// tiles, so a 6-token routed segment does not pay for a 64-token shared one.
#include <algorithm>

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t frag_load(const bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8_t frag_zero() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct FfnMfmaArgs {
  const bf16* x;                 // [T][H]
  const bf16* w0;                // up: gate [E][I][H]     down: w_down [E][H][I]
  const bf16* w1;                // up: up   [E][I][H]     down: unused
  const bf16* ws0;               // up: shared gate        down: shared down [ns][H][Is]
  const bf16* ws1;               // up: shared up          down: unused
  const bf16* wl;                // up: lore_A [E][r][H]   down: lore_B [E][H][r]
  const bf16 *act_hi, *act_lo;   // routed act [P][I]   (up writes, down reads)
  const bf16 *acts_hi, *acts_lo; // shared act [T][ns*Is]
  const bf16 *z_hi, *z_lo;       // LoRE z [T*k][r]
  bf16 *o_hi, *o_lo;             // up: routed act out
  bf16 *os_hi, *os_lo;           // up: shared act out
  bf16 *oz_hi, *oz_lo;           // up: LoRE z out
  float* y;                      // down: y_perm [T*k][H] (routed and LoRE rows)
  float* ys;                     // down: y_s [T][H]
  const int32_t* offsets;        // exact segments [E+1]
  const int32_t* moffsets;       // LoRE segments [E+1] (positions after the exact ones)
  const int32_t* perm;
  int H, I, Is, ns, r, E, k, T;
  int use_lo;
  int slots_r, tiles_r;          // routed slots x row tiles
  int n_shared_seg, tiles_s;     // shared segments (up: ns, down: 1) x row tiles
  int slots_l, tiles_l;          // LoRE slots x row tiles
};

struct TileInfo {
  int kind;   // 0 routed, 1 shared, 2 LoRE, -1 none
  int e;      // expert or shared index
  int seg0, n;
  int row0;   // first row of this block
};

// slot-th non-empty segment of `offs` (E+1 entries) -> (expert, start, count)
__device__ __forceinline__ void nth_segment(const int32_t* __restrict__ offs, int E, int slot,
                                            int* s_e, int* s_seg0, int* s_n) {
  if (threadIdx.x < MOE_WAVE) {
    const int lane = threadIdx.x;
    int o0 = 0, n = 0;
    if (lane < E) {
      o0 = offs[lane];
      n = offs[lane + 1] - o0;
    }
    const uint64_t bal = __ballot(n > 0);
    if (n > 0 && __popcll(bal & ((1ull << lane) - 1ull)) == slot) {
      *s_e = lane;
      *s_seg0 = o0;
      *s_n = n;
    }
    if (lane == 0 && __popcll(bal) <= slot) *s_e = -1;
  }
  __syncthreads();
}

template <int WM>
__device__ __forceinline__ TileInfo tile_of(const FfnMfmaArgs a) {
  __shared__ int s_e, s_seg0, s_n;
  TileInfo ti;
  int b = blockIdx.x;
  const int nr = a.slots_r * a.tiles_r;
  const int nsh = a.n_shared_seg * a.tiles_s;
  if (b < nr) {
    ti.kind = 0;
    ti.row0 = (b % a.tiles_r) * 16 * WM;
    nth_segment(a.offsets, a.E, b / a.tiles_r, &s_e, &s_seg0, &s_n);
  } else if (b < nr + nsh) {
    b -= nr;
    ti.kind = 1;
    ti.e = b / a.tiles_s;
    ti.row0 = (b % a.tiles_s) * 16 * WM;
    ti.seg0 = 0;
    ti.n = a.T;
    return ti;
  } else {
    b -= nr + nsh;
    ti.kind = 2;
    ti.row0 = (b % a.tiles_l) * 16 * WM;
    nth_segment(a.moffsets, a.E, b / a.tiles_l, &s_e, &s_seg0, &s_n);
  }
  if (s_e < 0) ti.kind = -1;
  ti.e = s_e;
  ti.seg0 = s_seg0;
  ti.n = s_n;
  return ti;
}

__device__ __forceinline__ void store_hi_lo(bf16* hi, bf16* lo, int64_t off, const float (&v)[4]) {
  uint16_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f_to_bf16(v[i]);
    l[i] = f_to_bf16(v[i] - bf16_to_f(h[i]));
  }
  *reinterpret_cast<uint2*>(hi + off) =
      make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  if (lo)
    *reinterpret_cast<uint2*>(lo + off) =
        make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

// k-steps loaded together before their MFMAs: enough independent 16-byte
// loads in flight per wave to cover HBM latency, bounded by registers.
template <int NA>
struct Unroll {
  static constexpr int U = NA <= 2 ? 4 : (NA <= 4 ? 2 : 1);
};

// ---------------------------------------------------------------- gate+up --
// One chunk of up to 16*NA tokens of a segment: k loop, LDS reduction over
// the WK k-splits, epilogue.
template <int NA, int NTT, int WM, int WK>
__device__ __forceinline__ void up_chunk(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                         const bf16* ag_row, const bf16* au_row, bool gated,
                                         bool rows_ok, int row_base,
                                         f32x4_t (*red)[(WK > 1) ? 2 * NTT : 1][MOE_WAVE]) {
  constexpr int U = Unroll<NA>::U;
  const int lane = lane_id(), wv = threadIdx.x >> 6, wk = wv / WM;
  const int r16 = lane & 15, kg = lane >> 4;
  const int H = a.H, ksteps = H >> 5;
  const bf16* xrow[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    int r = c0 + 16 * j + r16;
    if (r >= ti.n) r = c0;
    const int tok = ti.kind == 1 ? r : a.perm[ti.seg0 + r] / a.k;
    xrow[j] = a.x + (int64_t)tok * H + 8 * kg;
  }
  f32x4_t accg[NA], accu[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) accg[j] = accu[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (rows_ok) {
    for (int ks = wk; ks < ksteps; ks += U * WK) {
      bf16x8_t fg[U], fu[U], fx[U][NA];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = ks + u * WK;
        if (kk < ksteps) {
          const int ko = kk << 5;
          fg[u] = frag_load(ag_row + ko);
          fu[u] = gated ? frag_load(au_row + ko) : fg[u];
#pragma unroll
          for (int j = 0; j < NA; ++j) fx[u][j] = frag_load(xrow[j] + ko);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ks + u * WK < ksteps) {
#pragma unroll
          for (int j = 0; j < NA; ++j) {
            accg[j] = mfma16(fg[u], fx[u][j], accg[j]);
            if (gated) accu[j] = mfma16(fu[u], fx[u][j], accu[j]);
          }
        }
      }
    }
  }
  if (WK > 1) {
    if (wk > 0 && rows_ok) {
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        red[wk - 1][2 * j][lane] = accg[j];
        red[wk - 1][2 * j + 1][lane] = accu[j];
      }
    }
    __syncthreads();
    if (wk == 0 && rows_ok) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w)
#pragma unroll
        for (int j = 0; j < NA; ++j) {
          accg[j] += red[w][2 * j][lane];
          accu[j] += red[w][2 * j + 1][lane];
        }
    }
    __syncthreads();
  }
  if (wk == 0 && rows_ok) {
    const int i = row_base + 4 * kg;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int r = c0 + 16 * j + r16;
      if (r < ti.n) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = gated ? silu_f(accg[j][q]) * accu[j][q] : accg[j][q];
        if (ti.kind == 0)
          store_hi_lo(a.o_hi, a.o_lo, (int64_t)(ti.seg0 + r) * a.I + i, v);
        else if (ti.kind == 1)
          store_hi_lo(a.os_hi, a.os_lo, (int64_t)r * ((int64_t)a.ns * a.Is) + (int64_t)ti.e * a.Is + i, v);
        else
          store_hi_lo(a.oz_hi, a.oz_lo, (int64_t)(ti.seg0 + r) * a.r + i, v);
      }
    }
  }
}

template <int NTT, int WM, int WK>
__global__ void __launch_bounds__(256) ffn_up_mfma_kernel(FfnMfmaArgs a) {
  static_assert(WM * WK == 4, "four waves per block");
  __shared__ f32x4_t red[(WK > 1) ? (WK - 1) : 1][(WK > 1) ? 2 * NTT : 1][MOE_WAVE];
  const TileInfo ti = tile_of<WM>(a);
  if (ti.kind < 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int wm = wv % WM;
  const int H = a.H;
  const bool gated = ti.kind != 2;
  const int R = ti.kind == 0 ? a.I : (ti.kind == 1 ? a.Is : a.r);
  const int row_base = ti.row0 + 16 * wm;
  const bool rows_ok = row_base < R;  // wave-uniform
  const bf16 *wg, *wu;
  if (ti.kind == 0) {
    wg = a.w0 + (int64_t)ti.e * a.I * H;
    wu = a.w1 + (int64_t)ti.e * a.I * H;
  } else if (ti.kind == 1) {
    wg = a.ws0 + (int64_t)ti.e * a.Is * H;
    wu = a.ws1 + (int64_t)ti.e * a.Is * H;
  } else {
    wg = a.wl + (int64_t)ti.e * a.r * H;
    wu = wg;
  }
  const int r16 = lane & 15, kg = lane >> 4;
  const bf16* ag_row = wg + (int64_t)(row_base + r16) * H + 8 * kg;
  const bf16* au_row = wu + (int64_t)(row_base + r16) * H + 8 * kg;
  for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT) {
    const int nt = min(NTT, (ti.n - c0 + 15) >> 4);  // block-uniform
    if (nt <= 1) {
      up_chunk<1, NTT, WM, WK>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, red);
    } else if constexpr (NTT >= 2) {
      if (nt <= 2) {
        up_chunk<2, NTT, WM, WK>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, red);
      } else if constexpr (NTT >= 4) {
        if (nt <= 4) {
          up_chunk<4, NTT, WM, WK>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, red);
        } else if constexpr (NTT >= 8) {
          if (nt <= 8)
            up_chunk<8, NTT, WM, WK>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, red);
          else if constexpr (NTT >= 16)
            up_chunk<16, NTT, WM, WK>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, red);
        }
      }
    }
  }
}

// ------------------------------------------------------------------- down --
template <int NA, int NTT, int WM, int WK>
__device__ __forceinline__ void down_chunk(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                           bool rows_ok, int row_base,
                                           f32x4_t (*red)[(WK > 1) ? NTT : 1][MOE_WAVE]) {
  constexpr int U = Unroll<NA>::U;
  const int lane = lane_id(), wv = threadIdx.x >> 6, wk = wv / WM;
  const int r16 = lane & 15, kg = lane >> 4;
  const int H = a.H;
  const int K = ti.kind == 0 ? a.I : (ti.kind == 1 ? a.Is : a.r);
  const int nsub = ti.kind == 1 ? a.ns : 1;
  const int64_t ld = ti.kind == 0 ? a.I : (ti.kind == 1 ? (int64_t)a.ns * a.Is : a.r);
  const bf16* bhi = ti.kind == 0 ? a.act_hi : (ti.kind == 1 ? a.acts_hi : a.z_hi);
  const bf16* blo = ti.kind == 0 ? a.act_lo : (ti.kind == 1 ? a.acts_lo : a.z_lo);
  const bool two = a.use_lo != 0;
  const int kfull = K >> 5;  // full 32-wide steps; K % 8 == 0 may leave a partial one
  int64_t brow[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    int r = c0 + 16 * j + r16;
    if (r >= ti.n) r = c0;
    brow[j] = (int64_t)(ti.kind == 1 ? r : ti.seg0 + r) * ld + 8 * kg;
  }
  f32x4_t acc[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (rows_ok) {
    for (int s = 0; s < nsub; ++s) {
      const bf16* wrow;
      if (ti.kind == 0)
        wrow = a.w0 + ((int64_t)ti.e * H + row_base + r16) * a.I + 8 * kg;
      else if (ti.kind == 1)
        wrow = a.ws0 + ((int64_t)s * H + row_base + r16) * a.Is + 8 * kg;
      else
        wrow = a.wl + ((int64_t)ti.e * H + row_base + r16) * a.r + 8 * kg;
      const int64_t so = ti.kind == 1 ? (int64_t)s * a.Is : 0;
      for (int ks = wk; ks < kfull; ks += U * WK) {
        bf16x8_t fw[U], fh[U][NA], fl[U][NA];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kk = ks + u * WK;
          if (kk < kfull) {
            const int ko = kk << 5;
            fw[u] = frag_load(wrow + ko);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
              fh[u][j] = frag_load(bhi + brow[j] + so + ko);
              fl[u][j] = two ? frag_load(blo + brow[j] + so + ko) : frag_zero();
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ks + u * WK < kfull) {
#pragma unroll
            for (int j = 0; j < NA; ++j) {
              acc[j] = mfma16(fw[u], fh[u][j], acc[j]);
              if (two) acc[j] = mfma16(fw[u], fl[u][j], acc[j]);
            }
          }
        }
      }
      // partial last step (K % 32 != 0): lanes whose 8 k values lie past K
      // feed zeros to both operands
      if ((K & 31) && wk == kfull % WK) {
        const int ko = kfull << 5;
        const bool live = ko + 8 * kg < K;
        const bf16x8_t fw = live ? frag_load(wrow + ko) : frag_zero();
#pragma unroll
        for (int j = 0; j < NA; ++j) {
          acc[j] = mfma16(fw, live ? frag_load(bhi + brow[j] + so + ko) : frag_zero(), acc[j]);
          if (two) acc[j] = mfma16(fw, live ? frag_load(blo + brow[j] + so + ko) : frag_zero(), acc[j]);
        }
      }
    }
  }
  if (WK > 1) {
    if (wk > 0 && rows_ok) {
#pragma unroll
      for (int j = 0; j < NA; ++j) red[wk - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wk == 0 && rows_ok) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w)
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] += red[w][j][lane];
    }
    __syncthreads();
  }
  if (wk == 0 && rows_ok) {
    const int h = row_base + 4 * kg;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int r = c0 + 16 * j + r16;
      if (r < ti.n) {
        float* dst = ti.kind == 1 ? a.ys + (int64_t)r * H + h : a.y + (int64_t)(ti.seg0 + r) * H + h;
        *reinterpret_cast<float4*>(dst) = float4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      }
    }
  }
}

template <int NTT, int WM, int WK>
__global__ void __launch_bounds__(256) ffn_down_mfma_kernel(FfnMfmaArgs a) {
  static_assert(WM * WK == 4, "four waves per block");
  __shared__ f32x4_t red[(WK > 1) ? (WK - 1) : 1][(WK > 1) ? NTT : 1][MOE_WAVE];
  const TileInfo ti = tile_of<WM>(a);
  if (ti.kind < 0) return;
  const int wv = threadIdx.x >> 6;
  const int row_base = ti.row0 + 16 * (wv % WM);
  const bool rows_ok = row_base < a.H;
  for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT) {
    const int nt = min(NTT, (ti.n - c0 + 15) >> 4);  // block-uniform
    if (nt <= 1) {
      down_chunk<1, NTT, WM, WK>(a, ti, c0, rows_ok, row_base, red);
    } else if constexpr (NTT >= 2) {
      if (nt <= 2) {
        down_chunk<2, NTT, WM, WK>(a, ti, c0, rows_ok, row_base, red);
      } else if constexpr (NTT >= 4) {
        if (nt <= 4) {
          down_chunk<4, NTT, WM, WK>(a, ti, c0, rows_ok, row_base, red);
        } else if constexpr (NTT >= 8) {
          if (nt <= 8)
            down_chunk<8, NTT, WM, WK>(a, ti, c0, rows_ok, row_base, red);
          else if constexpr (NTT >= 16)
            down_chunk<16, NTT, WM, WK>(a, ti, c0, rows_ok, row_base, red);
        }
      }
    }
  }
}

template <int NTT, int WM, int WK>
static void launch_kernels(const FfnMfmaArgs& up, const FfnMfmaArgs& dn, int n_up, int n_dn,
                           hipStream_t s, int which) {
  if ((which & 1) && n_up > 0) ffn_up_mfma_kernel<NTT, WM, WK><<<n_up, 256, 0, s>>>(up);
  if ((which & 2) && n_dn > 0) ffn_down_mfma_kernel<NTT, WM, WK><<<n_dn, 256, 0, s>>>(dn);
}

// which: bit 0 = gate/up kernel, bit 1 = down kernel.  lore: LoRE tiles on.
hipError_t launch_ffn_mfma(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* moffsets, const int32_t* perm,
                           const FfnBuffers& b, int routed, int shared, int lore, hipStream_t s,
                           int which) {
  const int ntiles_tok = (T + 15) / 16;  // the largest segment has at most T tokens
  int NTT = 1;
  while (NTT < ntiles_tok && NTT < 16) NTT <<= 1;
  const int WM = NTT <= 4 ? 1 : (NTT == 8 ? 2 : 4);
  const int rows = 16 * WM;
  const int slots = std::min(d.n_experts, T * d.top_k);
  FfnMfmaArgs up{};
  up.x = (const bf16*)x;
  up.w0 = (const bf16*)w.w_gate;
  up.w1 = (const bf16*)w.w_up;
  up.ws0 = (const bf16*)w.ws_gate;
  up.ws1 = (const bf16*)w.ws_up;
  up.wl = (const bf16*)w.lore_A;
  up.o_hi = b.act_hi;
  up.o_lo = b.act_lo;
  up.os_hi = b.acts_hi;
  up.os_lo = b.acts_lo;
  up.oz_hi = b.z_hi;
  up.oz_lo = b.z_lo;
  up.act_hi = b.act_hi;
  up.act_lo = b.act_lo;
  up.acts_hi = b.acts_hi;
  up.acts_lo = b.acts_lo;
  up.z_hi = b.z_hi;
  up.z_lo = b.z_lo;
  up.y = b.y;
  up.ys = b.ys;
  up.offsets = offsets;
  up.moffsets = moffsets;
  up.perm = perm;
  up.H = d.hidden;
  up.I = d.inter;
  up.Is = d.shared_inter;
  up.ns = d.n_shared;
  up.r = d.lore_rank;
  up.E = d.n_experts;
  up.k = d.top_k;
  up.T = T;
  up.use_lo = b.act_lo != nullptr;
  up.slots_r = routed ? slots : 0;
  up.tiles_r = (d.inter + rows - 1) / rows;
  up.n_shared_seg = shared ? d.n_shared : 0;
  up.tiles_s = d.n_shared > 0 ? (d.shared_inter + rows - 1) / rows : 0;
  up.slots_l = lore ? slots : 0;
  up.tiles_l = lore ? (d.lore_rank + rows - 1) / rows : 0;
  FfnMfmaArgs dn = up;
  dn.w0 = (const bf16*)w.w_down;
  dn.w1 = nullptr;
  dn.ws0 = (const bf16*)w.ws_down;
  dn.ws1 = nullptr;
  dn.wl = (const bf16*)w.lore_B;
  dn.tiles_r = (d.hidden + rows - 1) / rows;
  dn.n_shared_seg = (shared && d.n_shared > 0) ? 1 : 0;
  dn.tiles_s = dn.tiles_r;
  dn.tiles_l = lore ? dn.tiles_r : 0;
  const int n_up = up.slots_r * up.tiles_r + up.n_shared_seg * up.tiles_s + up.slots_l * up.tiles_l;
  const int n_dn = dn.slots_r * dn.tiles_r + dn.n_shared_seg * dn.tiles_s + dn.slots_l * dn.tiles_l;
  switch (NTT) {
    case 1: launch_kernels<1, 1, 4>(up, dn, n_up, n_dn, s, which); break;
    case 2: launch_kernels<2, 1, 4>(up, dn, n_up, n_dn, s, which); break;
    case 4: launch_kernels<4, 1, 4>(up, dn, n_up, n_dn, s, which); break;
    case 8: launch_kernels<8, 2, 2>(up, dn, n_up, n_dn, s, which); break;
    default: launch_kernels<16, 4, 1>(up, dn, n_up, n_dn, s, which); break;
  }
  return hipGetLastError();
}

}  // namespace moe
