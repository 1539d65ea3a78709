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
// Tile kinds, in the order blockIdx.x enumerates them:
//   1 shared   up:   act_s = SiLU(W_sg x) * (W_su x)   down: y_s = sum_s W_sd act_s
//   2 LoRE     up:   z = A_e x  (r rows)               down: y = B_e z (128-row tiles)
//   0 routed   up:   act = SiLU(W_g x) * (W_u x)       down: y = W_d act
// Shared tiles carry every token of the batch and LoRE tiles are short
// latency-bound chains, so both start before the routed bulk instead of
// running as a tail.  SPICE's surrogate for a non-resident slot is
// y_shared + B_e A_e x [SPICE page, "LoRE low-rank surrogate"]; the B_e A_e x
// part lands in the pair's y_perm row and the combine adds y_shared.
//
// The up epilogue rounds SiLU(g) * u to bf16 (the layer's dtype), which the
// down kernel reads as MFMA fragments; every sum accumulates in fp32.
//
// Work split: a block of 4 waves owns WM row strips of one segment and splits
// K over WK = 4/WM waves that reduce through LDS.  Each wave walks a
// contiguous range of k-steps, so its loads cover whole 128-byte lines of its
// rows, and the loop is software-pipelined: batch b+1 (U k-steps) is loading
// while the MFMAs of batch b run.  In the down kernel a wave's strip is RW
// row tiles, which reuses each activation fragment RW times.  Each block
// picks, per chunk of tokens, the smallest instantiation covering its live
// token tiles, so a 6-token routed segment does not pay for a 64-token shared
// one.
#include <algorithm>

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t frag_load(const bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#ifndef FFN_NT_WEIGHTS
#define FFN_NT_WEIGHTS 1
#endif
// Weight fragments are read once per launch, so their loads are marked
// non-temporal: streamed without displacing the token rows and activations
// that the blocks of a segment share in L2.  Measured on every decode row
// (fragment-major weights, cold caches): 5-10% off the step, e.g. the
// one-token Qwen2-57B-shaped step 177 -> 159 us and the 8-token
// DeepSeek-V2-Lite-shaped one 126 -> 113 us.  FFN_NT_WEIGHTS = 0 restores
// ordinary loads.
__device__ __forceinline__ bf16x8_t wfrag_load(const bf16* p) {
#if FFN_NT_WEIGHTS
  return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
#else
  return frag_load(p);
#endif
}
__device__ __forceinline__ bf16x8_t frag_zero() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct FfnMfmaArgs {
  const bf16* x;          // [T][H]
  const bf16* w0;         // up: gate [E][I][H]     down: w_down [E][H][I]
  const bf16* w1;         // up: up   [E][I][H]     down: unused
  const bf16* ws0;        // up: shared gate        down: shared down [ns][H][Is]
  const bf16* ws1;        // up: shared up          down: unused
  const bf16* wl;         // up: lore_A [E][r][H]   down: lore_B [E][H][r]
  bf16* act;              // routed act [P][I]      (up writes, down reads)
  bf16* acts;             // shared act [T][ns*Is]
  bf16* z;                // LoRE z [T*k][r]
  float* y;               // down: y_perm [T*k][H] (routed and LoRE rows)
  float* ys;              // down: y_s [T][H]
  const int32_t* offsets;   // exact segments [E+1]
  const int32_t* moffsets;  // LoRE segments [E+1] (positions after the exact ones)
  const int32_t* perm;
  int H, I, Is, ns, r, E, k, T;
  int packed;             // routed and shared matrices fragment-major (LoRE row-major)
  int slots_r, tiles_r;       // routed slots x row tiles
  int n_shared_seg, tiles_s;  // shared segments (up: ns, down: 1) x row tiles
  int slots_l, tiles_l;       // LoRE slots x row tiles
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

// ROWS = rows a block covers (ROWS_L for LoRE tiles).
template <int ROWS, int ROWS_L = ROWS>
__device__ __forceinline__ TileInfo tile_of(const FfnMfmaArgs a) {
  __shared__ int s_e, s_seg0, s_n;
  TileInfo ti;
  int b = blockIdx.x;
  const int nsh = a.n_shared_seg * a.tiles_s;
  if (b < nsh) {
    ti.kind = 1;
    ti.e = b / a.tiles_s;
    ti.row0 = (b % a.tiles_s) * ROWS;
    ti.seg0 = 0;
    ti.n = a.T;
    return ti;
  }
  b -= nsh;
  const int nl = a.slots_l * a.tiles_l;
  if (b < nl) {
    ti.kind = 2;
    ti.row0 = (b % a.tiles_l) * ROWS_L;
    nth_segment(a.moffsets, a.E, b / a.tiles_l, &s_e, &s_seg0, &s_n);
  } else {
    b -= nl;
    ti.kind = 0;
    ti.row0 = (b % a.tiles_r) * ROWS;
    nth_segment(a.offsets, a.E, b / a.tiles_r, &s_e, &s_seg0, &s_n);
  }
  if (s_e < 0) ti.kind = -1;
  ti.e = s_e;
  ti.seg0 = s_seg0;
  ti.n = s_n;
  return ti;
}

__device__ __forceinline__ void store_bf16x4(bf16* dst, int64_t off, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(dst + off) =
      make_uint2(f2_to_bf16x2(v[0], v[1]), f2_to_bf16x2(v[2], v[3]));
}

// k-steps per batch of the pipelined loop: two register sets of U steps each.
#ifndef FFN_UNROLL_SMALL
#define FFN_UNROLL_SMALL 2
#endif
#ifndef FFN_UNROLL_MID
#define FFN_UNROLL_MID 1
#endif
// Gate/up with two row tiles per wave (long segments): one step per set up
// to two token tiles, whose registers the wide rows already fill.
#ifndef FFN_UNROLL_WIDE_UP
#define FFN_UNROLL_WIDE_UP 1
#endif
template <int NA>
struct Unroll {
  static constexpr int U = NA <= 2 ? FFN_UNROLL_SMALL : (NA == 4 ? FFN_UNROLL_MID : 1);
};
template <int NA, int RW>
struct UpUnroll {
  static constexpr int U = (RW > 1 && NA <= 2) ? FFN_UNROLL_WIDE_UP : Unroll<NA>::U;
};

// Wave wk's contiguous share [beg, end) of nsteps k-steps, in nb batches of U.
struct KRange {
  int beg, end, nb;
};

template <int U>
__device__ __forceinline__ KRange k_range(int nsteps, int wk, int WK) {
  const int per = (nsteps + WK - 1) / WK;
  KRange r;
  r.beg = wk * per;
  r.end = min(nsteps, r.beg + per);
  r.nb = r.end > r.beg ? (r.end - r.beg + U - 1) / U : 0;
  return r;
}

// Up to 4 token tiles the kernels are held to >= 3 waves per SIMD (at most
// 168 registers per lane), which keeps enough weight loads in flight per CU;
// the wide-row forms for long segments (gate/up with 2 row tiles per wave,
// down with 4) take 2 waves per SIMD and the registers they need.
#define FFN_UP_OCCUPANCY __attribute__((amdgpu_waves_per_eu(NTT <= 4 ? (RW > 1 ? 2 : 3) : 1)))
#define FFN_DOWN_OCCUPANCY __attribute__((amdgpu_waves_per_eu(NTT <= 4 ? (RW > 2 ? 2 : 3) : 1)))

// ---------------------------------------------------------------- gate+up --
// One chunk of up to 16*NA tokens of a segment: pipelined k loop, LDS
// reduction over the WK k-splits, epilogue.  A wave owns RW row tiles of
// gate and up, so each token fragment feeds 2*RW MFMAs.  Steps past a wave's
// range in its last batch load an in-range address and feed a zero token
// fragment.
template <int NA, int NTT, int WM, int WK, int RW>
__device__ __forceinline__ void up_chunk(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                         const bf16* const (&ag_row)[RW],
                                         const bf16* const (&au_row)[RW], bool gated,
                                         bool rows_ok, int row_base, int R,
                                         f32x4_t (*red)[(WK > 1) ? 2 * NTT * RW : 1][MOE_WAVE]) {
  constexpr int U = UpUnroll<NA, RW>::U;
  const int lane = lane_id(), wv = threadIdx.x >> 6, wk = wv / WM, wm = wv % WM;
  const int r16 = lane & 15, kg = lane >> 4;
  const int H = a.H, ksteps = H >> 5;
  // k-step stride of the weight pointers: 32 elements row-major, one 1 KiB
  // fragment (512 elements) fragment-major
  const int wsh = (a.packed && ti.kind != 2) ? 4 : 0;
  const bf16* xrow[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    int r = c0 + 16 * j + r16;
    if (r >= ti.n) r = c0;
    const int tok = ti.kind == 1 ? r : a.perm[ti.seg0 + r] / a.k;
    xrow[j] = a.x + (int64_t)tok * H + 8 * kg;
  }
  f32x4_t accg[NA][RW], accu[NA][RW];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int q = 0; q < RW; ++q) accg[j][q] = accu[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const KRange kr = k_range<U>(ksteps, wk, WK);
  if (rows_ok && kr.nb > 0) {
    bf16x8_t g0[U][RW], u0[U][RW], x0[U][NA], g1[U][RW], u1[U][RW], x1[U][NA];
#define UP_LOAD(G, UU, X, b)                                                   \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                              \
    const int ko = min(kr.beg + (b) * U + u, kr.end - 1) << 5;                 \
    _Pragma("unroll") for (int q = 0; q < RW; ++q) {                           \
      G[u][q] = wfrag_load(ag_row[q] + (ko << wsh));                           \
      UU[u][q] = wfrag_load(au_row[q] + (ko << wsh));                          \
    }                                                                          \
    _Pragma("unroll") for (int j = 0; j < NA; ++j) X[u][j] = frag_load(xrow[j] + ko); \
  }
#define UP_MFMA(G, UU, X, b)                                                   \
  _Pragma("unroll") for (int u = 0; u < U; ++u)                                \
    _Pragma("unroll") for (int j = 0; j < NA; ++j) {                           \
      const bool live = kr.beg + (b) * U + u < kr.end;                         \
      const bf16x8_t xv = live ? X[u][j] : frag_zero();                        \
      _Pragma("unroll") for (int q = 0; q < RW; ++q) {                         \
        accg[j][q] = mfma16(G[u][q], xv, accg[j][q]);                          \
        accu[j][q] = mfma16(UU[u][q], xv, accu[j][q]);                         \
      }                                                                        \
    }
    UP_LOAD(g0, u0, x0, 0);
    for (int bb = 0; bb < kr.nb; bb += 2) {
      if (bb + 1 < kr.nb) { UP_LOAD(g1, u1, x1, bb + 1); }
      UP_MFMA(g0, u0, x0, bb);
      if (bb + 2 < kr.nb) { UP_LOAD(g0, u0, x0, bb + 2); }
      if (bb + 1 < kr.nb) { UP_MFMA(g1, u1, x1, bb + 1); }
    }
#undef UP_LOAD
#undef UP_MFMA
  }
  if (WK > 1) {
    if (wk > 0 && rows_ok) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int q = 0; q < RW; ++q) {
          red[(wk - 1) * WM + wm][2 * (j * RW + q)][lane] = accg[j][q];
          red[(wk - 1) * WM + wm][2 * (j * RW + q) + 1][lane] = accu[j][q];
        }
    }
    __syncthreads();
    if (wk == 0 && rows_ok) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w)
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
          for (int q = 0; q < RW; ++q) {
            accg[j][q] += red[w * WM + wm][2 * (j * RW + q)][lane];
            accu[j][q] += red[w * WM + wm][2 * (j * RW + q) + 1][lane];
          }
    }
    __syncthreads();
  }
  if (wk == 0 && rows_ok) {
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int i = row_base + 16 * q + 4 * kg;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const int r = c0 + 16 * j + r16;
        if (r < ti.n && i < R) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gated ? silu_f(accg[j][q][e]) * accu[j][q][e] : accg[j][q][e];
          if (ti.kind == 0)
            store_bf16x4(a.act, (int64_t)(ti.seg0 + r) * a.I + i, v);
          else if (ti.kind == 1)
            store_bf16x4(a.acts, (int64_t)r * ((int64_t)a.ns * a.Is) + (int64_t)ti.e * a.Is + i, v);
          else
            store_bf16x4(a.z, (int64_t)(ti.seg0 + r) * a.r + i, v);
        }
      }
    }
  }
}

// The smallest instantiation covering the live token tiles of chunk c0.
template <int NTT, int WM, int WK, int RW>
__device__ __forceinline__ void up_dispatch(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                            const bf16* const (&ag_row)[RW],
                                            const bf16* const (&au_row)[RW], bool gated,
                                            bool rows_ok, int row_base, int R,
                                            f32x4_t (*red)[(WK > 1) ? 2 * NTT * RW : 1][MOE_WAVE]) {
  const int nt = min(NTT, (ti.n - c0 + 15) >> 4);  // block-uniform
  if (nt <= 1) {
    up_chunk<1, NTT, WM, WK, RW>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, R, red);
  } else if constexpr (NTT >= 2) {
    if (nt <= 2) {
      up_chunk<2, NTT, WM, WK, RW>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, R, red);
    } else if constexpr (NTT >= 4) {
      if (nt <= 4) {
        up_chunk<4, NTT, WM, WK, RW>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, R, red);
      } else if constexpr (NTT >= 8) {
        if (nt <= 8)
          up_chunk<8, NTT, WM, WK, RW>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, R, red);
        else if constexpr (NTT >= 16)
          up_chunk<16, NTT, WM, WK, RW>(a, ti, c0, ag_row, au_row, gated, rows_ok, row_base, R, red);
      }
    }
  }
}

// RW: row tiles per wave for routed and shared tiles (LoRE tiles, with only
// r rows, keep one).
template <int NTT, int WM, int WK, int RW>
__global__ void __launch_bounds__(256) FFN_UP_OCCUPANCY ffn_up_mfma_kernel(FfnMfmaArgs a) {
  static_assert(WM * WK == 4, "four waves per block");
  // k-split partials, one slot per (k-split > 0, row strip)
  __shared__ f32x4_t red[(WK > 1) ? (WK - 1) * WM : 1][(WK > 1) ? 2 * NTT * RW : 1][MOE_WAVE];
  const TileInfo ti = tile_of<16 * WM * RW, 16 * WM>(a);
  if (ti.kind < 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int wm = wv % WM;
  const int H = a.H;
  const bool gated = ti.kind != 2;
  const int R = ti.kind == 0 ? a.I : (ti.kind == 1 ? a.Is : a.r);
  const bf16 *wg, *wu;
  if (ti.kind == 0) {
    wg = a.w0 + (int64_t)ti.e * a.I * H;
    wu = a.w1 + (int64_t)ti.e * a.I * H;
  } else if (ti.kind == 1) {
    wg = a.ws0 + (int64_t)ti.e * a.Is * H;
    wu = a.ws1 + (int64_t)ti.e * a.Is * H;
  } else {
    wg = a.wl + (int64_t)ti.e * a.r * H;
    wu = wg;  // LoRE A: one matrix; the second product is computed and unused
  }
  const int r16 = lane & 15, kg = lane >> 4;
  // a 16-row tile can overhang R (a LoRE rank that is a multiple of 8 only):
  // overhanging lanes reread row R-1 and their outputs are not stored
  if (ti.kind == 2) {
    const int row_base = ti.row0 + 16 * wm;
    const bool rows_ok = row_base < R;  // wave-uniform
    const int wrow_i = min(row_base + r16, R - 1);
    const bf16* const ag[1] = {wg + (int64_t)wrow_i * H + 8 * kg};
    for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT)
      up_dispatch<NTT, WM, WK, 1>(a, ti, c0, ag, ag, gated, rows_ok, row_base, R,
                                  reinterpret_cast<f32x4_t(*)[(WK > 1) ? 2 * NTT : 1][MOE_WAVE]>(red));
    return;
  }
  const int row_base = ti.row0 + 16 * RW * wm;
  const bool rows_ok = row_base < R;  // wave-uniform
  const bf16* ag[RW];
  const bf16* au[RW];
#pragma unroll
  for (int q = 0; q < RW; ++q) {
    if (a.packed) {  // fragment (row tile, k step 0); R % 16 == 0, tiles past R reread the last
      const int64_t f = (int64_t)min((row_base >> 4) + q, (R >> 4) - 1) * (H >> 5) * 512 + lane * 8;
      ag[q] = wg + f;
      au[q] = wu + f;
    } else {
      const int wrow_i = min(row_base + 16 * q + r16, R - 1);
      ag[q] = wg + (int64_t)wrow_i * H + 8 * kg;
      au[q] = wu + (int64_t)wrow_i * H + 8 * kg;
    }
  }
  for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT)
    up_dispatch<NTT, WM, WK, RW>(a, ti, c0, ag, au, gated, rows_ok, row_base, R, red);
}

// ------------------------------------------------------------------- down --
// Output rows are H for every kind; K is I (routed), Is per shared expert
// (summed over the ns sub-matrices), or r (LoRE).  A wave owns RW row tiles.
// solo (block-uniform): the wave covers the whole contraction itself and no
// k-split reduction takes place (LoRE B_e tiles, where K = r is short).
template <int NA, int NTT, int WM, int WK, int RW>
__device__ __forceinline__ void down_chunk(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                           bool rows_ok, int row_base,
                                           f32x4_t (*red)[(WK > 1) ? NTT * RW : 1][MOE_WAVE],
                                           bool solo) {
  constexpr int U = Unroll<NA>::U;
  const int lane = lane_id(), wv = threadIdx.x >> 6, wm = wv % WM;
  const int wk = solo ? 0 : wv / WM, nwk = solo ? 1 : WK;
  const int r16 = lane & 15, kg = lane >> 4;
  const int H = a.H;
  const int K = ti.kind == 0 ? a.I : (ti.kind == 1 ? a.Is : a.r);
  const int nsub = ti.kind == 1 ? a.ns : 1;
  const int64_t ld = ti.kind == 0 ? a.I : (ti.kind == 1 ? (int64_t)a.ns * a.Is : a.r);
  const bf16* bsrc = ti.kind == 0 ? a.act : (ti.kind == 1 ? a.acts : a.z);
  const int kfull = K >> 5;  // full 32-wide steps; K % 8 == 0 may leave a partial one
  const int wsh = (a.packed && ti.kind != 2) ? 4 : 0;  // weight k-step stride, as in up_chunk
  int64_t brow[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    int r = c0 + 16 * j + r16;
    if (r >= ti.n) r = c0;
    brow[j] = (int64_t)(ti.kind == 1 ? r : ti.seg0 + r) * ld + 8 * kg;
  }
  f32x4_t acc[NA][RW];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int q = 0; q < RW; ++q) acc[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (rows_ok) {
    for (int s = 0; s < nsub; ++s) {
      const bf16* wrow[RW];
#pragma unroll
      for (int q = 0; q < RW; ++q) {
        const int h = min(row_base + 16 * q + r16, H - 1);
        if (wsh) {  // fragment-major [H/16][ceil(K/32)][64][8] per matrix
          const int ks = (K + 31) >> 5;
          const int64_t f = (int64_t)min((row_base >> 4) + q, (H >> 4) - 1) * ks * 512 + lane * 8;
          wrow[q] = (ti.kind == 0 ? a.w0 + (int64_t)ti.e * H * (ks << 5)
                                  : a.ws0 + (int64_t)s * H * (ks << 5)) + f;
        } else if (ti.kind == 0) {
          wrow[q] = a.w0 + ((int64_t)ti.e * H + h) * a.I + 8 * kg;
        } else if (ti.kind == 1) {
          wrow[q] = a.ws0 + ((int64_t)s * H + h) * a.Is + 8 * kg;
        } else {
          wrow[q] = a.wl + ((int64_t)ti.e * H + h) * a.r + 8 * kg;
        }
      }
      const int64_t so = ti.kind == 1 ? (int64_t)s * a.Is : 0;
      const KRange kr = k_range<U>(kfull, wk, nwk);
      if (kr.nb > 0) {
        bf16x8_t w0[U][RW], b0[U][NA], w1[U][RW], b1[U][NA];
#define DN_LOAD(W, B, b)                                                       \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                              \
    const int ko = min(kr.beg + (b) * U + u, kr.end - 1) << 5;                 \
    _Pragma("unroll") for (int q = 0; q < RW; ++q) W[u][q] = wfrag_load(wrow[q] + (ko << wsh)); \
    _Pragma("unroll") for (int j = 0; j < NA; ++j) B[u][j] = frag_load(bsrc + brow[j] + so + ko); \
  }
#define DN_MFMA(W, B, b)                                                       \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                              \
    const bool live = kr.beg + (b) * U + u < kr.end;                           \
    _Pragma("unroll") for (int j = 0; j < NA; ++j) {                           \
      const bf16x8_t bv = live ? B[u][j] : frag_zero();                        \
      _Pragma("unroll") for (int q = 0; q < RW; ++q) acc[j][q] = mfma16(W[u][q], bv, acc[j][q]); \
    }                                                                          \
  }
        DN_LOAD(w0, b0, 0);
        for (int bb = 0; bb < kr.nb; bb += 2) {
          if (bb + 1 < kr.nb) { DN_LOAD(w1, b1, bb + 1); }
          DN_MFMA(w0, b0, bb);
          if (bb + 2 < kr.nb) { DN_LOAD(w0, b0, bb + 2); }
          if (bb + 1 < kr.nb) { DN_MFMA(w1, b1, bb + 1); }
        }
#undef DN_LOAD
#undef DN_MFMA
      }
      // partial last step (K % 32 != 0): lanes whose 8 k values lie past K
      // feed zeros to both operands
      if ((K & 31) && wk == nwk - 1) {
        const int ko = kfull << 5;
        const bool live = ko + 8 * kg < K;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
          const bf16x8_t bv = live ? frag_load(bsrc + brow[j] + so + ko) : frag_zero();
#pragma unroll
          for (int q = 0; q < RW; ++q)
            acc[j][q] = mfma16(live ? frag_load(wrow[q] + (ko << wsh)) : frag_zero(), bv, acc[j][q]);
        }
      }
    }
  }
  if (WK > 1 && !solo) {
    if (wk > 0 && rows_ok) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int q = 0; q < RW; ++q) red[(wk - 1) * WM + wm][j * RW + q][lane] = acc[j][q];
    }
    __syncthreads();
    if (wk == 0 && rows_ok) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w)
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
          for (int q = 0; q < RW; ++q) acc[j][q] += red[w * WM + wm][j * RW + q][lane];
    }
    __syncthreads();
  }
  if (wk == 0 && rows_ok) {
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int h = row_base + 16 * q + 4 * kg;
      if (h >= H) continue;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const int r = c0 + 16 * j + r16;
        if (r < ti.n) {
          float* dst = ti.kind == 1 ? a.ys + (int64_t)r * H + h : a.y + (int64_t)(ti.seg0 + r) * H + h;
          *reinterpret_cast<float4*>(dst) = float4{acc[j][q][0], acc[j][q][1], acc[j][q][2], acc[j][q][3]};
        }
      }
    }
  }
}

// Rows of one LoRE down tile: one row strip of RW row tiles per wave.  K = r
// is one short step, so a LoRE tile is mostly fixed cost; at H = 2048 and
// two row tiles per wave this gives 16 blocks per missed expert.
template <int RW>
struct LoreDownRows {
  static constexpr int ROWS = 16 * RW * 4;
};

// The smallest instantiation covering the live token tiles of chunk c0.
template <int NTT, int WM, int WK, int RW>
__device__ __forceinline__ void down_dispatch(const FfnMfmaArgs a, const TileInfo& ti, int c0,
                                              bool rows_ok, int row_base,
                                              f32x4_t (*red)[(WK > 1) ? NTT * RW : 1][MOE_WAVE],
                                              bool solo) {
  const int nt = min(NTT, (ti.n - c0 + 15) >> 4);  // block-uniform
  if (nt <= 1) {
    down_chunk<1, NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, solo);
  } else if constexpr (NTT >= 2) {
    if (nt <= 2) {
      down_chunk<2, NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, solo);
    } else if constexpr (NTT >= 4) {
      if (nt <= 4) {
        down_chunk<4, NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, solo);
      } else if constexpr (NTT >= 8) {
        if (nt <= 8)
          down_chunk<8, NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, solo);
        else if constexpr (NTT >= 16)
          down_chunk<16, NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, solo);
      }
    }
  }
}

template <int NTT, int WM, int WK, int RW>
__global__ void __launch_bounds__(256) FFN_DOWN_OCCUPANCY ffn_down_mfma_kernel(FfnMfmaArgs a) {
  static_assert(WM * WK == 4, "four waves per block");
  // k-split partials, one slot per (k-split > 0, row strip)
  __shared__ f32x4_t red[(WK > 1) ? (WK - 1) * WM : 1][(WK > 1) ? NTT * RW : 1][MOE_WAVE];
  const TileInfo ti = tile_of<16 * RW * WM, LoreDownRows<RW>::ROWS>(a);
  if (ti.kind < 0) return;
  const int wv = threadIdx.x >> 6;
  if (ti.kind == 2) {
    // LoRE B_e: a block covers LoreDownRows rows; each wave takes whole row
    // strips with the full (short) contraction
    const int r_end = min(a.H, ti.row0 + LoreDownRows<RW>::ROWS);
    for (int rb = ti.row0 + 16 * RW * wv; rb < r_end; rb += 16 * RW * 4)
      for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT) down_dispatch<NTT, WM, WK, RW>(a, ti, c0, true, rb, red, true);
    return;
  }
  const int row_base = ti.row0 + 16 * RW * (wv % WM);
  const bool rows_ok = row_base < a.H;
  for (int c0 = 0; c0 < ti.n; c0 += 16 * NTT) down_dispatch<NTT, WM, WK, RW>(a, ti, c0, rows_ok, row_base, red, false);
}

#ifndef FFN_LONG_DOWN_RW
#define FFN_LONG_DOWN_RW 4
#endif
#ifndef FFN_LONG_UP_RW
#define FFN_LONG_UP_RW 2
#endif

// Row tiles per wave.  Short segments (the decode case, a few tokens per
// expert): gate/up 1; down 1 with one token tile, 2 with two to four
// (activation fragments reused twice), 1 beyond.  With one token tile the
// single row tile doubles the blocks, so no tail of CUs holding two blocks
// remains (one-token Qwen2-57B-shaped step 158 -> 153 us); with two to four
// token tiles one row tile measured 9-20 us slower.  Long segments (more
// than one token tile per expert on average): each token fragment is reused
// over more weight rows, gate/up 2 and down 4 up to 4 token tiles.
template <int NTT, bool LONG>
struct RowTiles {
  static constexpr int UP = (LONG && NTT <= 4) ? FFN_LONG_UP_RW : 1;
  static constexpr int DOWN = NTT == 1 ? 1 : (NTT <= 4 ? (LONG ? FFN_LONG_DOWN_RW : 2) : 1);
};

template <int NTT, int WM, int WK, bool LONG>
static void launch_kernels(FfnMfmaArgs up, FfnMfmaArgs dn, hipStream_t s, int which) {
  constexpr int RW = RowTiles<NTT, LONG>::DOWN;
  constexpr int RWU = RowTiles<NTT, LONG>::UP;
  const int H = up.H;
  up.tiles_r = (up.I + 16 * WM * RWU - 1) / (16 * WM * RWU);
  up.tiles_s = up.Is > 0 ? (up.Is + 16 * WM * RWU - 1) / (16 * WM * RWU) : 0;
  dn.tiles_r = (H + 16 * RW * WM - 1) / (16 * RW * WM);
  dn.tiles_s = dn.tiles_r;
  dn.tiles_l = dn.slots_l > 0 ? (H + LoreDownRows<RW>::ROWS - 1) / LoreDownRows<RW>::ROWS : 0;
  const int n_up = up.slots_r * up.tiles_r + up.n_shared_seg * up.tiles_s + up.slots_l * up.tiles_l;
  const int n_dn = dn.slots_r * dn.tiles_r + dn.n_shared_seg * dn.tiles_s + dn.slots_l * dn.tiles_l;
  if ((which & 1) && n_up > 0) ffn_up_mfma_kernel<NTT, WM, WK, RWU><<<n_up, 256, 0, s>>>(up);
  if ((which & 2) && n_dn > 0) ffn_down_mfma_kernel<NTT, WM, WK, RW><<<n_dn, 256, 0, s>>>(dn);
}

// Row strips per block for long segments up to 4 token tiles (the rest of
// the 4 waves split K): two strips, each wave streaming half of K (the
// Qwen2-57B-shaped 256-token step about 885 -> 875 us against one strip
// with a four-way k split).
#ifndef FFN_LONG_WM
#define FFN_LONG_WM 2
#endif

// which: bit 0 = gate/up kernel, bit 1 = down kernel.  lore: LoRE tiles on.
hipError_t launch_ffn_mfma(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* moffsets, const int32_t* perm,
                           const FfnBuffers& b, int routed, int shared, int lore, hipStream_t s,
                           int which) {
  // Token tiles per pass: every token when shared tiles are in the launch;
  // otherwise about twice the mean routed segment (a longer segment loops
  // over chunks, rereading its weights from cache).
  const bool shared_on = shared && d.n_shared > 0;
  const int seg_est = std::max(16, (int)((2LL * T * d.top_k + d.n_experts - 1) / d.n_experts));
  const int cover = shared_on ? T : std::min(T, seg_est);
  const int ntiles_tok = (cover + 15) / 16;
  int NTT = 1;
  while (NTT < ntiles_tok && NTT < 16) NTT <<= 1;
  const bool long_seg = routed && (int64_t)T * d.top_k > 16LL * d.n_experts;
  const int WM = NTT <= 4 ? (long_seg ? FFN_LONG_WM : 1) : (NTT == 8 ? 2 : 4);
  const int rows = 16 * WM;
  const int slots = std::min(d.n_experts, T * d.top_k);
  FfnMfmaArgs up{};
  up.x = (const bf16*)x;
  up.w0 = (const bf16*)w.w_gate;
  up.w1 = (const bf16*)w.w_up;
  up.ws0 = (const bf16*)w.ws_gate;
  up.ws1 = (const bf16*)w.ws_up;
  up.wl = (const bf16*)w.lore_A;
  up.act = b.act;
  up.acts = b.acts;
  up.z = b.z;
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
  up.packed = d.weight_layout == MOE_LAYOUT_MFMA16;
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
  dn.n_shared_seg = (shared && d.n_shared > 0) ? 1 : 0;
  // long segments: more than one token tile per routed expert on average
  if (long_seg) {
    constexpr int LWM = FFN_LONG_WM, LWK = 4 / FFN_LONG_WM;
    switch (NTT) {
      case 1: launch_kernels<1, LWM, LWK, true>(up, dn, s, which); break;
      case 2: launch_kernels<2, LWM, LWK, true>(up, dn, s, which); break;
      case 4: launch_kernels<4, LWM, LWK, true>(up, dn, s, which); break;
      case 8: launch_kernels<8, 2, 2, true>(up, dn, s, which); break;
      default: launch_kernels<16, 4, 1, true>(up, dn, s, which); break;
    }
  } else {
    switch (NTT) {
      case 1: launch_kernels<1, 1, 4, false>(up, dn, s, which); break;
      case 2: launch_kernels<2, 1, 4, false>(up, dn, s, which); break;
      case 4: launch_kernels<4, 1, 4, false>(up, dn, s, which); break;
      case 8: launch_kernels<8, 2, 2, false>(up, dn, s, which); break;
      default: launch_kernels<16, 4, 1, false>(up, dn, s, which); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
