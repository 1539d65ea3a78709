// bf16 grouped GEMM for the expert SwiGLU FFN at prefill sizes (hundreds of
// tokens per expert) on gfx950 matrix cores, v_mfma_f32_16x16x32_bf16.
//
//   GEMM1 (gate+up):  C_g = W_g X^T, C_u = W_u X^T  over one expert segment,
//                     act = SiLU(C_g) * C_u  stored bf16 [pair][I]
//   GEMM2 (down):     Y = W_d act^T                 stored fp32 [pair][H]
// [FloE page, Sec. 1, forward a^S(x) with S_t = identity.]
//
// Block tile: 256 tokens (N) x 256 weight rows (M: 128 gate + 128 up, or 256
// down) x 32 k per stage, 8 waves (two per SIMD) in a 2 x 4 grid, each wave
// 128 weight rows x 64 tokens = 8 x 4 MFMA tiles in 128 accumulator
// registers.  Per stage a wave reads 12 fragments (12 KiB) from LDS for 32
// MFMAs, and while one wave of a SIMD waits on LDS the other issues MFMAs;
// a block pulls 32 KiB per stage from L2 for 4.2 MFLOP (128 flop/B).  A
// (weights) and B (token rows, gathered through the permutation) are both
// k-contiguous in HBM.  Stages move global -> LDS directly (16-byte LDS DMA
// loads, no register staging) into two rings: weight rows 4 deep (three
// stages in flight) and the gathered token rows 5 deep.  Weight rows are read
// 64 bytes (32 k) per stage; token rows 128 bytes (64 k, one whole cache
// line) per load, so a token slot holds half the rows of a pair of stages
// (rows 0-127 or 128-255, 64 k each): fetching each line's two halves in two
// stages had made the L2 -> LDS stream 15% slower (with the arithmetic left
// out, 131 -> 114 us for the Granite-shaped gate/up launch).  With both the
// stream and the arithmetic measured apart (114 and 105 us there) the
// whole launch takes about 132 us: the two overlap only in part.  Each
// 64-byte weight row holds four 16-byte k chunks stored at chunk ^ ((row / 2)
// % 4), each 128-byte token row eight stored at chunk ^ (row % 8): a 16-byte
// LDS read is served eight lanes at a time over 32 banks, and the eight rows
// of one such group then cover all 32 banks once.  Ordering is explicit: a
// thread waits for its own DMA loads with a vmcnt wait, then a workgroup
// barrier publishes the stage; a slot is refilled only after the barrier
// that ends its last read.  A long contraction over few tiles (the shared
// experts' down projection at a few hundred tokens) is split over grid.y
// into partial sums that a small kernel adds up.
//
// Tiles are (segment m-tile, weight n-tile) pairs enumerated expert by expert;
// block ids are remapped so each XCD (blocks are dealt to the 8 XCDs round-
// robin) gets a contiguous range of tiles, keeping an expert's weights and
// token tiles inside one XCD's L2.
#include <algorithm>

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GN = 256;        // tokens per block tile
constexpr int GK = 32;         // k per stage
#ifndef GEMM_WSTAGES
#define GEMM_WSTAGES 4
#endif
#ifndef GEMM_TSTAGES
#define GEMM_TSTAGES 5
#endif
constexpr int GWST = GEMM_WSTAGES;  // weight-row LDS ring depth (stages in flight: GWST - 1)
constexpr int GTST = GEMM_TSTAGES;  // token-row LDS ring depth (stages in flight: GTST - 1)
constexpr int GROWS = 512;     // LDS rows per stage: 256 weight + 256 token
constexpr int GTHREADS = 512;  // 8 waves: two per SIMD
constexpr int GWAVES = GTHREADS / 64;
constexpr int GTT = 4;         // token tiles (16 each) per wave: 64 tokens
constexpr int NXCD = 8;

struct GemmArgs {
  const bf16* x;        // GEMM1 B rows: x [T][H] (token of pair via perm)
  const bf16* act_in;   // GEMM2 B rows: act [rows][ld_in]
  const bf16* w0;       // GEMM1: gate [G][R][K]; GEMM2: down [G][R][K] (per sub-matrix)
  const bf16* w1;       // GEMM1: up
  int64_t w_stride;     // elements between groups (experts or shared experts)
  int64_t sub_stride;   // GEMM2 shared: elements between the n_sub down matrices
  int n_sub;            // GEMM2 shared: sub-matrices summed (K of each = K)
  int64_t ld_in;        // GEMM2: row stride of act_in
  int64_t sub_k_off;    // GEMM2 shared: column offset of sub-matrix s in act_in (= K)
  bf16* act_out;        // GEMM1 out
  int64_t ld_out;       // GEMM1 out row stride
  int64_t col_off;      // GEMM1 out column offset per group (shared: I_s)
  float* y_out;         // GEMM2 out [rows][R]
  bf16* yb_out;         // GEMM2 out as bf16 [rows][R] instead (nullptr: y_out)
  const int32_t* offsets;  // routed segments [E+1]; nullptr = one segment of T rows per group
  const int32_t* perm;
  int k;                // top-k (pair -> token)
  int R, K;             // weight rows (output width), contraction length
  int G;                // groups: experts (routed) or shared experts
  int T;
  int tiles_n;          // weight-row tiles (128 gate+up rows or 256 down rows)
  int ksplit;           // GEMM2: k-stage ranges (grid.y); partial sums to y_out + y * part_stride
  int64_t part_stride;
  int n_blocks;         // grid size (upper bound of tiles)
  int packed;           // weights fragment-major [R/16][K/32][64][8] (R % 16 == K % 32 == 0 here)
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte LDS read issued as an instruction the compiler's wait-count pass
// does not track: the ring's DMA writes are ordered by explicit waits and
// barriers instead (the pass would otherwise drain every DMA in flight before
// each read).  Results are used only after lds_wait_all.
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
// Same, with a compile-time byte offset folded into the instruction.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF) : "memory");
  return r;
}

// 8-byte LDS store issued outside the compiler's wait-count tracking, like
// the reads above (stores have no result register).
__device__ __forceinline__ void lds_write8(uint32_t addr, uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = {lo, hi};
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Wait for this wave's LDS reads; the fragments are in/out operands so no
// use of them can be scheduled above the wait.
template <int NA, int NB>
__device__ __forceinline__ void lds_wait_all(u32x4 (&b)[NB], u32x4 (&a)[NA]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(b[j]));
#pragma unroll
  for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(a[i]));
}

// Segment table in LDS, entry e for group e (expert, or shared expert):
// start, rows, and the m-tiles of the groups before it.  Built by wave 0;
// the caller publishes it with a barrier.  Returns the total m-tiles.
struct SegTable {
  int o0[MOE_WAVE], n[MOE_WAVE], excl[MOE_WAVE];
};

__device__ __forceinline__ int seg_table_build(const GemmArgs& a, SegTable& t) {
  const int lane = lane_id();
  int o0 = 0, n = 0;
  if (lane < a.G) {
    if (a.offsets) {
      o0 = a.offsets[lane];
      n = a.offsets[lane + 1] - o0;
    } else {
      n = a.T;
    }
  }
  const int tiles = (n + GN - 1) / GN;
  const int incl = wave_incl_scan_i(tiles);
  if (threadIdx.x < MOE_WAVE) {
    t.o0[lane] = o0;
    t.n[lane] = n;
    t.excl[lane] = incl - tiles;
  }
  return __builtin_amdgcn_readlane(incl, MOE_WAVE - 1);
}

// One (m-tile, weight-tile) pair, or half of one: group, first row in the
// segment, the end of its live rows (segment rows, capped at the tile's
// span), segment start, weight-row tile.
struct TileMeta {
  int g, row0, lim, seg0, n_idx;
};
constexpr int GEMM_MAX_TILES = 14;  // tiles per persistent block (the grid grows beyond)
struct TileTable {
  int g[GEMM_MAX_TILES], row0[GEMM_MAX_TILES], lim[GEMM_MAX_TILES], seg0[GEMM_MAX_TILES],
      n_idx[GEMM_MAX_TILES];
};

// How an XCD's tiles are dealt to its blocks.  The `cnt` tiles from `base`
// go round-robin to the `nbx` blocks, `full` whole rounds and then `rem`
// tiles.  When that last, partial round holds at most half as many tiles as
// there are blocks, each of its tiles is split into two 128-token halves, a
// block apiece: a half keeps only the four waves of its 128 tokens busy
// (waves 0-3, one per SIMD when waves are dealt to the SIMDs in turn) and
// measured a little over half a tile's time, so the round no longer
// costs a whole tile while half the CUs idle.  Either way every output
// element is formed by the same MFMA sequence, so results do not change.
struct TileDeal {
  int base, full, rem;
  bool split;
};
__device__ __forceinline__ TileDeal tile_deal(int n_tiles, int per_x, int xcd, int nbx) {
  TileDeal d;
  d.base = xcd * per_x;
  const int cnt = max(0, min(n_tiles, d.base + per_x) - d.base);
  d.full = cnt / nbx;
  d.rem = cnt % nbx;
  d.split = d.rem > 0 && 2 * d.rem <= nbx;
  return d;
}
__device__ __forceinline__ int tile_count(const TileDeal& d, int bi, int nbx) {
  if (d.split) return d.full + (bi < 2 * d.rem ? 1 : 0);
  const int cnt = d.full * nbx + d.rem;
  return bi < cnt ? (cnt - bi + nbx - 1) / nbx : 0;
}

// Lane j of the calling wave fills entry j of block bi's tiles from the
// published segment table.
__device__ __forceinline__ void tile_table_build(const GemmArgs& a, const SegTable& sg,
                                                 const TileDeal& d, int bi, int nbx, int count,
                                                 TileTable& tt) {
  const int j = lane_id();
  if (j >= count) return;
  int t, half = -1;
  if (d.split && j == d.full) {
    t = d.base + d.full * nbx + bi / 2;
    half = bi & 1;
  } else {
    t = d.base + bi + j * nbx;
  }
  const int m_idx = t / a.tiles_n;
  int g = 0;
  for (int e = 0; e < a.G; ++e) {
    const int tiles = (sg.n[e] + GN - 1) / GN;
    if (m_idx >= sg.excl[e] && m_idx < sg.excl[e] + tiles) g = e;
  }
  const int row0 = (m_idx - sg.excl[g]) * GN + (half > 0 ? GN / 2 : 0);
  tt.g[j] = g;
  tt.row0[j] = row0;
  tt.lim[j] = min(sg.n[g], row0 + (half >= 0 ? GN / 2 : GN));
  tt.seg0[j] = sg.o0[g];
  tt.n_idx[j] = t % a.tiles_n;
}

__device__ __forceinline__ TileMeta tile_get(const TileTable& tt, int j) {
  TileMeta m;
  m.g = __builtin_amdgcn_readfirstlane(tt.g[j]);
  m.row0 = __builtin_amdgcn_readfirstlane(tt.row0[j]);
  m.lim = __builtin_amdgcn_readfirstlane(tt.lim[j]);
  m.seg0 = __builtin_amdgcn_readfirstlane(tt.seg0[j]);
  m.n_idx = __builtin_amdgcn_readfirstlane(tt.n_idx[j]);
  return m;
}

// Wait until at most N of this wave's vector-memory operations are pending
// (LDS DMA loads complete in issue order).
#define GEMM_VMCNT(N) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory")

// The GTT token fragments (LDS rows sb + 16j, RS bytes a row) and NW*WT weight
// fragments (rows sa + m*MW + 16i) of one stage; row offsets are instruction
// immediates.
template <int J, int NJ, int RS>
__device__ __forceinline__ void read_fb(u32x4 (&fb)[NJ], uint32_t sb) {
  if constexpr (J < NJ) {
    fb[J] = lds_read16_at<16 * J * RS>(sb);
    read_fb<J + 1, NJ, RS>(fb, sb);
  }
}
// Entries LO..HI-1 of the stage's read list: the NJ token fragments (128-byte
// token rows), then the weight fragments.
template <int L, int HI, int NJ, int NW, int WT, int MW>
__device__ __forceinline__ void read_range(u32x4 (&fb)[NJ], u32x4 (&fa)[NW * WT], uint32_t sb,
                                           uint32_t sa) {
  if constexpr (L < HI) {
    if constexpr (L < NJ) {
      fb[L] = lds_read16_at<16 * L * 128>(sb);
    } else {
      constexpr int Q = L - NJ, m = Q / WT, i = Q % WT;
      fa[Q] = lds_read16_at<(m * MW + 16 * i) * GK * 2>(sa);
    }
    read_range<L + 1, HI, NJ, NW, WT, MW>(fb, fa, sb, sa);
  }
}
template <int NW, int WT, int MW, int Q>
__device__ __forceinline__ void read_fa(u32x4 (&fa)[NW * WT], uint32_t sa) {
  if constexpr (Q < NW * WT) {
    constexpr int m = Q / WT, i = Q % WT;
    fa[Q] = lds_read16_at<(m * MW + 16 * i) * GK * 2>(sa);
    read_fa<NW, WT, MW, Q + 1>(fa, sa);
  }
}

// GATED: GEMM1 (gate and up matrices, 128 rows each, SiLU product, bf16 out);
// else GEMM2 (256 down rows, fp32 or bf16 out).  Either way a block stages
// 256 weight rows and 256 token rows per 32-wide k stage, and each wave owns a
// 128 x 64 output tile (8 x 4 MFMA tiles, 128 fp32 accumulators per lane).
//
// Blocks are persistent: block b works through its share of the tiles (those
// of its XCD, strided by the XCD's blocks), and its k stages form one stream
// through the LDS ring across tile boundaries, so the first stages of the
// next tile load while the current tile finishes and writes its outputs.
// YB (GEMM2 only): the outputs are bf16 rows (a.yb_out), else fp32 (a.y_out).
template <bool GATED, bool YB = false>
__global__ void __launch_bounds__(GTHREADS) ffn_gemm_kernel(GemmArgs a) {
  constexpr int NW = GATED ? 2 : 1;          // weight matrices
  constexpr int MW = GATED ? 128 : 256;      // weight rows per matrix per block
  constexpr int WT = MW / 2 / 16;            // weight tiles per wave per matrix (4 or 8)
  __shared__ __attribute__((aligned(16))) bf16 lds_w[GWST][GN * GK];   // 256 weight rows per stage
  __shared__ __attribute__((aligned(16))) bf16 lds_t[GTST][GN * GK];   // 256 token rows per stage
  __shared__ SegTable seg;
  const int n_tiles = seg_table_build(a, seg) * a.tiles_n;   // every wave: same total
  __syncthreads();
  // this block's tiles: XCD x owns a contiguous range, dealt to its blocks
  const int nbx = gridDim.x / NXCD, xcd = blockIdx.x % NXCD, bi = blockIdx.x / NXCD;
  const int per_x = (n_tiles + NXCD - 1) / NXCD;
  const TileDeal deal = tile_deal(n_tiles, per_x, xcd, nbx);
  const int n_my = tile_count(deal, bi, nbx);
  if (n_my == 0) return;
  __shared__ TileTable tt;
  if (threadIdx.x < MOE_WAVE) tile_table_build(a, seg, deal, bi, nbx, n_my, tt);
  __syncthreads();
  // element offset of every token row of every tile of this block, gathered
  // up front so the stream never waits on the permutation mid-flight
  __shared__ int tok_base[GEMM_MAX_TILES][GN];
  static_assert(GN <= GTHREADS, "one token row per thread");
  if (threadIdx.x < GN) {
    const int ld = GATED ? a.K : (int)a.ld_in;
    const int r = threadIdx.x;
    for (int j0 = 0; j0 < n_my; j0 += 4) {   // four tiles' permutation loads in flight
      int tok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const TileMeta m = tile_get(tt, min(j0 + u, n_my - 1));
        const int rr = min(m.row0 + r, m.lim - 1);   // rows past the live ones repeat the last
        tok[u] = GATED ? (a.offsets ? a.perm[m.seg0 + rr] / a.k : rr) : m.seg0 + rr;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n_my) tok_base[j0 + u][r] = tok[u] * ld;
    }
  }
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
  const int wm = wv & 1, wn = wv >> 1;       // 2 x 4 waves: weight half, token quarter
  const int r16 = lane & 15, kg = lane >> 4;

  const int nsub = GATED ? 1 : a.n_sub;
  const int kst = a.K / GK;          // K % 32 == 0 on this path
  const int nst_all = nsub * kst;
  // every k range even, so a pair of stages never straddles two
  const int kper = 2 * ((nst_all + 2 * a.ksplit - 1) / (2 * a.ksplit));
  const int k_lo = a.ksplit > 1 ? blockIdx.y * kper : 0;
  const int k_hi = a.ksplit > 1 ? min(nst_all, k_lo + kper) : nst_all;
  const int nst = max(0, k_hi - k_lo);       // stages per tile
  const int S = n_my * nst;                  // stages of this block's stream

  // DMA plan: one wave instruction writes 1 KiB of LDS (16 B per lane, lane
  // l at byte 16 l).  Waves 0-3 load the weight rows of stage s (256 rows x
  // 64 B, GATED: rows 0-127 gate, 128-255 up; instruction q of wave w: rows
  // 16 (NQ w + q) + l / 4, slot l % 4 holding k chunk (l % 4) ^ ((row / 2) % 4)).
  // Waves 4-7 load, at stream stage s, half s % 2 of the token rows of the
  // stage pair (s & ~1, s | 1): 128 rows x 128 B (instruction q of wave w:
  // rows 128 (s % 2) + 32 (w - 4) + 8 q + l / 8, slot l % 8 holding k chunk
  // (l % 8) ^ (row % 8) of the pair's 64 k) into token slot s % GTST.
  const bool is_w = wv < GWAVES / 2;
  // A weight wave issues stage s + GWST - 1 at step s, a token wave stream
  // stage s + GTST - 1 (the sweep of the two depths at the Granite shape put
  // the longer lead on the gathered token rows).  Before the barrier of step
  // s each thread's own loads for the reads of stage s + 1 must have landed:
  // for weights stage s + 1 (at most GWST - 3 later stages pending), for
  // tokens both halves of its pair, the later being stream stage s + 1 (s
  // even: GTST - 3 pending) or s + 2 (s odd: GTST - 4).  A token slot is
  // refilled GTST stream stages later, after the last read of its pair (the
  // reads of stage 2v + 1 at step 2v), which lead <= GTST - 1 guarantees.
  const int lead = is_w ? GWST - 1 : GTST - 1;
  static_assert(GWST >= 3 && GTST >= 4 && GWST + GTST <= 9, "ring depths");
  const int wsh = a.packed ? 4 : 0;
  constexpr int NQ = GROWS / 16 / GWAVES;   // DMA instructions per wave per stage
  constexpr int NMF = NW * WT * GTT;        // MFMAs per wave per stage

  // DMA state: the tile the stream is loading, its base and per-lane offsets
  int dj = 0, dk = 0;   // stream position of the next DMA stage: tile, stage in tile
  TileMeta dm = tile_get(tt, 0);
  const bf16* dbase;
  int off[2][NQ];   // [token half][instruction]; weight waves use off[0]
  // Only at tile switches: the lane index is formed afresh (an opaque copy),
  // so nothing lane-derived stays live across the stage loop for it (a value
  // spilled there would be reloaded behind a full vmcnt wait, draining the
  // ring).
  auto set_dma = [&](const TileMeta& m, int j) __attribute__((always_inline)) {
    int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(ln));
    const int chunk = (ln & 3) ^ ((ln >> 3) & 3);
    auto dma_row = [&](int q) __attribute__((always_inline)) { return 16 * (NQ * wv + q) + (ln >> 2); };
    if (is_w) {
      const bf16* w = (GATED && wv >= GWAVES / 4) ? a.w1 : a.w0;
      dbase = w + (int64_t)m.g * a.w_stride;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int r = GATED ? (dma_row(q) & 127) : dma_row(q);
        const int row = min(m.n_idx * MW + r, a.R - 1);
        // fragment-major: the 16 rows of one DMA instruction are one
        // contiguous 1 KiB fragment, row r%16 chunk c at lane slot 16c + r%16
        off[0][q] = a.packed ? (row >> 4) * (a.K >> 5) * 512 + (16 * chunk + (row & 15)) * 8
                             : row * a.K + 8 * chunk;
      }
    } else {
      dbase = GATED ? a.x : a.act_in;
      // half h of a stage pair: token row 128 h + 32 (w - 4) + 8 q + lane / 8,
      // 16-byte slot lane % 8 holding k chunk (lane % 8) ^ (row % 8) of the
      // pair's 64 k: eight lanes read one whole 128-byte line of a row
      const int c8 = (ln & 7) ^ ((ln >> 3) & 7);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          off[h][q] = tok_base[j][128 * h + 32 * (wv - GWAVES / 2) + 8 * q + (ln >> 3)] + 8 * c8;
    }
  };
  set_dma(dm, 0);
  // The DMA stream visits (tile, k stage) in order; dma_next() returns the k
  // stage of the next stream stage.  Stages past the end reload the last one
  // into a slot nobody reads again, so every step issues exactly NQ loads per
  // thread and "stream stage x has landed" is a fixed count of pending loads.
  auto dma_next = [&]() __attribute__((always_inline)) {
    if (dk == nst) {            // the previous stage ended a tile
      if (dj + 1 < n_my) {
        dk = 0;
        ++dj;
        dm = tile_get(tt, dj);
        set_dma(dm, dj);
      } else {
        dk = nst - 1;           // past the end: the last stage again
      }
    }
    return k_lo + dk++;
  };
  auto issue_one = [&](int s, int kstage, int q) __attribute__((always_inline)) {
    bf16* dst = is_w ? &lds_w[s % GWST][(16 * NQ * wv) * GK]
                     : &lds_t[s % GTST][(16 * NQ * (wv - GWAVES / 2)) * GK];
    const int s_ = kstage / kst;
    // token pairs: stream stage s is half s % 2 of the pair starting at the
    // even k stage (stage and stream parities agree: every k range is even)
    const int th = is_w ? 0 : (kstage & 1);
    const int ko = ((kstage % kst) - th) * GK;
    // weight k stage stride: 32 elements row-major, a 512-element fragment packed
    const bf16* src = dbase + (is_w ? (int64_t)s_ * a.sub_stride + (ko << wsh)
                                    : (int64_t)s_ * a.sub_k_off + ko);
    __builtin_amdgcn_global_load_lds((const void*)(src + (th ? off[1][q] : off[0][q])),
                                     (__attribute__((address_space(3))) void*)(dst + q * 16 * GK),
                                     16, 0, 0);
  };

  // compute state: the tile whose stages the MFMAs consume
  int cj = 0, ck = 0;   // compute position: tile, stage in tile
  TileMeta cm = dm;
  // a wave whose 64 tokens all lie past the tile's live rows (the last m-tile
  // of a segment, the upper half of a tile split in two) still moves its
  // share of the stages but skips its fragment reads and MFMAs
  bool tok_live = cm.row0 + wn * 16 * GTT < cm.lim;

  f32x4_t acc[NW][WT][GTT];
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int i = 0; i < WT; ++i)
#pragma unroll
      for (int j = 0; j < GTT; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // epilogue of the compute tile: lane holds weight rows 4*kg..+3 of tile i,
  // token r16 of tile j; then the accumulators restart for the next tile
  // GEMM2's bf16 rows go through LDS (staged): the wave's 4 KiB region of a
  // ring slot that the tile's last stage has finished with (nothing refills
  // it before the next barrier), written in the accumulator layout and read
  // back row by row, so each global store writes whole 256-byte row
  // segments instead of 32-byte pieces of 16 rows (the Granite-shaped down
  // GEMM: 95 -> 85 us).  16-byte chunk c of row r sits at chunk c ^ (r % 16),
  // so the row reads are free of bank conflicts.  The gate/up epilogue keeps
  // its direct stores: staging it measured no faster there (the extra
  // registers spill) and slower on the shared experts' GEMM.
  auto epilogue = [&](uint32_t ebase, bool staged) __attribute__((always_inline)) {
    const int row_w0 = cm.n_idx * MW;
    // Lane-derived values are formed here from an opaque copy of the lane
    // index, not kept in registers across the stage loop: one spilled there
    // would be reloaded here behind a full vmcnt wait, draining the ring.
    int eln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(eln));
    const int r16 = eln & 15, kg = eln >> 4;
    if (YB && staged) {
      // bf16 rows: columns col0..col0+127, four passes of 16 tokens
      const int col0 = row_w0 + wm * (MW / 2);
#pragma unroll
      for (int j = 0; j < GTT; ++j) {
        __builtin_amdgcn_sched_barrier(0);   // one pass at a time (register pressure)
#pragma unroll
        for (int i = 0; i < WT; ++i) {
          const f32x4_t& v = acc[0][i][j];
          const int c16 = 2 * i + (kg >> 1);
          lds_write8(ebase + r16 * 256 + ((c16 ^ r16) << 4) + ((kg & 1) << 3),
                     f2_to_bf16x2(v[0], v[1]), f2_to_bf16x2(v[2], v[3]));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) {   // one 4-row group at a time (register pressure)
          const int row = kg + 4 * q, c = r16;
          u32x4 v[1] = {lds_read16(ebase + row * 256 + ((c ^ row) << 4))};
          lds_wait_all(v, v);
          const int tr = cm.row0 + wn * 16 * GTT + 16 * j + row;
          const int col = col0 + 8 * c;
          if (tr < cm.lim && col < a.R) {
            bf16* dst = a.yb_out + (int64_t)(cm.seg0 + tr) * a.R + col;
            *reinterpret_cast<u32x4*>(dst) = v[0];
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < GTT; ++j) {
        const int tr = cm.row0 + wn * 16 * GTT + 16 * j + r16;   // token row within segment
        if (tr >= cm.lim) continue;
#pragma unroll
        for (int i = 0; i < WT; ++i) {
          const int wr = row_w0 + wm * (MW / 2) + 16 * i + 4 * kg;
          if (wr >= a.R) continue;
          if (GATED) {
            float h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = silu_f(acc[0][i][j][q]) * acc[NW - 1][i][j][q];
            bf16* dst = a.act_out + (int64_t)(cm.seg0 + tr) * a.ld_out + (int64_t)cm.g * a.col_off + wr;
            *reinterpret_cast<uint2*>(dst) = make_uint2(f2_to_bf16x2(h[0], h[1]), f2_to_bf16x2(h[2], h[3]));
          } else {   // fp32 rows (bf16 rows are always staged: they come with k-split 1)
            float* dst = a.y_out + (int64_t)blockIdx.y * a.part_stride + (int64_t)(cm.seg0 + tr) * a.R + wr;
            *reinterpret_cast<float4*>(dst) =
                float4{acc[0][i][j][0], acc[0][i][j][1], acc[0][i][j][2], acc[0][i][j][3]};
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NW; ++m)
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < GTT; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  auto next_compute_tile = [&]() __attribute__((always_inline)) {
    ++cj;
    if (cj < n_my) {
      cm = tile_get(tt, cj);
      tok_live = cm.row0 + wn * 16 * GTT < cm.lim;
    }
  };

  if (nst == 0) {  // an empty k range (k split): the partial sums are zero
    for (int j = 0; j < n_my; ++j) {
      epilogue(0u, false);
      next_compute_tile();
    }
    return;
  }

  // byte address of this lane's weight fragment slot: logical chunk kg of row
  // r lives at physical chunk kg ^ ((r/2) % 4); rows here are 16-aligned + r16
  const uint32_t ldsw0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&lds_w[0][0];
  const uint32_t ldst0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&lds_t[0][0];
  uint32_t lane_off = (uint32_t)(r16 * GK * 2 + ((kg ^ ((r16 >> 1) & 3)) * 16));
  // token pairs: 128-byte rows, chunk c of row r at slot c ^ (r % 8); the
  // odd stage of a pair reads chunks 4..7 (byte offset bit 6 toggled)
  uint32_t lane_off_t = (uint32_t)(r16 * 128 + ((kg ^ (r16 & 7)) * 16));

  // Stage s's fragments sit in one register set while the next stage's are
  // read into the other: after the barrier that publishes stage s+1 a wave
  // starts its LDS reads, runs stage s's MFMAs from registers, then waits for
  // the reads.  The last stage reads a slot holding a duplicate stage, which
  // is never multiplied.
#define GEMM_ADDR(st_)                                                                  \
    asm volatile("" : "+v"(lane_off)); /* addresses formed here, not kept live */       \
    asm volatile("" : "+v"(lane_off_t));                                                \
    const uint32_t slw = ldsw0 + (uint32_t)(((st_) % GWST) * GN * GK * 2) + lane_off     \
                         + (uint32_t)(wm * (MW / 2) * GK * 2);                          \
    /* the wave's 64 token rows lie in half wn / 2 of the pair of stage st_ */         \
    const uint32_t slt = ldst0 + (uint32_t)(((((st_) & ~1) + (wn >> 1)) % GTST) * GN * GK * 2) \
                         + (uint32_t)((wn & 1) * 64 * 128) + (lane_off_t ^ (((st_) & 1) << 6));
#define GEMM_READ(FB, FA, st_)                                                          \
  {                                                                                     \
    GEMM_ADDR(st_)                                                                      \
    read_fb<0, GTT, 128>(FB, slt);                                                      \
    read_fa<NW, WT, MW, 0>(FA, slw);                                                    \
  }
  constexpr int NRD = (GTT + NW * WT) / NQ;   // fragment reads per MFMA part
  static_assert((GTT + NW * WT) % NQ == 0, "reads split evenly over the parts");
#define GEMM_READ_PART(FB, FA, q)                                                       \
  {                                                                                     \
    if ((q) == 0) read_range<0, NRD, GTT, NW, WT, MW>(FB, FA, slt, slw);                \
    else if ((q) == 1) read_range<NRD, 2 * NRD, GTT, NW, WT, MW>(FB, FA, slt, slw);     \
    else if ((q) == 2) read_range<2 * NRD, 3 * NRD, GTT, NW, WT, MW>(FB, FA, slt, slw); \
    else read_range<3 * NRD, 4 * NRD, GTT, NW, WT, MW>(FB, FA, slt, slw);               \
  }
#define GEMM_MFMA_PART(FB, FA, q)                                                       \
  _Pragma("unroll") for (int t = 0; t < NMF / NQ; ++t) {                                \
    const int L = (q) * (NMF / NQ) + t;                                                 \
    const int m = L / (WT * GTT), i = (L / GTT) % WT, j = L % GTT;                      \
    acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
        __builtin_bit_cast(bf16x8_t, FA[m * WT + i]), __builtin_bit_cast(bf16x8_t, FB[j]), \
        acc[m][i][j], 0, 0, 0);                                                         \
  }
  // The next stage's fragment reads and the refill of the slot freed two
  // barriers ago are spread over the MFMA parts (three reads and one DMA
  // load before each eight MFMAs), so the eight waves leaving a barrier do
  // not queue their LDS reads all at once (1-2% off the Granite-shaped
  // launches against issuing the twelve reads first).  A tile's last stage is
  // followed by its epilogue, and the next stage's fragments are read only
  // after it (they are not live while the outputs are formed).
// PAR: parity of st_.  Token pairs: the reads of stage st_ + 1 need both
// halves of its pair, the later of which is stream stage st_ + 2 (st_ odd) or
// st_ + 1 (st_ even); stages up to st_ + GTST - 2 have been issued.
#define GEMM_STEP(FBc, FAc, FBn, FAn, st_, PAR)                                         \
  {                                                                                     \
    const bool last = ++ck == nst;                                                      \
    if (is_w) GEMM_VMCNT((GWST - 3) * NQ); else GEMM_VMCNT((GTST - 3 - (PAR)) * NQ);  \
    __builtin_amdgcn_s_barrier();                                                       \
    {                                                                                   \
      const bool rd = !last && tok_live;                                                \
      GEMM_ADDR((st_) + 1)                                                              \
      const int kref = dma_next();                                                      \
      _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                  \
        if (rd) GEMM_READ_PART(FBn, FAn, q);                                            \
        __builtin_amdgcn_sched_barrier(0);                                              \
        issue_one((st_) + lead, kref, q);                                               \
        __builtin_amdgcn_sched_barrier(0);                                              \
        if (tok_live) { GEMM_MFMA_PART(FBc, FAc, q); }                                  \
        __builtin_amdgcn_sched_barrier(0);                                              \
      }                                                                                 \
    }                                                                                   \
    if (last) {                                                                         \
      ck = 0;                                                                           \
      epilogue(is_w ? ldsw0 + (uint32_t)(((st_) % GWST) * GN * GK * 2 + wv * 4096)        \
                    : ldst0 + (uint32_t)(((st_) % GTST) * GN * GK * 2 + (wv - 4) * 4096), \
               true);                                                                   \
      next_compute_tile();                                                              \
      /* unconditional, so the fragment sets are not live across the epilogue */       \
      GEMM_READ(FBn, FAn, (st_) + 1);                                                   \
    }                                                                                   \
    lds_wait_all(FBn, FAn);                                                             \
  }
  {
    u32x4 fb0[GTT], fa0[NW * WT], fb1[GTT], fa1[NW * WT];
    for (int s0 = 0; s0 < lead; ++s0) {
      const int kref = dma_next();
#pragma unroll
      for (int q = 0; q < NQ; ++q) issue_one(s0, kref, q);
    }
    // stage 0 landed (token pairs: both halves of pair 0, stream stages 0 and 1)
    if (is_w) GEMM_VMCNT((GWST - 2) * NQ); else GEMM_VMCNT((GTST - 3) * NQ);
    __builtin_amdgcn_s_barrier();
    if (tok_live) GEMM_READ(fb0, fa0, 0);
    lds_wait_all(fb0, fa0);
    for (int st = 0; st < S; st += 2) {
      GEMM_STEP(fb0, fa0, fb1, fa1, st, 0);
      if (st + 1 < S) GEMM_STEP(fb1, fa1, fb0, fa0, st + 1, 1);
    }
  }
#undef GEMM_READ
#undef GEMM_READ_PART
#undef GEMM_ADDR
#undef GEMM_STEP
#undef GEMM_MFMA_PART
  GEMM_VMCNT(0);      // no DMA may outlive the workgroup's LDS
}
#undef GEMM_VMCNT

// Sum of k-split partials: y[i] = sum_s part[s][i] (float4 per thread).
__global__ void __launch_bounds__(256)
ksplit_reduce_kernel(const float* __restrict__ part, int64_t n4, int64_t stride, int ns,
                     float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 acc = reinterpret_cast<const float4*>(part)[i];
  for (int s = 1; s < ns; ++s) {
    const float4 v = reinterpret_cast<const float4*>(part + s * stride)[i];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4*>(y)[i] = acc;
}

// k-splits of the shared experts' down GEMM: enough blocks to cover the CUs
// when there are few (token, row) tiles and a long contraction, but no more
// than one block per CU: the grid's x extent is the tile count rounded up to
// the XCD count, and a block fills its CU, so a grid past 256 blocks runs a
// second round (14 tiles split 18 ways took two rounds; split 16 ways, one).
int gemm_shared_down_ksplit(const moe_dims_t& d, int T) {
  const int tiles = ((T + GN - 1) / GN) * ((d.hidden + 255) / 256);
  const int nst = d.n_shared * (d.shared_inter / GK);
  const int gx = ((std::max(tiles, 1) + NXCD - 1) / NXCD) * NXCD;
  int ks = 256 / gx;
  ks = ks < 1 ? 1 : (ks > nst ? nst : ks);
  return ks;
}

// Persistent grid: one block per CU (a block's LDS ring fills a CU), shared
// by the k splits, a multiple of the XCD count; fewer when there are fewer
// tiles (an upper bound here: the routing decides the exact count).
constexpr int GEMM_CUS = 256;
static int gemm_grid(int tiles_upper, int ksplit) {
  int g = std::min(tiles_upper, std::max(NXCD, GEMM_CUS / std::max(1, ksplit)));
  // each XCD's range is dealt to its blocks: at most GEMM_MAX_TILES apiece
  const int per_x = (tiles_upper + NXCD - 1) / NXCD;
  g = std::max(g, NXCD * ((per_x + GEMM_MAX_TILES - 1) / GEMM_MAX_TILES));
  return ((g + NXCD - 1) / NXCD) * NXCD;
}

// Routed experts (offsets != nullptr) or shared experts (offsets == nullptr).
// GEMM1 writes bf16 act (routed [P][I], shared [T][ns*Is]); GEMM2 writes fp32
// y (shared: through k-split partials in `part`, then summed).
hipError_t launch_ffn_gemm(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* perm, bool shared, bf16* act,
                           float* y, bf16* yb, float* part, hipStream_t s, int which) {
  const int H = d.hidden, E = d.n_experts;
  const int R1 = shared ? d.shared_inter : d.inter;     // GEMM1 rows
  const int G = shared ? d.n_shared : E;
  const int P = T * d.top_k;
  // upper bound of m-tiles over all segments
  const int mt_max = shared ? G * ((T + GN - 1) / GN) : (P + GN - 1) / GN + std::min(E, P);
  // token pairs take the contraction 64 at a time
  if (H % 64 != 0 || R1 % 64 != 0) return hipErrorInvalidValue;
  if (which & 1) {
    GemmArgs a{};
    a.x = (const bf16*)x;
    a.w0 = (const bf16*)(shared ? w.ws_gate : w.w_gate);
    a.w1 = (const bf16*)(shared ? w.ws_up : w.w_up);
    a.w_stride = (int64_t)R1 * H;
    a.n_sub = 1;
    a.act_out = act;
    a.ld_out = shared ? (int64_t)d.n_shared * d.shared_inter : d.inter;
    a.col_off = shared ? d.shared_inter : 0;
    a.offsets = shared ? nullptr : offsets;
    a.perm = perm;
    a.k = d.top_k;
    a.R = R1;
    a.K = H;
    a.G = G;
    a.T = T;
    a.tiles_n = (R1 + 127) / 128;            // 128 gate + 128 up rows per block
    a.n_blocks = mt_max * a.tiles_n;
    a.ksplit = 1;
    a.packed = d.weight_layout == MOE_LAYOUT_MFMA16;
    const int grid = gemm_grid(a.n_blocks, 1);
    if (a.n_blocks > 0) ffn_gemm_kernel<true><<<grid, GTHREADS, 0, s>>>(a);
  }
  if (which & 2) {
    GemmArgs a{};
    a.act_in = act;
    a.w0 = (const bf16*)(shared ? w.ws_down : w.w_down);
    a.w1 = nullptr;
    a.w_stride = shared ? 0 : (int64_t)H * d.inter;
    a.sub_stride = shared ? (int64_t)H * d.shared_inter : 0;
    a.n_sub = shared ? d.n_shared : 1;
    a.ld_in = shared ? (int64_t)d.n_shared * d.shared_inter : d.inter;
    a.sub_k_off = shared ? d.shared_inter : 0;
    a.offsets = shared ? nullptr : offsets;
    a.perm = perm;
    a.k = d.top_k;
    a.R = H;
    a.K = R1;
    a.G = shared ? 1 : E;      // shared: one segment of T tokens, sub-matrices summed
    a.T = T;
    a.tiles_n = (H + 255) / 256;             // 256 down rows per block
    const int mt2 = shared ? (T + GN - 1) / GN : mt_max;
    a.n_blocks = mt2 * a.tiles_n;
    a.packed = d.weight_layout == MOE_LAYOUT_MFMA16;
    a.ksplit = shared ? gemm_shared_down_ksplit(d, T) : 1;
    a.y_out = a.ksplit > 1 ? part : y;
    a.yb_out = a.ksplit > 1 ? nullptr : yb;
    a.part_stride = (int64_t)T * H;
    const int grid = gemm_grid(a.n_blocks, a.ksplit);
    if (a.n_blocks > 0) {
      if (a.yb_out)
        ffn_gemm_kernel<false, true><<<dim3(grid, a.ksplit), GTHREADS, 0, s>>>(a);
      else
        ffn_gemm_kernel<false, false><<<dim3(grid, a.ksplit), GTHREADS, 0, s>>>(a);
    }
    if (a.ksplit > 1) {
      const int64_t n4 = (int64_t)T * H / 4;
      ksplit_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(part, n4, a.part_stride,
                                                                         a.ksplit, y);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
