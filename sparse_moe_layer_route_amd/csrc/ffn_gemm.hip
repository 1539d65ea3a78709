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
// loads, no register staging) into a 4-deep ring, so three stages are in
// flight while one feeds the MFMAs: the L2/HBM latency of a stage (microseconds under load)
// is covered by three stages of math.  Each 64-byte LDS row holds four
// 16-byte k chunks stored at chunk ^ ((row / 2) % 4): a 16-byte LDS read is
// served eight lanes at a time over 32 banks, and the eight rows of one such
// group then cover all 32 banks once.  Ordering is explicit: a thread
// waits for its own DMA loads with a vmcnt wait, then a workgroup barrier
// publishes the stage; a slot is refilled only after the barrier that ends
// its last read.  A long contraction over few tiles (the shared experts' down
// projection at a few hundred tokens) is split over grid.y into partial sums
// that a small kernel adds up.
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
constexpr int GSTAGES = 4;     // LDS ring depth (stages in flight: GSTAGES - 1)
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

// Block id -> logical tile id with each XCD owning a contiguous range.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int per = (n + NXCD - 1) / NXCD;
  const int xcd = b % NXCD, idx = b / NXCD;
  return xcd * per + idx;   // may exceed n for the last XCD: caller checks
}

// Logical m-tile index -> (group, first row in segment, rows, segment start).
struct MTile {
  int g, row0, n, seg0;
};

__device__ __forceinline__ bool find_mtile(const GemmArgs a, int m_idx, MTile& mt) {
  __shared__ int s_g, s_row0, s_n, s_seg0;
  if (threadIdx.x < MOE_WAVE) {
    const int lane = threadIdx.x;
    int n = 0, o0 = 0;
    if (lane < a.G) {
      if (a.offsets) {
        o0 = a.offsets[lane];
        n = a.offsets[lane + 1] - o0;
      } else {
        n = a.T;
      }
    }
    const int tiles = (n + GN - 1) / GN;
    int incl = tiles;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
      const int v = __shfl_up(incl, o, MOE_WAVE);
      if (lane >= o) incl += v;
    }
    const int excl = incl - tiles;
    if (lane == 0) s_g = -1;
    __builtin_amdgcn_wave_barrier();
    if (lane < a.G && m_idx >= excl && m_idx < incl) {
      s_g = lane;
      s_row0 = (m_idx - excl) * GN;
      s_n = n;
      s_seg0 = o0;
    }
  }
  __syncthreads();
  mt.g = s_g;
  mt.row0 = s_row0;
  mt.n = s_n;
  mt.seg0 = s_seg0;
  return mt.g >= 0;
}

// Wait until at most N of this wave's vector-memory operations are pending
// (LDS DMA loads complete in issue order).
#define GEMM_VMCNT(N) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory")
// at most two later stages of this thread's DMA loads still pending
#define GEMM_VMCNT_STAGES2() GEMM_VMCNT(2 * NQ)
#define GEMM_VMCNT_STAGES1() GEMM_VMCNT(NQ)

// The GTT token fragments (LDS rows sb + 16j) and NW*WT weight fragments (rows
// sa + m*MW + 16i) of one stage; row offsets are instruction immediates.
template <int J, int NJ>
__device__ __forceinline__ void read_fb(u32x4 (&fb)[NJ], uint32_t sb) {
  if constexpr (J < NJ) {
    fb[J] = lds_read16_at<16 * J * GK * 2>(sb);
    read_fb<J + 1, NJ>(fb, sb);
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
// else GEMM2 (256 down rows, fp32 out).  Either way a block stages 256 weight
// rows and 256 token rows per 32-wide k stage, and each wave owns a 128 x 64
// output tile (8 x 4 MFMA tiles, 128 fp32 accumulators per lane).
template <bool GATED>
__global__ void __launch_bounds__(GTHREADS) ffn_gemm_kernel(GemmArgs a) {
  constexpr int NW = GATED ? 2 : 1;          // weight matrices
  constexpr int MW = GATED ? 128 : 256;      // weight rows per matrix per block
  constexpr int WT = MW / 2 / 16;            // weight tiles per wave per matrix (4 or 8)
  __shared__ __attribute__((aligned(16))) bf16 lds[GSTAGES][GROWS * GK];
  const int tile = xcd_tile(blockIdx.x, a.n_blocks);
  if (tile >= a.n_blocks) return;
  const int m_idx = tile / a.tiles_n, n_idx = tile % a.tiles_n;
  MTile mt;
  if (!find_mtile(a, m_idx, mt)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;       // 2 x 4 waves: weight half, token quarter
  const int r16 = lane & 15, kg = lane >> 4;
  const int row_w0 = n_idx * MW;             // first weight row of the tile
  // a wave whose 64 tokens all lie past the segment end (the last m-tile of a
  // segment) still moves its share of the stages but skips the MFMAs
  const bool tok_live = mt.row0 + wn * 16 * GTT < mt.n;

  // DMA plan: a stage is 512 LDS rows x 64 B; one wave instruction writes 16
  // rows (1 KiB, lane l -> row l/4, 16-byte slot l%4).  Wave w issues
  // instructions NQ*w..NQ*w+NQ-1: waves 0-3 the weight rows (GATED: 0-127
  // gate, 128-255 up), waves 4-7 the token rows.  Slot p of row r holds k chunk
  // p ^ ((r/2) % 4), so each 8-row group of a fragment read hits 32 distinct
  // banks.
  const int chunk = (lane & 3) ^ ((lane >> 3) & 3);
  const bf16* base_w0 = a.w0 + (int64_t)mt.g * a.w_stride;
  const bf16* base_w1 = GATED ? a.w1 + (int64_t)mt.g * a.w_stride : base_w0;
  const bf16* base_x = GATED ? a.x : a.act_in;
  const bool is_w = wv < GWAVES / 2;
  // GATED: LDS rows 0-127 (waves 0-1) gate, 128-255 (waves 2-3) up
  const bf16* dma_base = is_w ? ((GATED && wv >= GWAVES / 4) ? base_w1 : base_w0) : base_x;
  constexpr int NQ = GROWS / 16 / GWAVES;   // DMA instructions per wave per stage
  constexpr int NMF = NW * WT * GTT;        // MFMAs per wave per stage
  int off[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int row = 16 * (NQ * wv + q) + (lane >> 2);   // LDS row 0..511
    if (is_w) {
      const int r = GATED ? (row & 127) : row;
      off[q] = min(row_w0 + r, a.R - 1) * a.K + 8 * chunk;
    } else {
      const int r = min(mt.row0 + (row - 256), mt.n - 1);
      if (GATED) {
        const int tok = a.offsets ? a.perm[mt.seg0 + r] / a.k : r;
        off[q] = tok * a.K + 8 * chunk;
      } else {
        off[q] = (mt.seg0 + r) * (int)a.ld_in + 8 * chunk;
      }
    }
  }

  f32x4_t acc[NW][WT][GTT];
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int i = 0; i < WT; ++i)
#pragma unroll
      for (int j = 0; j < GTT; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsub = GATED ? 1 : a.n_sub;
  const int kst = a.K / GK;          // K % 32 == 0 on this path
  const int nst = nsub * kst;
  const int per = (nst + a.ksplit - 1) / a.ksplit;
  const int k_lo = a.ksplit > 1 ? blockIdx.y * per : 0;
  const int k_hi = a.ksplit > 1 ? min(nst, k_lo + per) : nst;

  // Every step issues exactly NQ DMA loads per thread (stages past the range
  // reload the last stage into a slot nobody reads again), so "stage s+1 has
  // landed" is always "at most 2 * NQ of this thread's loads pending".
  // DMA instruction q of stage st (each stage is NQ instructions per thread).
  auto issue_one = [&](int st, int q) __attribute__((always_inline)) {
    bf16* dst = &lds[st % GSTAGES][(16 * NQ * wv) * GK];
    st = min(st, k_hi - 1);
    const int s_ = st / kst, ko = (st % kst) * GK;
    const bf16* src = dma_base + (is_w ? (int64_t)s_ * a.sub_stride : (int64_t)s_ * a.sub_k_off) + ko;
    __builtin_amdgcn_global_load_lds((const void*)(src + off[q]),
                                     (__attribute__((address_space(3))) void*)(dst + q * 16 * GK),
                                     16, 0, 0);
  };
  auto issue = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) issue_one(st, q);
  };

  // byte address of this lane's fragment slot: logical chunk kg of row r
  // lives at physical chunk kg ^ ((r/2) % 4); rows here are 16-aligned + r16
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&lds[0][0];
  const uint32_t lane_off = (uint32_t)(r16 * GK * 2 + ((kg ^ ((r16 >> 1) & 3)) * 16));

  // Stage st's fragments sit in one register set while the next stage's are
  // read into the other: after the barrier that publishes stage st+1 a wave
  // starts its LDS reads, runs stage st's MFMAs from registers, then waits for
  // the reads.  The last stage reads a slot holding a duplicate stage, which
  // is never multiplied.
#define GEMM_READ(FB, FA, st_)                                                          \
  {                                                                                     \
    const uint32_t sl = lds0 + (uint32_t)(((st_) % GSTAGES) * GROWS * GK * 2) + lane_off; \
    read_fb<0, GTT>(FB, sl + (uint32_t)((256 + wn * 16 * GTT) * GK * 2));              \
    read_fa<NW, WT, MW, 0>(FA, sl + (uint32_t)(wm * (MW / 2) * GK * 2));               \
  }
#define GEMM_MFMA(FB, FA)                                                               \
  _Pragma("unroll") for (int m = 0; m < NW; ++m)                                        \
    _Pragma("unroll") for (int i = 0; i < WT; ++i)                                      \
      _Pragma("unroll") for (int j = 0; j < GTT; ++j)                                   \
        acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                         \
            __builtin_bit_cast(bf16x8_t, FA[m * WT + i]), __builtin_bit_cast(bf16x8_t, FB[j]), \
            acc[m][i][j], 0, 0, 0);
#define GEMM_MFMA_PART(FB, FA, q)                                                       \
  _Pragma("unroll") for (int t = 0; t < NMF / NQ; ++t) {                                \
    const int L = (q) * (NMF / NQ) + t;                                                 \
    const int m = L / (WT * GTT), i = (L / GTT) % WT, j = L % GTT;                      \
    acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                             \
        __builtin_bit_cast(bf16x8_t, FA[m * WT + i]), __builtin_bit_cast(bf16x8_t, FB[j]), \
        acc[m][i][j], 0, 0, 0);                                                         \
  }
  // The refill of the slot freed two barriers ago is spread over the MFMAs so
  // the waves do not queue their DMA instructions all at once.
#define GEMM_STEP(FBc, FAc, FBn, FAn, st_)                                              \
  {                                                                                     \
    GEMM_VMCNT_STAGES1();                                                               \
    __builtin_amdgcn_s_barrier();                                                       \
    GEMM_READ(FBn, FAn, (st_) + 1);                                                     \
    __builtin_amdgcn_sched_barrier(0); /* reads issue before the MFMAs */              \
    _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                    \
      issue_one((st_) + GSTAGES - 1, q);                                                \
      __builtin_amdgcn_sched_barrier(0);                                                \
      if (tok_live) { GEMM_MFMA_PART(FBc, FAc, q); }                                    \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
    lds_wait_all(FBn, FAn);                                                             \
  }
  if (k_lo < k_hi) {
    u32x4 fb0[GTT], fa0[NW * WT], fb1[GTT], fa1[NW * WT];
    issue(k_lo);
    issue(k_lo + 1);
    issue(k_lo + 2);
    GEMM_VMCNT_STAGES2();
    __builtin_amdgcn_s_barrier();
    GEMM_READ(fb0, fa0, k_lo);
    lds_wait_all(fb0, fa0);
    for (int st = k_lo; st < k_hi; st += 2) {
      GEMM_STEP(fb0, fa0, fb1, fa1, st);
      if (st + 1 < k_hi) GEMM_STEP(fb1, fa1, fb0, fa0, st + 1);
    }
  }
#undef GEMM_READ
#undef GEMM_MFMA
#undef GEMM_STEP
#undef GEMM_MFMA_PART
  GEMM_VMCNT(0);      // no DMA may outlive the workgroup's LDS

  // epilogue: lane holds weight rows 4*kg..+3 of tile i, token r16 of tile j
#pragma unroll
  for (int j = 0; j < GTT; ++j) {
    const int tr = mt.row0 + wn * 16 * GTT + 16 * j + r16;   // token row within segment
    if (tr >= mt.n) continue;
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int wr = row_w0 + wm * (MW / 2) + 16 * i + 4 * kg;
      if (wr >= a.R) continue;
      if (GATED) {
        float h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = silu_f(acc[0][i][j][q]) * acc[NW - 1][i][j][q];
        bf16* dst = a.act_out + (int64_t)(mt.seg0 + tr) * a.ld_out + (int64_t)mt.g * a.col_off + wr;
        *reinterpret_cast<uint2*>(dst) = make_uint2(f2_to_bf16x2(h[0], h[1]), f2_to_bf16x2(h[2], h[3]));
      } else if (a.yb_out) {
        const f32x4_t& v = acc[0][i][j];
        bf16* dst = a.yb_out + (int64_t)(mt.seg0 + tr) * a.R + wr;
        *reinterpret_cast<uint2*>(dst) = make_uint2(f2_to_bf16x2(v[0], v[1]), f2_to_bf16x2(v[2], v[3]));
      } else {
        float* dst = a.y_out + (int64_t)blockIdx.y * a.part_stride + (int64_t)(mt.seg0 + tr) * a.R + wr;
        *reinterpret_cast<float4*>(dst) =
            float4{acc[0][i][j][0], acc[0][i][j][1], acc[0][i][j][2], acc[0][i][j][3]};
      }
    }
  }
}
#undef GEMM_VMCNT
#undef GEMM_VMCNT_STAGES2
#undef GEMM_VMCNT_STAGES1

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
// when there are few (token, row) tiles and a long contraction.
int gemm_shared_down_ksplit(const moe_dims_t& d, int T) {
  const int tiles = ((T + GN - 1) / GN) * ((d.hidden + 255) / 256);
  const int nst = d.n_shared * (d.shared_inter / GK);
  int ks = 256 / (tiles > 0 ? tiles : 1);
  ks = ks < 1 ? 1 : (ks > nst ? nst : ks);
  return ks;
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
    const int grid = ((a.n_blocks + NXCD - 1) / NXCD) * NXCD;
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
    a.ksplit = shared ? gemm_shared_down_ksplit(d, T) : 1;
    a.y_out = a.ksplit > 1 ? part : y;
    a.yb_out = a.ksplit > 1 ? nullptr : yb;
    a.part_stride = (int64_t)T * H;
    const int grid = ((a.n_blocks + NXCD - 1) / NXCD) * NXCD;
    if (a.n_blocks > 0) ffn_gemm_kernel<false><<<dim3(grid, a.ksplit), GTHREADS, 0, s>>>(a);
    if (a.ksplit > 1) {
      const int64_t n4 = (int64_t)T * H / 4;
      ksplit_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(part, n4, a.part_stride,
                                                                         a.ksplit, y);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
