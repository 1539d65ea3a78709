// bf16 grouped GEMM for the expert SwiGLU FFN at prefill sizes (hundreds of
// tokens per expert) on gfx950 matrix cores, v_mfma_f32_16x16x32_bf16.
//
//   GEMM1 (gate+up):  C_g = W_g X^T, C_u = W_u X^T  over one expert segment,
//                     act = SiLU(C_g) * C_u  stored bf16 [pair][I]
//   GEMM2 (down):     Y = W_d act^T                 stored fp32 [pair][H]
// [FloE page, Sec. 1, forward a^S(x) with S_t = identity.]
//
// Block tile: 128 weight rows (M) x 128 tokens (N) x 64 k per stage, 4 waves
// in a 2 x 2 grid, each wave 64 x 64 = 4 x 4 MFMA tiles (x2 for gate and up).
// A (weights) and B (token rows, gathered through the permutation) are both
// k-contiguous in HBM; each stage is copied global -> registers -> LDS with
// 16-byte loads while the previous stage feeds the MFMAs (double-buffered
// LDS, one barrier per stage).  LDS rows are padded to 72 elements so the
// 16 lanes reading one fragment column hit distinct banks.
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

constexpr int GM = 128;        // weight rows per block tile
constexpr int GN = 128;        // tokens per block tile
constexpr int GK = 64;         // k per stage
constexpr int GLD = GK + 8;    // padded LDS row (elements)
constexpr int GTHREADS = 256;
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
  const int32_t* offsets;  // routed segments [E+1]; nullptr = one segment of T rows per group
  const int32_t* perm;
  int k;                // top-k (pair -> token)
  int R, K;             // weight rows (output width), contraction length
  int G;                // groups: experts (routed) or shared experts
  int T;
  int tiles_n;          // R / GM (rounded up)
  int n_blocks;         // grid size (upper bound of tiles)
};

__device__ __forceinline__ bf16x8_t lds_frag(const bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
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

// GATED: GEMM1 (two weight matrices, SiLU product, bf16 out); else GEMM2.
template <bool GATED>
__global__ void __launch_bounds__(GTHREADS) ffn_gemm_kernel(GemmArgs a) {
  constexpr int NW = GATED ? 2 : 1;
  __shared__ bf16 lds_w[2][NW][GM][GLD];
  __shared__ bf16 lds_x[2][GN][GLD];
  const int tile = xcd_tile(blockIdx.x, a.n_blocks);
  if (tile >= a.n_blocks) return;
  const int m_idx = tile / a.tiles_n, n_idx = tile % a.tiles_n;
  MTile mt;
  if (!find_mtile(a, m_idx, mt)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;     // 2 x 2 waves
  const int r16 = lane & 15, kg = lane >> 4;
  const int row_w0 = n_idx * GM;           // first weight row of the tile

  // global -> LDS copy plan: chunk c (16 B) = row c/8, k-chunk c%8; 1024
  // chunks per 128x64 tile, 4 per thread per matrix
  const bf16* wsrc[NW][4];
  const bf16* xsrc[4];
  int crow[4], ccol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + GTHREADS * i;
    crow[i] = c >> 3;
    ccol[i] = (c & 7) * 8;
    const int wr = min(row_w0 + crow[i], a.R - 1);
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const bf16* base = (m == 0 ? a.w0 : a.w1) + (int64_t)mt.g * a.w_stride;
      wsrc[m][i] = base + (int64_t)wr * a.K + ccol[i];
    }
    const int r = min(mt.row0 + crow[i], mt.n - 1);
    if (GATED) {
      const int tok = a.offsets ? a.perm[mt.seg0 + r] / a.k : r;
      xsrc[i] = a.x + (int64_t)tok * a.K + ccol[i];
    } else {
      xsrc[i] = a.act_in + (int64_t)(mt.seg0 + r) * a.ld_in + ccol[i];
    }
  }

  f32x4_t acc[NW][4][4];
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsub = GATED ? 1 : a.n_sub;
  const int kst = a.K / GK;          // K % 64 == 0 on this path
  const int nst = nsub * kst;
  // one stage in flight per thread: 4 chunks of gate (or down), up, token rows
  uint4 w0a, w0b, w0c, w0d, w1a, w1b, w1c, w1d, xa, xb, xc, xd;
  auto gload = [&](int st) __attribute__((always_inline)) {
    const int s_ = st / kst, ko_ = (st % kst) * GK;
    const int64_t wo = (int64_t)s_ * a.sub_stride + ko_;
    const int64_t xo = (int64_t)s_ * a.sub_k_off + ko_;
    w0a = *reinterpret_cast<const uint4*>(wsrc[0][0] + wo);
    w0b = *reinterpret_cast<const uint4*>(wsrc[0][1] + wo);
    w0c = *reinterpret_cast<const uint4*>(wsrc[0][2] + wo);
    w0d = *reinterpret_cast<const uint4*>(wsrc[0][3] + wo);
    if constexpr (GATED) {
      w1a = *reinterpret_cast<const uint4*>(wsrc[NW - 1][0] + wo);
      w1b = *reinterpret_cast<const uint4*>(wsrc[NW - 1][1] + wo);
      w1c = *reinterpret_cast<const uint4*>(wsrc[NW - 1][2] + wo);
      w1d = *reinterpret_cast<const uint4*>(wsrc[NW - 1][3] + wo);
    }
    xa = *reinterpret_cast<const uint4*>(xsrc[0] + xo);
    xb = *reinterpret_cast<const uint4*>(xsrc[1] + xo);
    xc = *reinterpret_cast<const uint4*>(xsrc[2] + xo);
    xd = *reinterpret_cast<const uint4*>(xsrc[3] + xo);
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(&lds_w[buf][0][crow[0]][ccol[0]]) = w0a;
    *reinterpret_cast<uint4*>(&lds_w[buf][0][crow[1]][ccol[1]]) = w0b;
    *reinterpret_cast<uint4*>(&lds_w[buf][0][crow[2]][ccol[2]]) = w0c;
    *reinterpret_cast<uint4*>(&lds_w[buf][0][crow[3]][ccol[3]]) = w0d;
    if constexpr (GATED) {
      *reinterpret_cast<uint4*>(&lds_w[buf][NW - 1][crow[0]][ccol[0]]) = w1a;
      *reinterpret_cast<uint4*>(&lds_w[buf][NW - 1][crow[1]][ccol[1]]) = w1b;
      *reinterpret_cast<uint4*>(&lds_w[buf][NW - 1][crow[2]][ccol[2]]) = w1c;
      *reinterpret_cast<uint4*>(&lds_w[buf][NW - 1][crow[3]][ccol[3]]) = w1d;
    }
    *reinterpret_cast<uint4*>(&lds_x[buf][crow[0]][ccol[0]]) = xa;
    *reinterpret_cast<uint4*>(&lds_x[buf][crow[1]][ccol[1]]) = xb;
    *reinterpret_cast<uint4*>(&lds_x[buf][crow[2]][ccol[2]]) = xc;
    *reinterpret_cast<uint4*>(&lds_x[buf][crow[3]][ccol[3]]) = xd;
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
#pragma unroll
    for (int kk = 0; kk < GK; kk += 32) {
      bf16x8_t fa[NW][4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int m = 0; m < NW; ++m)
          fa[m][i] = lds_frag(&lds_w[buf][m][wm * 64 + 16 * i + r16][kk + 8 * kg]);
        fb[i] = lds_frag(&lds_x[buf][wn * 64 + 16 * i + r16][kk + 8 * kg]);
      }
#pragma unroll
      for (int m = 0; m < NW; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m][i], fb[j], acc[m][i][j], 0, 0, 0);
    }
    if (st + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds weight rows 4*kg..+3 of tile i, token r16 of tile j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tr = mt.row0 + wn * 64 + 16 * j + r16;   // token row within segment
    if (tr >= mt.n) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wr = row_w0 + wm * 64 + 16 * i + 4 * kg;
      if (wr >= a.R) continue;
      if (GATED) {
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = f_to_bf16(silu_f(acc[0][i][j][q]) * acc[NW - 1][i][j][q]);
        bf16* dst = a.act_out + (int64_t)(mt.seg0 + tr) * a.ld_out + (int64_t)mt.g * a.col_off + wr;
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
        float* dst = a.y_out + (int64_t)(mt.seg0 + tr) * a.R + wr;
        *reinterpret_cast<float4*>(dst) =
            float4{acc[0][i][j][0], acc[0][i][j][1], acc[0][i][j][2], acc[0][i][j][3]};
      }
    }
  }
}

// Routed experts (offsets != nullptr) or shared experts (offsets == nullptr).
// GEMM1 writes bf16 act (routed [P][I], shared [T][ns*Is]); GEMM2 writes fp32 y.
hipError_t launch_ffn_gemm(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* perm, bool shared, bf16* act,
                           float* y, hipStream_t s, int which) {
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
    a.tiles_n = (R1 + GM - 1) / GM;
    a.n_blocks = mt_max * a.tiles_n;
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
    a.y_out = y;
    a.offsets = shared ? nullptr : offsets;
    a.perm = perm;
    a.k = d.top_k;
    a.R = H;
    a.K = R1;
    a.G = shared ? 1 : E;      // shared: one segment of T tokens, sub-matrices summed
    a.T = T;
    a.tiles_n = (H + GM - 1) / GM;
    const int mt2 = shared ? (T + GN - 1) / GN : mt_max;
    a.n_blocks = mt2 * a.tiles_n;
    const int grid = ((a.n_blocks + NXCD - 1) / NXCD) * NXCD;
    if (a.n_blocks > 0) ffn_gemm_kernel<false><<<grid, GTHREADS, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
