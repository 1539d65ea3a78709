// FloE expert [FloE page, Sec. 1 "Hybrid compression"; Sec. 3 sparse GEMV]:
//   u = x W_up with 2-bit group-quantised W_up, decoded in registers;
//   S_t keeps the floe_keep channels of largest |u| (ties -> lower channel);
//   g_i = x . W_gate[i] and a_i = SiLU(g_i) u_i only for kept channels;
//   y = sum over kept i of a_i W_down[i, :]  (down stored channel-major).
//
// up:     each wave owns a few consecutive up rows and issues all their
//         loads before any arithmetic; lane l owns quantisation group l (16
//         bytes of codes = one 16-byte load) and forms s * (sum_h q_h x_h -
//         z * sum_h x_h), the group's (q - z) * s dot product, before one
//         transposed wave reduction for all rows of the wave.  bf16 inputs
//         decode codes straight into bf16 pairs for pair-dot instructions
//         (see floe_up_bf16_kernel); fp32 inputs unpack four codes at a time,
//         (word >> 2j) & 0x03030303 leaving code j of every byte in that
//         byte, which converts to float with a single byte-to-float op.
// select: one 1024-thread workgroup per pair; |u| is staged through LDS with
//         coalesced reads, then each thread holds the bit patterns (monotone
//         for non-negative floats) of up to 16 consecutive channels in
//         registers; MSB-first radix select (12 + 12 + 8 bits) for the
//         keep-th largest with LDS histograms; one block scan lists the kept
//         channels in ascending order (a second one ranks equal keys when
//         only some of them are kept: lower channels first).
// gate+down (layer forward): one block per slice of 16 kept channels of a
//         pair forms their activations and their contribution to all H
//         outputs (down rows prefetched during the gate sweep) into a slice
//         partial; one more launch sums the slices in a fixed order and
//         applies the combine weights, writing the layer output.
// gate, down, reduce (the unfused expert-FFN entry point, which returns the
//         per-pair rows): each gate wave owns two kept channel rows; each
//         down thread owns 8 output columns of a 32-channel slice, eight rows
//         in flight; the slices are summed in a fixed order.
#include <type_traits>

#include "common.h"

namespace moe {

// Expert weights (INT2 codes, kept gate and down rows) are read once per
// call, so their loads are non-temporal: streamed without displacing x and
// the small per-pair arrays the blocks share in L2.  FLOE_NT_WEIGHTS = 0
// restores ordinary loads.
#ifndef FLOE_NT_WEIGHTS
#define FLOE_NT_WEIGHTS 1
#endif
typedef unsigned int floe_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 weight_load16(const void* p) {
#if FLOE_NT_WEIGHTS
  const floe_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const floe_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

constexpr int FLOE_UP_RPW = 4;          // up rows per wave
constexpr int FLOE_GATE_RPW = 2;        // gate rows per wave
constexpr int FLOE_DOWN_COLS = 1024;    // output columns per down block (8 per thread)
constexpr int FLOE_SELECT_THREADS = 1024;
constexpr int FLOE_SELECT_CH = 16;      // channels per select thread (I <= 16384)
constexpr int FLOE_MAX_INTER = MOE_FLOE_MAX_DIM;
static_assert(FLOE_MAX_INTER <= FLOE_SELECT_THREADS * FLOE_SELECT_CH, "select covers every channel");
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
  const int i0 = (blockIdx.x * 4 + wv) * FLOE_UP_RPW;
  if (i0 >= I) return;
  const Tin* xr = x + (int64_t)t * H;
  for (int g0 = 0; g0 < G; g0 += MOE_WAVE) {
    const int g = g0 + lane;
    const bool act = g < G;
    uint4 cw[FLOE_UP_RPW];
    float sc[FLOE_UP_RPW], zp[FLOE_UP_RPW];
    if (act) {
#pragma unroll
      for (int q = 0; q < FLOE_UP_RPW; ++q) {
        const int64_t row = (int64_t)e * I + min(i0 + q, I - 1);
        cw[q] = weight_load16(up_q + row * (H >> 2) + (int64_t)g * 16);
        sc[q] = half_bits_to_f(up_s[row * G + g]);
        zp[q] = half_bits_to_f(up_z[row * G + g]);
      }
    }
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
    float part[FLOE_UP_RPW];
#pragma unroll
    for (int q = 0; q < FLOE_UP_RPW; ++q) {
      part[q] = 0.f;
      if (act) {
        const uint32_t words[4] = {cw[q].x, cw[q].y, cw[q].z, cw[q].w};
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
        part[q] = sc[q] * (acc - zp[q] * xs);
      }
    }
#pragma unroll
    for (int q = 0; q < FLOE_UP_RPW; ++q) {
      const float uval = wave_sum(part[q]);
      if (lane == 0 && i0 + q < I) {
        float* o = u_out + (int64_t)blockIdx.y * I + i0 + q;
        if (g0 == 0) *o = uval;
        else *o += uval;
      }
    }
  }
}

// bf16 inputs: the group dot product runs on bf16 pair dot instructions.
// Code word w of a group holds h = 16w + 4b + j at bits 8b + 2j, so the codes
// of h and h + 8 sit 16 bits apart and one shift moves a pair of them under
// a mask in both bf16 halves.  OR-ing the masked codes into 1.0 (0x3F80)
// gives the exact bf16 values 1 + q/4 (codes at mantissa bits 5-6) or
// 1 + q/16 (bits 3-4); one shift serves both, so a code word costs four
// shifts, eight and-or and eight pair dots for its 16 codes.  With
//   accH = sum over odd h of (1 + q_h/4) x_h,  accL = sum over even h of
//   (1 + q_h/16) x_h,  xsH / xsL the odd / even sums of x,
// the group term is s * (4 accH + 16 accL - (4 + z) xsH - (16 + z) xsL).
// The block first stores x as (x_h, x_{h+8}) pairs in LDS (16-byte chunks
// XOR-swizzled by group) with the odd / even sums of every group.
// v + (value of the lane given by DPP control CTRL)
template <int CTRL>
__device__ __forceinline__ float dpp_take(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sums RPW per-lane values over the wave; lane r (r < RPW) returns the total
// of value r.  The first log2(RPW) steps halve the values a lane carries:
// step b keeps the values whose index bit 0 equals lane bit b and adds the
// partner's copy of them.  Partners are lane ^ 1, lane ^ 2, then rotations by
// 4 and 8 inside the 16-lane row (each pairs lanes of opposite bit 2 or 3 and
// equal lower bits), then lanes 16 and 32 apart.
template <int RPW>
__device__ __forceinline__ float floe_wave_sum_rows(float (&v)[RPW], int lane) {
  static_assert(RPW == 4 || RPW == 8, "rows per wave");
#pragma unroll
  for (int b = 0, n = RPW; n > 1; ++b, n >>= 1) {
    const bool up = (lane >> b) & 1;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float mine = up ? v[2 * j + 1] : v[2 * j];
      const float other = up ? v[2 * j] : v[2 * j + 1];
      float got;
      if (b == 0) got = dpp_take<0xB1>(other);        // lane ^ 1
      else if (b == 1) got = dpp_take<0x4E>(other);   // lane ^ 2
      else got = dpp_take<0x124>(other);              // row rotate by 4
      v[j] = mine + got;
    }
  }
  float r = v[0];
  if (RPW == 4) r += dpp_take<0x124>(r);  // row rotate by 4
  r += dpp_take<0x128>(r);                // row rotate by 8
  r += __shfl_xor(r, 16, MOE_WAVE);
  r += __shfl_xor(r, 32, MOE_WAVE);
  return r;
}

constexpr int FLOE_UP_BF16_RPW = 4;  // up rows per wave (bf16 path)
constexpr int FLOE_MAX_HIDDEN = MOE_FLOE_MAX_DIM;

template <int RPW>
__global__ void __launch_bounds__(256)
floe_up_bf16_kernel(const bf16* __restrict__ x, const uint8_t* __restrict__ up_q,
                    const uint16_t* __restrict__ up_s, const uint16_t* __restrict__ up_z, int H,
                    int I, int E, int k, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ perm, float* __restrict__ u_out) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  // dynamic LDS: H / 8 chunks of x pairs (8 per group), then G (odd, even) sums
  extern __shared__ uint4 xl[];
  float2* xsl = reinterpret_cast<float2*>(xl + H / 8);
  int f, t, e;
  if (!pair_of(blockIdx.y, E, k, offsets, perm, f, t, e)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int G = H >> 6;  // groups per row
  constexpr uint32_t ONES = 0x3F803F80u;  // bf16 pair (1, 1)
  constexpr uint32_t ODD = 0x3F800000u;  // bf16 pair (0, 1): upper x of a raw pair (odd h)
  // bf16 pair (1, 0): lower x (even h).  Kept in a VGPR: as an immediate the
  // compiler encodes it as the inline constant 1.0, which the pair dot does
  // not read as bf16 (1, 0).
  uint32_t even = 0x00003F80u;
  asm volatile("" : "+v"(even));
  {
    // item (g, w): the 16 x of code word w of group g -> eight pairs
    const uint4* xg = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
    for (int it = threadIdx.x; it < H / 16; it += 256) {
      const int g = it >> 2, w = it & 3;
      const uint4 lo = xg[2 * it], hi = xg[2 * it + 1];  // h = 16w .. 16w+7, 16w+8 .. 16w+15
      const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, c[4] = {hi.x, hi.y, hi.z, hi.w};
      uint32_t pw[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[2 * i] = (a[i] & 0xFFFFu) | (c[i] << 16);
        pw[2 * i + 1] = (a[i] >> 16) | (c[i] & 0xFFFF0000u);
      }
      float so = 0.f, se = 0.f;  // odd h are the upper halves of the raw pairs
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        so = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[i]),
                                             __builtin_bit_cast(bf16x2, ODD), so, false);
        so = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c[i]),
                                             __builtin_bit_cast(bf16x2, ODD), so, false);
        se = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[i]),
                                             __builtin_bit_cast(bf16x2, even), se, false);
        se = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c[i]),
                                             __builtin_bit_cast(bf16x2, even), se, false);
      }
      xl[g * 8 + ((2 * w) ^ (g & 7))] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      xl[g * 8 + ((2 * w + 1) ^ (g & 7))] = make_uint4(pw[4], pw[5], pw[6], pw[7]);
      // the four items of a group are adjacent lanes (H / 16 is a multiple of 4)
      so += __shfl_xor(so, 1, MOE_WAVE);
      so += __shfl_xor(so, 2, MOE_WAVE);
      se += __shfl_xor(se, 1, MOE_WAVE);
      se += __shfl_xor(se, 2, MOE_WAVE);
      if (w == 0) xsl[g] = make_float2(so, se);
    }
  }
  __syncthreads();
  // wave-uniform row numbers, so the row addresses stay scalar
  const int i0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wv)) * RPW;
  if (i0 >= I) return;
  const int64_t rbase = (int64_t)e * I + i0;
  uint32_t ones = ONES;  // opaque VGPR: (v & mask) | ones is one v_and_or_b32
  asm volatile("" : "+v"(ones));
  float part[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) part[q] = 0.f;
  for (int g0 = 0; g0 < G; g0 += MOE_WAVE) {
    // lanes past the last group redo it and drop the result
    const bool act = g0 + lane < G;
    const int g = act ? g0 + lane : G - 1;
    uint4 cw[RPW];
    uint32_t sz[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int64_t row = rbase + min(q, I - 1 - i0);
      const uint8_t* qr = up_q + row * (H >> 2);
      const uint16_t* sr = up_s + row * G;
      const uint16_t* zr = up_z + row * G;
      cw[q] = weight_load16(qr + g * 16);
      sz[q] = (uint32_t)sr[g] | ((uint32_t)zr[g] << 16);
    }
    uint32_t xp[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 v = xl[g * 8 + (c ^ (g & 7))];
      xp[4 * c] = v.x;
      xp[4 * c + 1] = v.y;
      xp[4 * c + 2] = v.z;
      xp[4 * c + 3] = v.w;
    }
    const float2 xsg = xsl[g];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const uint32_t words[4] = {cw[q].x, cw[q].y, cw[q].z, cw[q].w};
      float accH = 0.f, accL = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // codes 2m+1 and 2m (and their +8 partners) to bits 5-6 and 3-4
          const int sh = 4 * m - 3;
          const uint32_t v = sh >= 0 ? words[w] >> sh : words[w] << -sh;
          const uint32_t ph = (v & 0x00600060u) | ones, pl = (v & 0x00180018u) | ones;
          accH = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ph),
                                                 __builtin_bit_cast(bf16x2, xp[8 * w + 2 * m + 1]),
                                                 accH, false);
          accL = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pl),
                                                 __builtin_bit_cast(bf16x2, xp[8 * w + 2 * m]),
                                                 accL, false);
        }
      }
      const float sc = half_bits_to_f((uint16_t)(sz[q] & 0xFFFFu));
      const float zp = half_bits_to_f((uint16_t)(sz[q] >> 16));
      const float term = sc * (4.f * accH + 16.f * accL - (4.f + zp) * xsg.x - (16.f + zp) * xsg.y);
      part[q] += act ? term : 0.f;
    }
  }
  const float uval = floe_wave_sum_rows<RPW>(part, lane);
  if (lane < RPW && i0 + lane < I) u_out[(int64_t)blockIdx.y * I + i0 + lane] = uval;
}

// Wave-wide maximum (MAX) or minimum of unsigned values, in every lane, on
// the DPP network (lanes with no source keep their own value).
template <bool MAX>
__device__ __forceinline__ uint32_t dpp_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  int x = (int)v;
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x111, 0xf, false>(x, x));
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x112, 0xf, false>(x, x));
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x114, 0xf, false>(x, x));
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x118, 0xf, false>(x, x));
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x142, 0xa, false>(x, x));
  x = (int)op((uint32_t)x, (uint32_t)dpp_move<0x143, 0xc, false>(x, x));
  return (uint32_t)__builtin_amdgcn_readlane(x, MOE_WAVE - 1);
}

constexpr int FLOE_SELECT_WAVES = FLOE_SELECT_THREADS / MOE_WAVE;

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int s = wave_incl_scan_i(v);
  if (lane == MOE_WAVE - 1) wsum[wv] = s;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < FLOE_SELECT_WAVES; ++w) {
    const int c = wsum[w];
    base += w < wv ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + s - v;
}

// Thread tid owns the CH consecutive channels [tid*ch, tid*ch + ch) (ch <=
// FLOE_SELECT_CH) and keeps their |u| bit patterns in registers through all
// radix passes, so a pass is CH histogram increments per thread and the final
// ascending listing is one block scan over per-thread counts.  The select
// runs on one CU per pair as a chain of block-wide steps, so each step is
// kept short: scans and reductions on the DPP lane network, the histogram of
// the next pass cleared while this one fills (two buffers), the bin sums read
// 16 bytes at a time, and the mask-edge flag settled at the listing's
// barrier.  (At one Mixtral-shaped token these took the launch from 15.4 to
// 12.4 us in the kernel trace: LDS permutes for every scan step, a dependent
// loop of LDS reads over the later waves and two more barriers per pass had
// each waited on LDS round trips.)
__global__ void __launch_bounds__(FLOE_SELECT_THREADS)
floe_select_kernel(const float* __restrict__ u, int I, int n_keep, float margin, int E, int k,
                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                   int32_t* __restrict__ keep_out,
                   uint32_t* __restrict__ flags) {
  constexpr int CH = FLOE_SELECT_CH;
  __shared__ uint32_t stage[FLOE_MAX_INTER];  // coalesced landing area for |u|
  __shared__ __attribute__((aligned(16))) int hist[2][4096];
  __shared__ int wsum[FLOE_SELECT_WAVES];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ uint32_t s_next, s_kmin;
  __shared__ int s_eqcnt, s_done;
  int f, t, e;
  if (!pair_of(blockIdx.x, E, k, offsets, perm, f, t, e)) return;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int ch = (I + FLOE_SELECT_THREADS - 1) / FLOE_SELECT_THREADS;
  const int i0 = tid * ch;
  const float* ur = u + (int64_t)blockIdx.x * I;
  // coalesced global reads into LDS (all of a thread's loads in flight
  // together), then each thread takes its chunk; the first pass's
  // histogram is cleared meanwhile
  {
    float v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = tid + j * FLOE_SELECT_THREADS;
      v[j] = i < I ? ur[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[0][tid + j * FLOE_SELECT_THREADS] = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = tid + j * FLOE_SELECT_THREADS;
      if (i < I) stage[i] = __float_as_uint(fabsf(v[j]));
    }
  }
  if (tid == 0) {
    s_prefix = 0u;
    s_need = n_keep;
    s_next = 0u;
    s_kmin = 0xFFFFFFFFu;
    s_done = 0;
  }
  __syncthreads();
  uint32_t key[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int i = i0 + j;
    key[j] = (j < ch && i < I) ? stage[i] : 0u;
  }
  // MSB-first radix select on 12 + 12 + 8 bits: the 12-bit first digit
  // (exponent and three mantissa bits) spreads |u| over tens of bins, so the
  // histogram increments of the first pass, which every key makes, rarely
  // collide on one LDS word.  (Merging a thread's increments in registers
  // first costs more VALU issue than the atomics it saves: a wave64
  // instruction takes four cycles on a 16-lane SIMD, and the whole select
  // runs on one CU per pair.)
  uint32_t pmask = 0u;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = pass == 2 ? 256 : 4096;
    int* h = hist[pass & 1];
    // this pass's prefix and count, read before the barriers of the pass:
    // the thread that finds the bin rewrites both after the second one
    const uint32_t prefix = s_prefix;
    const int need = s_need;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (j < ch && i0 + j < I && (key[j] & pmask) == prefix)
        atomicAdd(&h[(key[j] >> shift) & (uint32_t)(nb - 1)], 1);
    }
    if (pass < 2) {   // the next pass's bins (4096, then 256)
      int* hn = hist[(pass + 1) & 1];
      for (int j = tid; j < (pass == 0 ? 4096 : 256); j += FLOE_SELECT_THREADS) hn[j] = 0;
    }
    __syncthreads();
    // thread tid owns bins [bpt*tid, bpt*tid + bpt); suffix sums over threads
    const int bpt = nb >= FLOE_SELECT_THREADS ? nb / FLOE_SELECT_THREADS : 1;
    const bool owns = tid * bpt < nb;
    int hb[4] = {0, 0, 0, 0};
    if (bpt == 4) {
      const int4 v4 = reinterpret_cast<const int4*>(h)[tid];
      hb[0] = v4.x; hb[1] = v4.y; hb[2] = v4.z; hb[3] = v4.w;
    } else if (owns) {
      hb[0] = h[tid];
    }
    const int tsum = hb[0] + hb[1] + hb[2] + hb[3];
    const int pre = wave_incl_scan_i(tsum);
    if (lane == MOE_WAVE - 1) wsum[wv] = pre;
    __syncthreads();
    int after = 0;   // the waves after this one
#pragma unroll
    for (int w = 0; w < FLOE_SELECT_WAVES; ++w) {
      const int c = wsum[w];
      after += w > wv ? c : 0;
    }
    // inclusive suffix sum: the keys in this thread's bins and above
    const int suf = __builtin_amdgcn_readlane(pre, MOE_WAVE - 1) - pre + tsum + after;
    if (owns && suf >= need && suf - tsum < need) {
      // the bin holding the need-th largest key: walk down from the top bin
      int gt = suf - tsum, sel = 0, gsel = 0, hsel = 0;
      bool found = false;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (b < bpt && !found) {
          if (gt + hb[b] >= need) {
            found = true;
            sel = b;
            gsel = gt;
            hsel = hb[b];
          } else {
            gt += hb[b];
          }
        }
      }
      s_prefix = prefix | ((uint32_t)(tid * bpt + sel) << shift);
      s_need = need - gsel;
      s_eqcnt = hsel;  // after the last pass: keys equal to the threshold
      // every key of the chosen bin is kept: the bin's lower bound already
      // separates kept from dropped keys, and the remaining passes can go
      s_done = hsel == need - gsel;
    }
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
    if (s_done) break;
  }
  const uint32_t thr = s_prefix;
  const int need_eq = s_need;
  const int eq_total = s_eqcnt;
  uint32_t below_max = 0u;
#pragma unroll
  for (int j = 0; j < CH; ++j)
    if (j < ch && i0 + j < I && key[j] < thr && key[j] > below_max) below_max = key[j];
  // kept: above the threshold, or among the first need_eq equal keys in
  // channel order (all of them when every equal key is kept)
  uint32_t kept = 0u;  // bit j: channel i0 + j kept
  if (eq_total == need_eq) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (j < ch && i0 + j < I && key[j] >= thr) kept |= 1u << j;
  } else {
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j) n_eq += (j < ch && i0 + j < I && key[j] == thr) ? 1 : 0;
    int eq_sum;
    int r = block_excl_scan(n_eq, wsum, eq_sum);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (j < ch && i0 + j < I) {
        bool kp = key[j] > thr;
        if (key[j] == thr) {
          kp = r < need_eq;
          ++r;
        }
        if (kp) kept |= 1u << j;
      }
    }
  }
  // smallest kept key (the threshold itself unless the passes stopped early)
  // and largest dropped key, per wave into LDS before the listing's barrier
  {
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (((kept >> j) & 1u) && key[j] < mn) mn = key[j];
    mn = dpp_reduce_u32<false>(mn);
    const uint32_t bm = dpp_reduce_u32<true>(below_max);
    if (lane == 0) {
      atomicMin(&s_kmin, mn);
      atomicMax(&s_next, bm);
    }
  }
  // ascending listing: exclusive scan of the per-thread kept counts
  const int cnt = __popc(kept);
  const int pre = wave_incl_scan_i(cnt);
  if (lane == MOE_WAVE - 1) wsum[wv] = pre;
  __syncthreads();
  int pos = pre - cnt;
#pragma unroll
  for (int w = 0; w < FLOE_SELECT_WAVES; ++w) {
    const int c = wsum[w];
    pos += w < wv ? c : 0;
  }
  int32_t* ko = keep_out + (int64_t)f * n_keep;
#pragma unroll
  for (int j = 0; j < CH; ++j)
    if (((kept >> j) & 1u) && pos < n_keep) ko[pos++] = i0 + j;
  // near-tie at the edge: next value below the threshold, or a tie at it
  if (n_keep < I && tid == 0) {
    const bool tie = eq_total > need_eq || (__uint_as_float(s_kmin) - __uint_as_float(s_next)) < margin;
    if (tie) atomicOr(&flags[t], 8u);
  }
}

// 8 consecutive inputs as raw bits, converted at use.
template <typename Tin> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_w(const bf16* p) { v = weight_load16(p); }
  __device__ __forceinline__ void to_f(float (&o)[8]) const {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load_w(const float* p) {
    const uint4 u = weight_load16(p), v = weight_load16(p + 4);
    a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    b = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
  __device__ __forceinline__ void to_f(float (&o)[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// A kept channel read from the keep list, held inside [0, I): the select
// writes exactly n_keep valid channels, and this keeps a weight-row address
// in bounds whatever the list holds.
__device__ __forceinline__ int keep_channel(int v, int I) { return (unsigned)v < (unsigned)I ? v : 0; }

// Kept channel c of pair p: a[p][c] = SiLU(x_t . W_gate[e][keep[c]]) * u[p][keep[c]].
// Wave w of block b owns channels (4b + w) * FLOE_GATE_RPW + q; the H loop
// takes 512 inputs per step (8 per lane) and loads both rows' chunks first.
template <typename Tin>
__global__ void __launch_bounds__(256)
floe_gate_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wg, const float* __restrict__ u,
                 int H, int I, int n_keep, int E, int k, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, const int32_t* __restrict__ keep,
                 float* __restrict__ a_out) {
  constexpr int R = FLOE_GATE_RPW;
  constexpr int NB = 8;  // 512-input chunks loaded together (4096 inputs)
  int f, t, e;
  if (!pair_of(blockIdx.y, E, k, offsets, perm, f, t, e)) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * 4 + wv) * R;
  if (c0 >= n_keep) return;
  const Tin* xr = x + (int64_t)t * H;
  int ch[R];
  const Tin* rows[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    ch[q] = keep_channel(keep[(int64_t)f * n_keep + min(c0 + q, n_keep - 1)], I);
    rows[q] = wg + ((int64_t)e * I + ch[q]) * H;
  }
  float acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = 0.f;
  for (int h0 = 0; h0 < H; h0 += NB * 512) {
    Raw8<Tin> w[R][NB], xv[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int h = min(h0 + 512 * j + 8 * lane, H - 8);
#pragma unroll
      for (int q = 0; q < R; ++q) w[q][j].load_w(rows[q] + h);
      xv[j].load(xr + h);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (h0 + 512 * j + 8 * lane >= H) continue;
      float xf[8];
      xv[j].to_f(xf);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        float wf[8];
        w[q][j].to_f(wf);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[q] = fmaf(wf[c], xf[c], acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const float g = wave_sum(acc[q]);
    if (lane == 0 && c0 + q < n_keep)
      a_out[(int64_t)blockIdx.y * n_keep + c0 + q] = silu_f(g) * u[(int64_t)blockIdx.y * I + ch[q]];
  }
}

// Partial y over one slice of FLOE_DOWN_SLICE kept channels; eight channel
// rows are loaded before their multiply-adds.
template <typename Tin>
__global__ void __launch_bounds__(FLOE_DOWN_COLS / 8)
floe_down_kernel(const Tin* __restrict__ wd, const float* __restrict__ a, int H, int I, int n_keep,
                 int P_max, int E, int k, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, const int32_t* __restrict__ keep,
                 float* __restrict__ part) {
  constexpr int B = 8;
  int f, t, e;
  if (!pair_of(blockIdx.z, E, k, offsets, perm, f, t, e)) return;
  const int h = (blockIdx.x * (FLOE_DOWN_COLS / 8) + threadIdx.x) * 8;
  if (h >= H) return;
  const int c0 = blockIdx.y * FLOE_DOWN_SLICE, c1 = min(n_keep, c0 + FLOE_DOWN_SLICE);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* ar = a + (int64_t)blockIdx.z * n_keep;
  const int32_t* kr = keep + (int64_t)f * n_keep;
  for (int c = c0; c < c1; c += B) {
    Raw8<Tin> w[B];
    float av[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int cc = min(c + u, c1 - 1);
      av[u] = c + u < c1 ? ar[cc] : 0.f;
      w[u].load_w(wd + ((int64_t)e * I + keep_channel(kr[cc], I)) * H + h);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      float wf[8];
      w[u].to_f(wf);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(av[u], wf[j], acc[j]);
    }
  }
  float* o = part + ((int64_t)blockIdx.y * P_max + blockIdx.z) * H + h;
  *reinterpret_cast<float4*>(o) = float4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<float4*>(o + 4) = float4{acc[4], acc[5], acc[6], acc[7]};
}

// y[p] = sum of the slices' partials, added in slice order.
__global__ void __launch_bounds__(256)
floe_reduce_kernel(const float* __restrict__ part, int H, int n_slices, int P_max, int E,
                   const int32_t* __restrict__ offsets, float* __restrict__ y) {
  constexpr int B = 8;
  const int p = blockIdx.y;
  if (p >= offsets[E]) return;
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  float s = 0.f;
  for (int sl = 0; sl < n_slices; sl += B) {
    float v[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
      v[u] = sl + u < n_slices ? part[((int64_t)(sl + u) * P_max + p) * H + h] : 0.f;
#pragma unroll
    for (int u = 0; u < B; ++u) s += v[u];
  }
  y[(int64_t)p * H + h] = s;
}

// Gate and down of one slice of FLOE_GD_SLICE kept channels of one pair, in
// one block of NWV waves: the waves form the slice's a_c = SiLU(x . W_gate[ch_c])
// u_ch (S / NWV channel rows each), then every thread sums a_c W_down[ch_c][h]
// over the slice for its columns (eight at a time) into the slice's partial
// row part[slice][p][:].  One launch instead of a gate and a down launch, and
// the activations never leave the block.  Loads are issued as: the first
// batch of gate chunks (every row's chunks and x's), then the first columns'
// down rows, then the gate multiply-adds, which wait only for their own batch
// (a wave's loads complete in issue order), while the down rows arrive.  With
// eight waves (bf16) a 4096-wide layer's gate and down rows are all in one
// batch each, a single round trip to memory per block.
#ifndef FLOE_GD_SLICE_N
#define FLOE_GD_SLICE_N 16
#endif
#ifndef FLOE_GD_WAVES_BF16
#define FLOE_GD_WAVES_BF16 8
#endif
constexpr int FLOE_GD_SLICE = FLOE_GD_SLICE_N;
template <typename Tin>
constexpr int floe_gd_waves() { return std::is_same<Tin, float>::value ? 4 : FLOE_GD_WAVES_BF16; }

template <typename Tin, int NWV>
__global__ void __launch_bounds__(NWV * 64)
floe_gate_down_kernel(const Tin* __restrict__ x, const Tin* __restrict__ wg,
                      const Tin* __restrict__ wd, const float* __restrict__ u, int H, int I,
                      int n_keep, int P_max, int E, int k, const int32_t* __restrict__ offsets,
                      const int32_t* __restrict__ perm, const int32_t* __restrict__ keep,
                      float* __restrict__ part) {
  constexpr int TH = NWV * 64, S = FLOE_GD_SLICE, R = S / NWV;
  constexpr int NB = NWV >= 8 ? 8 : 4;     // 512-input gate chunks per batch
  constexpr int CS = 8 * TH;               // columns per down pass
  constexpr int PRE = CS >= 4096 ? 1 : 4096 / CS;   // down passes whose rows load first
  static_assert(S % NWV == 0, "slice channels per wave");
  __shared__ int s_ch[S];
  __shared__ float s_a[S];
  int f, t, e;
  if (!pair_of(blockIdx.y, E, k, offsets, perm, f, t, e)) return;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int c0 = blockIdx.x * S, nc = min(S, n_keep - c0);
  if (tid < S) s_ch[tid] = keep_channel(keep[(int64_t)f * n_keep + c0 + min(tid, nc - 1)], I);
  __syncthreads();
  // gate: wave wv owns slice channels wv*R .. wv*R + R - 1
  const Tin* xr = x + (int64_t)t * H;
  const Tin* rows[R];
#pragma unroll
  for (int q = 0; q < R; ++q) rows[q] = wg + ((int64_t)e * I + s_ch[wv * R + q]) * H;
  float acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = 0.f;
  Raw8<Tin> w[R][NB], xv[NB];
  auto gate_load = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int h = min(h0 + 512 * j + 8 * lane, H - 8);
#pragma unroll
      for (int q = 0; q < R; ++q) w[q][j].load_w(rows[q] + h);
      xv[j].load(xr + h);
    }
  };
  auto gate_fma = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (h0 + 512 * j + 8 * lane >= H) continue;
      float xf[8];
      xv[j].to_f(xf);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        float wf[8];
        w[q][j].to_f(wf);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[q] = fmaf(wf[c], xf[c], acc[q]);
      }
    }
  };
  gate_load(0);
  // the first PRE passes' down rows (columns 8*tid + CS*m) load behind it
  Raw8<Tin> wpre[PRE][S];
#pragma unroll
  for (int m = 0; m < PRE; ++m) {
    const int h = min(8 * tid + CS * m, H - 8);
#pragma unroll
    for (int c = 0; c < S; ++c) wpre[m][c].load_w(wd + ((int64_t)e * I + s_ch[c]) * H + h);
  }
  gate_fma(0);
  for (int h0 = NB * 512; h0 < H; h0 += NB * 512) {
    gate_load(h0);
    gate_fma(h0);
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const float g = wave_sum(acc[q]);
    const int c = wv * R + q;
    if (lane == 0) s_a[c] = c < nc ? silu_f(g) * u[(int64_t)blockIdx.y * I + s_ch[c]] : 0.f;
  }
  __syncthreads();
  // down: columns 8*tid + CS*m; channels past the slice's end carry a = 0
  float a[S];
#pragma unroll
  for (int c = 0; c < S; ++c) a[c] = s_a[c];
  float* prow = part + ((int64_t)blockIdx.x * P_max + blockIdx.y) * H;
  auto sum_store = [&](const Raw8<Tin> (&wr)[S], int h) {
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S; ++c) {
      float wf[8];
      wr[c].to_f(wf);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc8[j] = fmaf(a[c], wf[j], acc8[j]);
    }
    *reinterpret_cast<float4*>(prow + h) = float4{acc8[0], acc8[1], acc8[2], acc8[3]};
    *reinterpret_cast<float4*>(prow + h + 4) = float4{acc8[4], acc8[5], acc8[6], acc8[7]};
  };
#pragma unroll
  for (int m = 0; m < PRE; ++m)
    if (8 * tid + CS * m < H) sum_store(wpre[m], 8 * tid + CS * m);
  for (int h = 8 * tid + CS * PRE; h < H; h += CS) {
    Raw8<Tin> wr[S];
#pragma unroll
    for (int c = 0; c < S; ++c) wr[c].load_w(wd + ((int64_t)e * I + s_ch[c]) * H + h);
    sum_store(wr, h);
  }
}

// The slices' partials summed per pair and weighted per token in one launch:
// out[t][h] = g_s(t) y_s(t)[h] + sum_j w_tj y_{p(t,j)}[h], y_p the sum of the
// pair's slice partials.  A block takes 64 columns of one token; its
// FLOE_RC_WAVES waves sum interleaved shares of the slices (each in slice
// order, eight loads in flight), the shares are added in wave order, then
// the k pairs in slot order as the combine does.
constexpr int FLOE_RC_WAVES = 16;

template <typename Tout>
__global__ void __launch_bounds__(FLOE_RC_WAVES * 64)
floe_reduce_combine_kernel(const float* __restrict__ part, int H, int k, int n_slices, int P_max,
                           const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
                           const uint8_t* __restrict__ exact, const float* __restrict__ y_s,
                           const float* __restrict__ g_s, Tout* __restrict__ out) {
  constexpr int B = 8, Q = FLOE_RC_WAVES;
  __shared__ float red[MOE_MAX_TOPK][Q][64];
  const int t = blockIdx.y, c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int h = blockIdx.x * 64 + c;
  // two slots at a time, so both pairs' partial loads are in flight together
  for (int j0 = 0; j0 < k; j0 += 2) {
    const int j1 = j0 + 1;
    const int p0 = row_of[(int64_t)t * k + j0];
    const int p1 = j1 < k ? row_of[(int64_t)t * k + j1] : -1;
    float s0 = 0.f, s1 = 0.f;
    for (int sl = q; sl < n_slices; sl += Q * B) {
      float v0[B], v1[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int ss = sl + Q * b;
        v0[b] = (p0 >= 0 && ss < n_slices) ? part[((int64_t)ss * P_max + p0) * H + h] : 0.f;
        v1[b] = (p1 >= 0 && ss < n_slices) ? part[((int64_t)ss * P_max + p1) * H + h] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < B; ++b) s0 += v0[b];
#pragma unroll
      for (int b = 0; b < B; ++b) s1 += v1[b];
    }
    red[j0][q][c] = s0;
    if (j1 < k) red[j1][q][c] = s1;
  }
  __syncthreads();
  if (q == 0) {
    const float gs = g_s ? g_s[t] : 1.f;
    const float ys = y_s ? y_s[(int64_t)t * H + h] : 0.f;
    float acc = gs * ys;
    for (int j = 0; j < k; ++j) {
      const int64_t o = (int64_t)t * k + j;
      if (row_of[o] < 0) continue;
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < Q; ++w) y += red[j][w][c];
      if (!exact[o]) y += ys;
      acc = fmaf(topk_w[o], y, acc);
    }
    elem<Tout>::store(out, (int64_t)t * H + h, acc);
  }
}

int floe_slices(int n_keep) {
  const int a = (n_keep + FLOE_DOWN_SLICE - 1) / FLOE_DOWN_SLICE;
  const int b = (n_keep + FLOE_GD_SLICE - 1) / FLOE_GD_SLICE;
  return a > b ? a : b;
}
int floe_max_inter() { return FLOE_MAX_INTER; }
int floe_max_hidden() { return FLOE_MAX_HIDDEN; }

template <typename Tin>
static hipError_t launch_floe_t(const moe_dims_t& d, int T, const Tin* x, const moe_weights_t& w,
                                const int32_t* offsets, const int32_t* perm, float* u,
                                int32_t* keep, float* a, float* part, float* y_perm,
                                uint32_t* flags, const Prof& pf, hipStream_t s,
                                const FloeCombine* cb) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k, nk = d.floe_keep;
  const int P = T * k;
  if (P == 0) return hipSuccess;
  hipError_t e = pf.begin(MOE_KERNEL_FLOE_UP, s);
  if constexpr (std::is_same<Tin, bf16>::value) {
    constexpr int R = FLOE_UP_BF16_RPW;
    const size_t lds = (size_t)H / 8 * 16 + (size_t)(H / 64) * 8;
    floe_up_bf16_kernel<R><<<dim3((I + 4 * R - 1) / (4 * R), P), 256, lds, s>>>(
        x, w.up_q, w.up_scale, w.up_zero, H, I, E, k, offsets, perm, u);
  } else {
    floe_up_kernel<Tin><<<dim3((I + 4 * FLOE_UP_RPW - 1) / (4 * FLOE_UP_RPW), P), 256, 0, s>>>(
        x, w.up_q, w.up_scale, w.up_zero, H, I, E, k, offsets, perm, u);
  }
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_UP, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_SELECT, s);
  floe_select_kernel<<<P, FLOE_SELECT_THREADS, 0, s>>>(u, I, nk, d.tie_margin, E, k, offsets, perm,
                                                        keep, flags);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_SELECT, s);
  if (cb) {
    // in the layer forward: gate + down per slice, then the slices' sum and
    // the weighted combine straight into the output
    const int ns = (nk + FLOE_GD_SLICE - 1) / FLOE_GD_SLICE;
    if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_GATE, s);
    constexpr int gdw = floe_gd_waves<Tin>();
    floe_gate_down_kernel<Tin, gdw><<<dim3(ns, P), gdw * 64, 0, s>>>(
        x, (const Tin*)w.w_gate, (const Tin*)w.w_down, u, H, I, nk, P, E, k, offsets, perm, keep,
        part);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_GATE, s);
    if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_DOWN, s);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_DOWN, s);
    if (e == hipSuccess) e = pf.begin(MOE_KERNEL_COMBINE, s);
    floe_reduce_combine_kernel<Tin><<<dim3(H / 64, T), FLOE_RC_WAVES * 64, 0, s>>>(
        part, H, k, ns, P, cb->row_of, cb->topk_w, cb->exact, cb->y_s, cb->g_s, (Tin*)cb->out);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_COMBINE, s);
    return e == hipSuccess ? hipGetLastError() : e;
  }
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_GATE, s);
  floe_gate_kernel<Tin><<<dim3((nk + 4 * FLOE_GATE_RPW - 1) / (4 * FLOE_GATE_RPW), P), 256, 0, s>>>(
      x, (const Tin*)w.w_gate, u, H, I, nk, E, k, offsets, perm, keep, a);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_GATE, s);
  const int ns = (nk + FLOE_DOWN_SLICE - 1) / FLOE_DOWN_SLICE;
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_FLOE_DOWN, s);
  floe_down_kernel<Tin><<<dim3((H + FLOE_DOWN_COLS - 1) / FLOE_DOWN_COLS, ns, P), FLOE_DOWN_COLS / 8, 0, s>>>(
      (const Tin*)w.w_down, a, H, I, nk, P, E, k, offsets, perm, keep, part);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_FLOE_DOWN, s);
  floe_reduce_kernel<<<dim3((H + 255) / 256, P), 256, 0, s>>>(part, H, ns, P, E, offsets, y_perm);
  return e == hipSuccess ? hipGetLastError() : e;
}

// FloE intra-expert predictor: the up projection and channel selection of the
// FloE forward, run on another hidden state (the previous layer's) for the
// pairs already permuted into `offsets` / `perm`.
hipError_t launch_floe_predict(const moe_dims_t& d, int T, const void* h, const moe_weights_t& w,
                               const int32_t* offsets, const int32_t* perm, float* u,
                               int32_t* keep, uint32_t* flags, hipStream_t s) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k, nk = d.floe_keep;
  const int P = T * k;
  if (P == 0) return hipSuccess;
  if (d.dtype == MOE_BF16) {
    constexpr int R = FLOE_UP_BF16_RPW;
    const size_t lds = (size_t)H / 8 * 16 + (size_t)(H / 64) * 8;
    floe_up_bf16_kernel<R><<<dim3((I + 4 * R - 1) / (4 * R), P), 256, lds, s>>>(
        (const bf16*)h, w.up_q, w.up_scale, w.up_zero, H, I, E, k, offsets, perm, u);
  } else {
    floe_up_kernel<float><<<dim3((I + 4 * FLOE_UP_RPW - 1) / (4 * FLOE_UP_RPW), P), 256, 0, s>>>(
        (const float*)h, w.up_q, w.up_scale, w.up_zero, H, I, E, k, offsets, perm, u);
  }
  floe_select_kernel<<<P, FLOE_SELECT_THREADS, 0, s>>>(u, I, nk, d.tie_margin, E, k, offsets, perm,
                                                        keep, flags);
  return hipGetLastError();
}

// Compact packing of the kept channels: for slot f = t*k + j with expert
// e = ids[f], rows keep[f][c] of W_gate[e] and W_down[e] (both [I][H]) are
// copied to gate_out[f][c] and down_out[f][c].  One block per (slot, group of
// FLOE_PACK_ROWS kept channels), 16 bytes per thread per row.
constexpr int FLOE_PACK_ROWS = 8;
__global__ void __launch_bounds__(256)
floe_pack_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ keep,
                 const uint4* __restrict__ wg, const uint4* __restrict__ wd, int I, int nk, int E,
                 int row_u4, uint4* __restrict__ gate_out, uint4* __restrict__ down_out) {
  const int f = blockIdx.x;
  const int e = ids[f];
  const int c0 = blockIdx.y * FLOE_PACK_ROWS, c1 = min(nk, c0 + FLOE_PACK_ROWS);
  const bool valid = (unsigned)e < (unsigned)E;
  for (int c = c0; c < c1; ++c) {
    const int ch = keep[(int64_t)f * nk + c];
    const bool ok = valid && (unsigned)ch < (unsigned)I;
    const int64_t src = ((int64_t)(ok ? e : 0) * I + (ok ? ch : 0)) * row_u4;
    const int64_t dst = ((int64_t)f * nk + c) * row_u4;
    for (int i = threadIdx.x; i < row_u4; i += blockDim.x) {
      gate_out[dst + i] = ok ? wg[src + i] : make_uint4(0u, 0u, 0u, 0u);
      down_out[dst + i] = ok ? wd[src + i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

hipError_t launch_floe_pack(const moe_dims_t& d, int T, const int32_t* ids, const int32_t* keep,
                            const void* w_gate, const void* w_down, void* gate_out,
                            void* down_out, hipStream_t s) {
  const int P = T * d.top_k, nk = d.floe_keep;
  if (P == 0) return hipSuccess;
  const int esz = d.dtype == MOE_BF16 ? 2 : 4;
  const int row_u4 = d.hidden * esz / 16;
  floe_pack_kernel<<<dim3(P, (nk + FLOE_PACK_ROWS - 1) / FLOE_PACK_ROWS), 256, 0, s>>>(
      ids, keep, (const uint4*)w_gate, (const uint4*)w_down, d.inter, nk, d.n_experts, row_u4,
      (uint4*)gate_out, (uint4*)down_out);
  return hipGetLastError();
}

hipError_t launch_floe(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                       const int32_t* offsets, const int32_t* perm, float* u,
                       int32_t* keep, float* a, float* part, float* y_perm, uint32_t* flags,
                       const Prof& pf, hipStream_t s, const FloeCombine* cb) {
  if (d.dtype == MOE_BF16)
    return launch_floe_t<bf16>(d, T, (const bf16*)x, w, offsets, perm, u, keep, a, part, y_perm,
                               flags, pf, s, cb);
  return launch_floe_t<float>(d, T, (const float*)x, w, offsets, perm, u, keep, a, part, y_perm,
                              flags, pf, s, cb);
}

}  // namespace moe
