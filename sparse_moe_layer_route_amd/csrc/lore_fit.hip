// LoRE fitting on the GPU [SPICE page, "LoRE low-rank surrogate": per
// expert, minimise ||y_e - y_shared - B_e A_e h||^2 over a calibration set,
// solved with an SVD].
//
//   targets:  R = y_e(h) - y_s(h) for the calibration rows, from the layer's
//             own expert and shared FFN kernels (one routed expert, k = 1).
//   whitening: G = h^T h / N and Z = G^-1/2 by the coupled Newton-Schulz
//             iteration (Higham, "Functions of Matrices", the Newton-Schulz
//             iteration for the matrix square root): Y0 = G / c, Z0 = I,
//             P = 3I - Z Y, Y <- Y P / 2, Z <- P Z / 2, so Y -> (G/c)^1/2 and
//             Z -> (G/c)^-1/2; c = the largest absolute row sum of G (a
//             Gershgorin bound on its largest eigenvalue) keeps the spectrum
//             of G / c in (0, 1], where the iteration converges.
//   map:      M = (R^T h / N) Z [H][H] fp32 -- the least-squares map in
//             whitened inputs; the rank-r minimiser of ||R - h W^T|| is
//             W = [M]_r Z (reduced-rank regression).  For an orthogonal
//             design (h^T h = N I) Z = I and M is the plain map.
//   factors:  the rank-r truncated SVD of M, B = U_r S_r, A = V_r^T Z, by
//             subspace iteration (Y <- M M^T Y, re-orthonormalised each half
//             step) from a caller-supplied Gaussian block, then a
//             Rayleigh-Ritz step: Bs = Q^T M, eigen-decomposition of
//             Bs Bs^T (s x s) by cyclic Jacobi rotations in one workgroup,
//             U = Q W, V^T = S^-1 W^T Bs.
//   error:    ||R - h (B A)^T||_F / ||R||_F on the calibration rows.
//
// Everything is fp32 (the calibration rows may be bf16).  The products are
// plain LDS-tiled fp32 GEMMs with arbitrary strides; the fit is a one-time
// calibration step, so these favour simplicity over peak rate.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace moe {

constexpr int FG_TILE = 64, FG_K = 16;

// C(m, n) = alpha * sum_k A(m, k) B(k, n) with A(m, k) = A[m*sam + k*sak],
// B(k, n) = B[k*sbk + n*sbn], C(m, n) = C[m*scm + n*scn].  64 x 64 output
// tile per 256-thread block, 4 x 4 per thread, k in steps of 16 through LDS.
template <typename TA, typename TB>
__global__ void __launch_bounds__(256)
fit_gemm_kernel(int M, int N, int K, float alpha, const TA* __restrict__ A, int64_t sam,
                int64_t sak, const TB* __restrict__ B, int64_t sbk, int64_t sbn,
                float* __restrict__ C, int64_t scm, int64_t scn) {
  __shared__ float As[FG_K][FG_TILE + 4];
  __shared__ float Bs[FG_K][FG_TILE + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FG_TILE, n0 = blockIdx.x * FG_TILE;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  // walk whichever index is contiguous in memory across neighbouring threads
  const bool a_k_inner = sak == 1, b_k_inner = sbk == 1;
  for (int k0 = 0; k0 < K; k0 += FG_K) {
    for (int i = tid; i < FG_TILE * FG_K; i += 256) {
      const int mm = a_k_inner ? i / FG_K : i % FG_TILE, kk = a_k_inner ? i % FG_K : i / FG_TILE;
      const int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < K) ? elem<TA>::load(A, (int64_t)gm * sam + (int64_t)gk * sak) : 0.f;
      const int nn = b_k_inner ? i / FG_K : i % FG_TILE, kb = b_k_inner ? i % FG_K : i / FG_TILE;
      const int gn = n0 + nn, gkb = k0 + kb;
      Bs[kb][nn] = (gn < N && gkb < K) ? elem<TB>::load(B, (int64_t)gkb * sbk + (int64_t)gn * sbn) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < FG_K; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < N) C[(int64_t)gm * scm + (int64_t)gn * scn] = alpha * acc[i][j];
    }
  }
}

template <typename TA, typename TB>
static void fit_gemm(int M, int N, int K, float alpha, const TA* A, int64_t sam, int64_t sak,
                     const TB* B, int64_t sbk, int64_t sbn, float* C, int64_t scm, int64_t scn,
                     hipStream_t s) {
  const dim3 grid((N + FG_TILE - 1) / FG_TILE, (M + FG_TILE - 1) / FG_TILE);
  fit_gemm_kernel<TA, TB><<<grid, 256, 0, s>>>(M, N, K, alpha, A, sam, sak, B, sbk, sbn, C, scm,
                                               scn);
}

// Sum over a 1024-thread workgroup (every thread gets the total).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

// Orthonormalises the s columns of Y, stored column after column ([s][H],
// each column contiguous), in place by classical Gram-Schmidt with one
// re-orthogonalisation pass; one 1024-thread workgroup.
// A column whose remaining norm falls below 1e-6 of its original norm is
// zeroed (the block then has numerical rank below s).
constexpr int FIT_MAX_S = 64;
__global__ void __launch_bounds__(1024) fit_orth_kernel(float* __restrict__ Y, int H, int s) {
  __shared__ float coef[FIT_MAX_S];
  __shared__ float red[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int j = 0; j < s; ++j) {
    float n0 = 0.f;
    float* yj = Y + (int64_t)j * H;
    for (int i = tid; i < H; i += 1024) n0 += yj[i] * yj[i];
    n0 = block_sum(n0, red);
    for (int pass = 0; pass < 2; ++pass) {
      // c_p = <q_p, y_j>, one wave per previous column
      for (int p = wv; p < j; p += 16) {
        float d = 0.f;
        const float* yp = Y + (int64_t)p * H;
        for (int i = lane; i < H; i += 64) d += yp[i] * yj[i];
        d = wave_sum(d);
        if (lane == 0) coef[p] = d;
      }
      __syncthreads();
      for (int i = tid; i < H; i += 1024) {
        float v = yj[i];
        for (int p = 0; p < j; ++p) v -= coef[p] * Y[(int64_t)p * H + i];
        yj[i] = v;
      }
      __syncthreads();
    }
    float nr = 0.f;
    for (int i = tid; i < H; i += 1024) nr += yj[i] * yj[i];
    nr = block_sum(nr, red);
    const float inv = (nr > 1e-12f * n0 && nr > 0.f) ? 1.f / sqrtf(nr) : 0.f;
    for (int i = tid; i < H; i += 1024) yj[i] *= inv;
    __syncthreads();
  }
}

// Symmetric eigen-decomposition of T [s][s] by cyclic Jacobi rotations (each
// rotation zeroes one off-diagonal pair: Golub & Van Loan, "Matrix
// Computations", the cyclic Jacobi method), one wave (thread i owns row and
// column i, so the rotations need only wave-level barriers).  Sweeps stop once
// the off-diagonal mass is below 1e-10 of the diagonal's (squared norms), or
// after max_sweeps.  Writes the eigenvalues in descending order to lam and
// the matching unit eigenvectors as the columns of W [s][s].
__global__ void __launch_bounds__(64)
fit_jacobi_kernel(const float* __restrict__ Tin, int s, int max_sweeps, float* __restrict__ lam,
                  float* __restrict__ W) {
  __shared__ float T[FIT_MAX_S][FIT_MAX_S + 1];
  __shared__ float V[FIT_MAX_S][FIT_MAX_S + 1];
  __shared__ float rot[2];
  __shared__ float s_off, s_diag;
  __shared__ int order[FIT_MAX_S];
  const int tid = threadIdx.x;
  for (int i = tid; i < s * s; i += 64) {
    const int r = i / s, c = i % s;
    T[r][c] = 0.5f * (Tin[r * s + c] + Tin[c * s + r]);
    V[r][c] = r == c ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    {
      float off = 0.f, dg = 0.f;
      if (tid < s)
        for (int c = 0; c < s; ++c) (tid == c ? dg : off) += T[tid][c] * T[tid][c];
      off = wave_sum(off);
      dg = wave_sum(dg);
      if (tid == 0) {
        s_off = off;
        s_diag = dg;
      }
    }
    __syncthreads();
    if (!(s_off > 1e-10f * s_diag)) break;
    for (int p = 0; p < s - 1; ++p) {
      for (int q = p + 1; q < s; ++q) {
        if (tid == 0) {
          const float apq = T[p][q];
          float c = 1.f, sn = 0.f;
          if (fabsf(apq) > 1e-30f) {
            const float th = (T[q][q] - T[p][p]) / (2.f * apq);
            const float t = (th >= 0.f ? 1.f : -1.f) / (fabsf(th) + sqrtf(th * th + 1.f));
            c = 1.f / sqrtf(t * t + 1.f);
            sn = t * c;
          }
          rot[0] = c;
          rot[1] = sn;
        }
        __syncthreads();
        const float c = rot[0], sn = rot[1];
        if (sn != 0.f) {
          // columns p, q of T and V
          if (tid < s) {
            const float tp = T[tid][p], tq = T[tid][q];
            T[tid][p] = c * tp - sn * tq;
            T[tid][q] = sn * tp + c * tq;
            const float vp = V[tid][p], vq = V[tid][q];
            V[tid][p] = c * vp - sn * vq;
            V[tid][q] = sn * vp + c * vq;
          }
          __syncthreads();
          // rows p, q of T
          if (tid < s) {
            const float tp = T[p][tid], tq = T[q][tid];
            T[p][tid] = c * tp - sn * tq;
            T[q][tid] = sn * tp + c * tq;
          }
        }
        __syncthreads();
      }
    }
  }
  // descending order of the diagonal (ties by index)
  if (tid < s) {
    const float d = T[tid][tid];
    int rank = 0;
    for (int j = 0; j < s; ++j) {
      const float e = T[j][j];
      rank += (e > d) || (e == d && j < tid);
    }
    order[rank] = tid;
  }
  __syncthreads();
  if (tid < s) lam[tid] = T[order[tid]][order[tid]];
  for (int i = tid; i < s * s; i += 64) {
    const int r = i / s, c = i % s;
    W[r * s + c] = V[r][order[c]];
  }
}

// B = U_r S_r as dtype [H][r] and fp32 from U stored by columns ([s][H]);
// sigma = sqrt(max(lam, 0)).
template <typename Tout>
__global__ void __launch_bounds__(256)
fit_b_kernel(const float* __restrict__ U, int H, int s, int r, const float* __restrict__ lam,
             float* __restrict__ Bf, Tout* __restrict__ Bout, float* __restrict__ sigma) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < r) sigma[threadIdx.x] = sqrtf(fmaxf(lam[threadIdx.x], 0.f));
  if (i >= (int64_t)H * r) return;
  const int h = (int)(i / r), j = (int)(i % r);
  const float v = U[(int64_t)j * H + h] * sqrtf(fmaxf(lam[j], 0.f));
  Bf[i] = v;
  elem<Tout>::store(Bout, i, v);
}

// V_r^T = S_r^-1 W_r^T Bs [r][H] fp32, from G = W^T Bs [s][H].
__global__ void __launch_bounds__(256)
fit_vt_kernel(const float* __restrict__ G, int H, int r, const float* __restrict__ lam,
              float* __restrict__ Vt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)r * H) return;
  const int j = (int)(i / H);
  const float sg = sqrtf(fmaxf(lam[j], 0.f));
  Vt[i] = sg > 0.f ? G[i] / sg : 0.f;
}

// c[0] = max_i sum_j |G[i][j]| over the H x H matrix G (one workgroup; a
// wave per row, rows in a fixed order per wave, then the waves' maxima).
__global__ void __launch_bounds__(1024)
fit_gersh_kernel(const float* __restrict__ G, int H, float* __restrict__ c) {
  __shared__ float red[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float m = 0.f;
  for (int i = wv; i < H; i += 16) {
    float r = 0.f;
    for (int j = lane; j < H; j += 64) r += fabsf(G[(int64_t)i * H + j]);
    m = fmaxf(m, wave_sum(r));
  }
  if (lane == 0) red[wv] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t = fmaxf(t, red[w]);
    c[0] = t;
  }
}

// Newton-Schulz start: Y = G / c (in place), Z = I.
__global__ void __launch_bounds__(256)
fit_ns_init_kernel(float* __restrict__ Y, float* __restrict__ Z, int H, const float* __restrict__ c) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * H) return;
  const float inv = c[0] > 0.f ? 1.f / c[0] : 0.f;
  Y[i] = Y[i] * inv;
  Z[i] = (i / H == i % H) ? 1.f : 0.f;
}

// P = 3I - P (in place).
__global__ void __launch_bounds__(256) fit_ns_sub_kernel(float* __restrict__ P, int H) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * H) return;
  P[i] = ((i / H == i % H) ? 3.f : 0.f) - P[i];
}

// Z = Z / sqrt(c): (G/c)^-1/2 -> G^-1/2.
__global__ void __launch_bounds__(256)
fit_ns_final_kernel(float* __restrict__ Z, int H, const float* __restrict__ c) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * H) return;
  Z[i] = c[0] > 0.f ? Z[i] / sqrtf(c[0]) : 0.f;
}

template <typename Tout>
__global__ void __launch_bounds__(256)
fit_store_kernel(const float* __restrict__ src, int64_t n, Tout* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) elem<Tout>::store(dst, i, src[i]);
}

// Partial sums of (R - P)^2 and R^2 per block, in a fixed order.
__global__ void __launch_bounds__(256)
fit_err_partial_kernel(const float* __restrict__ R, const float* __restrict__ P, int64_t n,
                       float* __restrict__ part) {
  __shared__ float red[2][4];
  float d2 = 0.f, r2 = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float d = R[i] - P[i];
    d2 = fmaf(d, d, d2);
    r2 = fmaf(R[i], R[i], r2);
  }
  d2 = wave_sum(d2);
  r2 = wave_sum(r2);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wv] = d2;
    red[1][wv] = r2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    part[2 * blockIdx.x + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

__global__ void __launch_bounds__(64)
fit_err_final_kernel(const float* __restrict__ part, int nb, float* __restrict__ err) {
  double d = 0.0, r = 0.0;
  for (int b = threadIdx.x; b < nb; b += 64) {
    d += part[2 * b];
    r += part[2 * b + 1];
  }
  for (int o = 32; o > 0; o >>= 1) {
    d += __shfl_xor(d, o, 64);
    r += __shfl_xor(r, o, 64);
  }
  if (threadIdx.x == 0) err[0] = r > 0.0 ? (float)sqrt(d / r) : 0.f;
}

// targets: R = y_perm - y_s (y_s may be null: no shared experts)
__global__ void __launch_bounds__(256)
fit_resid_kernel(const float* __restrict__ ye, const float* __restrict__ ys, int64_t n,
                 float* __restrict__ R) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) R[i] = ye[i] - (ys ? ys[i] : 0.f);
}

// offsets [E+1] and perm [N] routing every calibration row to expert e (k = 1)
__global__ void __launch_bounds__(256)
fit_route_kernel(int N, int E, int e, int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i <= E) offsets[i] = i <= e ? 0 : N;
  if (i < N) perm[i] = i;
}

constexpr int FIT_ERR_BLOCKS = 256;
// Newton-Schulz rounds: a Gershgorin-scaled start converges to fp32 accuracy
// in about 3 rounds for a nearly orthogonal design and in 10-12 rounds for
// cond(h^T h) near 35 (a Gaussian design of 2H rows); 20 leave room beyond.
constexpr int FIT_NS_ITERS = 20;

int64_t lore_fit_ws_elems(int H, int N, int r, int s) {
  auto al = [](int64_t v) { return (v + 63) & ~(int64_t)63; };
  return 6 * al((int64_t)H * H) + 2 * al((int64_t)H * s) + al((int64_t)s * H) + 2 * al((int64_t)s * s) +
         al(s) + al((int64_t)s * H) + 2 * al((int64_t)r * H) + al((int64_t)H * r) + al((int64_t)N * r) +
         al((int64_t)N * H) + al(2 * FIT_ERR_BLOCKS) + al(1);
}

template <typename Tin>
static hipError_t launch_lore_fit_t(int H, int N, const Tin* h, const float* R, int r, int s,
                                    int n_iter, const float* omega, Tin* A_out, Tin* B_out,
                                    float* sigma, float* err, float* ws, hipStream_t st) {
  auto al = [](int64_t v) { return (v + 63) & ~(int64_t)63; };
  const int64_t HH = al((int64_t)H * H);
  float* M = ws;
  float* Ya = M + HH;  // Newton-Schulz buffers; Ya starts as G
  float* Yb = Ya + HH;
  float* Za = Yb + HH;
  float* Zb = Za + HH;
  float* Pm = Zb + HH;
  float* Y = Pm + HH;
  float* Z = Y + al((int64_t)H * s);
  float* Bs = Z + al((int64_t)H * s);
  float* Tm = Bs + al((int64_t)s * H);
  float* Wv = Tm + al((int64_t)s * s);
  float* lam = Wv + al((int64_t)s * s);
  float* G = lam + al(s);
  float* Vt = G + al((int64_t)s * H);
  float* Af = Vt + al((int64_t)r * H);
  float* Bf = Af + al((int64_t)r * H);
  float* P1 = Bf + al((int64_t)H * r);
  float* P = P1 + al((int64_t)N * r);
  float* part = P + al((int64_t)N * H);
  float* cscale = part + al(2 * FIT_ERR_BLOCKS);
  const unsigned ew = (unsigned)(((int64_t)H * H + 255) / 256);
  // whitening Z = (h^T h / N)^-1/2: G(a, b) = sum_n h[n][a] h[n][b] / N
  fit_gemm<Tin, Tin>(H, H, N, 1.f / (float)N, h, 1, H, h, H, 1, Ya, H, 1, st);
  fit_gersh_kernel<<<1, 1024, 0, st>>>(Ya, H, cscale);
  fit_ns_init_kernel<<<ew, 256, 0, st>>>(Ya, Za, H, cscale);
  for (int it = 0; it < FIT_NS_ITERS; ++it) {
    // P = 3I - Z Y;  Y <- Y P / 2;  Z <- P Z / 2
    fit_gemm<float, float>(H, H, H, 1.f, Za, H, 1, Ya, H, 1, Pm, H, 1, st);
    fit_ns_sub_kernel<<<ew, 256, 0, st>>>(Pm, H);
    fit_gemm<float, float>(H, H, H, 0.5f, Ya, H, 1, Pm, H, 1, Yb, H, 1, st);
    fit_gemm<float, float>(H, H, H, 0.5f, Pm, H, 1, Za, H, 1, Zb, H, 1, st);
    std::swap(Ya, Yb);
    std::swap(Za, Zb);
  }
  fit_ns_final_kernel<<<ew, 256, 0, st>>>(Za, H, cscale);
  const float* Wh = Za;  // G^-1/2
  // M = (R^T h / N) G^-1/2: M0(a, b) = sum_n R[n][a] h[n][b] / N into Ya
  fit_gemm<float, Tin>(H, H, N, 1.f / (float)N, R, 1, H, h, H, 1, Ya, H, 1, st);
  fit_gemm<float, float>(H, H, H, 1.f, Ya, H, 1, Wh, H, 1, M, H, 1, st);
  // Y = M omega (Y, Z and U are stored by columns: element (h, j) at j*H + h)
  fit_gemm<float, float>(H, s, H, 1.f, M, H, 1, omega, s, 1, Y, 1, H, st);
  fit_orth_kernel<<<1, 1024, 0, st>>>(Y, H, s);
  for (int it = 0; it < n_iter; ++it) {
    // Z = M^T Y, orthonormalised; Y = M Z, orthonormalised
    fit_gemm<float, float>(H, s, H, 1.f, M, 1, H, Y, 1, H, Z, 1, H, st);
    fit_orth_kernel<<<1, 1024, 0, st>>>(Z, H, s);
    fit_gemm<float, float>(H, s, H, 1.f, M, H, 1, Z, 1, H, Y, 1, H, st);
    fit_orth_kernel<<<1, 1024, 0, st>>>(Y, H, s);
  }
  // Rayleigh-Ritz: Bs = Y^T M [s][H], Tm = Bs Bs^T, eigenpairs (lam, Wv)
  fit_gemm<float, float>(s, H, H, 1.f, Y, H, 1, M, H, 1, Bs, H, 1, st);
  fit_gemm<float, float>(s, s, H, 1.f, Bs, H, 1, Bs, 1, H, Tm, s, 1, st);
  fit_jacobi_kernel<<<1, 64, 0, st>>>(Tm, s, 30, lam, Wv);
  // U = Y Wv (into Z), B = U_r S_r; G = Wv^T Bs, V_r^T = S_r^-1 G_r, A = V_r^T G^-1/2
  fit_gemm<float, float>(H, s, s, 1.f, Y, 1, H, Wv, s, 1, Z, 1, H, st);
  fit_b_kernel<Tin><<<(unsigned)(((int64_t)H * r + 255) / 256), 256, 0, st>>>(Z, H, s, r, lam, Bf,
                                                                                B_out, sigma);
  fit_gemm<float, float>(r, H, s, 1.f, Wv, 1, s, Bs, H, 1, G, H, 1, st);
  fit_vt_kernel<<<(unsigned)(((int64_t)r * H + 255) / 256), 256, 0, st>>>(G, H, r, lam, Vt);
  fit_gemm<float, float>(r, H, H, 1.f, Vt, H, 1, Wh, H, 1, Af, H, 1, st);
  fit_store_kernel<Tin><<<(unsigned)(((int64_t)r * H + 255) / 256), 256, 0, st>>>(
      Af, (int64_t)r * H, A_out);
  // error of the fitted map on the calibration rows: P = (h A^T) B^T
  fit_gemm<Tin, float>(N, r, H, 1.f, h, H, 1, Af, 1, H, P1, r, 1, st);
  fit_gemm<float, float>(N, H, r, 1.f, P1, r, 1, Bf, 1, r, P, H, 1, st);
  fit_err_partial_kernel<<<FIT_ERR_BLOCKS, 256, 0, st>>>(R, P, (int64_t)N * H, part);
  fit_err_final_kernel<<<1, 64, 0, st>>>(part, FIT_ERR_BLOCKS, err);
  return hipGetLastError();
}

hipError_t launch_lore_fit(const moe_dims_t& d, int N, const void* h, const float* R, int r, int s,
                           int n_iter, const float* omega, void* A_out, void* B_out, float* sigma,
                           float* err, float* ws, hipStream_t st) {
  if (d.dtype == MOE_BF16)
    return launch_lore_fit_t<bf16>(d.hidden, N, (const bf16*)h, R, r, s, n_iter, omega,
                                   (bf16*)A_out, (bf16*)B_out, sigma, err, ws, st);
  return launch_lore_fit_t<float>(d.hidden, N, (const float*)h, R, r, s, n_iter, omega,
                                  (float*)A_out, (float*)B_out, sigma, err, ws, st);
}

hipError_t launch_fit_route(int N, int E, int e, int32_t* offsets, int32_t* perm, hipStream_t st) {
  fit_route_kernel<<<(std::max(N, E + 1) + 255) / 256, 256, 0, st>>>(N, E, e, offsets, perm);
  return hipGetLastError();
}

hipError_t launch_fit_resid(const float* ye, const float* ys, int64_t n, float* R, hipStream_t st) {
  fit_resid_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(ye, ys, n, R);
  return hipGetLastError();
}

}  // namespace moe
