// Host side of the C ABI declared in include/moe_route.h: argument checks,
// workspace carving and kernel enqueueing.  Nothing here allocates device
// memory, frees or synchronises, and every check runs before the first
// enqueue -- except moe_layer_forward_offload, which waits for the routed ids
// before it can plan the missed experts and runs the host FFN.
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <mutex>
#include <thread>

#include "common.h"

namespace moe {
hipError_t launch_route(const moe_dims_t& d, int T, const void* x, const void* w_router,
                        const uint64_t* resident, int64_t res_stride, int mode, int32_t* ids,
                        float* w, uint8_t* exact, uint32_t* flags, float* logits, float* mass,
                        const void* w_sg, float* g_s, hipStream_t s, const PermOut* po = nullptr,
                        bool* permuted = nullptr);
hipError_t launch_pack_mfma16(int G, int R, int K, const void* src, void* dst, hipStream_t s);
int64_t lore_fit_ws_elems(int H, int N, int r, int s);
hipError_t launch_lore_fit(const moe_dims_t& d, int N, const void* h, const float* R, int r, int s,
                           int n_iter, const float* omega, void* A_out, void* B_out, float* sigma,
                           float* err, float* ws, hipStream_t st);
hipError_t launch_fit_route(int N, int E, int e, int32_t* offsets, int32_t* perm, hipStream_t st);
hipError_t launch_fit_resid(const float* ye, const float* ys, int64_t n, float* R, hipStream_t st);
hipError_t launch_floe_predict(const moe_dims_t& d, int T, const void* h, const moe_weights_t& w,
                               const int32_t* offsets, const int32_t* perm, float* u,
                               int32_t* keep, uint32_t* flags, hipStream_t s);
hipError_t launch_floe_pack(const moe_dims_t& d, int T, const int32_t* ids, const int32_t* keep,
                            const void* w_gate, const void* w_down, void* gate_out,
                            void* down_out, hipStream_t s);
int64_t packed_elems(int R, int K);
hipError_t launch_prefetch_adaptive(const moe_dims_t& d, int T, const void* x, const void* w_p,
                                    const void* w_delta, const float* theta, float logit_tau,
                                    const int32_t* routed, int32_t* delta_out,
                                    uint64_t* mask_out, uint32_t* flags, int32_t* delta_star,
                                    int32_t* overlap, hipStream_t s);
hipError_t launch_prefetch(const moe_dims_t& d, int T, const void* x, const void* w_p,
                           const int32_t* delta, uint64_t* mask_out, uint32_t* flags,
                           hipStream_t s);
hipError_t launch_permute(int n_pairs, int E, const int32_t* ids, const uint8_t* exact,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* row_of,
                          int32_t* miss_offsets, int32_t* scratch, hipStream_t s);
int permute_scratch_bytes(int n_pairs, int E);
hipError_t launch_dense_ffn(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                            const int32_t* offsets, const int32_t* perm, int n_pairs_max,
                            float* act, float* y_perm, float* act_s, float* y_s, const Prof& pf,
                            hipStream_t s);
hipError_t launch_shared_gate(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                              float* g_s, hipStream_t s);
hipError_t launch_ffn_mfma(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* moffsets, const int32_t* perm,
                           const FfnBuffers& b, int routed, int shared, int lore, hipStream_t s,
                           int which);
hipError_t launch_ffn_gemm(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                           const int32_t* offsets, const int32_t* perm, bool shared, bf16* act,
                           float* y, bf16* yb, float* part, hipStream_t s, int which);
int gemm_shared_down_ksplit(const moe_dims_t& d, int T);
hipError_t launch_floe(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                       const int32_t* offsets, const int32_t* perm, float* u, int32_t* keep,
                       float* a, float* part, float* y_perm, uint32_t* flags, const Prof& pf,
                       hipStream_t s, const FloeCombine* cb);
hipError_t launch_combine(const moe_dims_t& d, int T, const float* y_perm, const int32_t* inv,
                          const float* topk_w, const uint8_t* exact, const int32_t* ids,
                          const float* y_s, const float* g_s, const float* lore_out, const void* x,
                          const void* lore_A, const void* lore_B, void* out, hipStream_t s);
hipError_t launch_combine_rows(const moe_dims_t& d, int T, const void* y_perm, bool y_bf16,
                               const int32_t* row_of, const float* topk_w, const uint8_t* exact,
                               const float* y_s, const float* g_s, void* out, hipStream_t s);
hipError_t launch_lore(const moe_dims_t& d, int T, const void* x, const int32_t* ids,
                       const uint8_t* exact, const void* lore_A, const void* lore_B,
                       float* lore_out, hipStream_t s);
int floe_slices(int n_keep);
int floe_max_inter();
int floe_max_hidden();
void offload_costs(double weight_bytes, double hidden_bytes, int tokens, double pcie_bytes_per_s,
                   double gpu_expert_s, double cpu_expert_s, double cpu_pair_s, double* fetch,
                   double* host);
void host_expert_ffn(const HostFfnArgs& a, bool bf16_weights, const void* x, const void* wg,
                     const void* wu, const void* wd);
hipError_t launch_offload_scatter(int n, int H, const int32_t* pairs, const float* y_host,
                                  const int32_t* row_of, float* y_perm, uint8_t* exact,
                                  hipStream_t s);
}  // namespace moe

using namespace moe;

namespace {

constexpr int32_t kMaxTokens = 1 << 22;

// Kernels form element offsets into token-major buffers (x, the routed and
// shared activations, y_perm) in 32 bits, so each such buffer must hold fewer
// than 2^31 elements: T * top_k * max(hidden, inter, n_shared * shared_inter).
inline bool tokens_fit(const moe_dims_t& d, int64_t T) {
  const int64_t wide = std::max<int64_t>(
      {(int64_t)d.hidden, (int64_t)d.inter, (int64_t)d.n_shared * d.shared_inter});
  return T <= kMaxTokens && T * d.top_k * wide < (int64_t(1) << 31);
}
// FloE kernels index (token, expert) pairs on a grid dimension capped at 65535
constexpr int64_t kFloeMaxPairs = 65535;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
inline bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

moe_status_t check_dims(const moe_dims_t* d) {
  if (!d) return MOE_EINVAL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_EINVAL;
  if (d->up_format != MOE_UP_DENSE && d->up_format != MOE_UP_INT2_G64) return MOE_EINVAL;
  if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->inter <= 0) return MOE_EINVAL;
  if (d->n_shared < 0 || d->shared_inter < 0 || d->lore_rank < 0) return MOE_EINVAL;
  if (!(d->tie_margin >= 0.f)) return MOE_EINVAL;
  if (d->n_experts > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK || d->top_k > d->n_experts)
    return MOE_EUNSUPPORTED;
  if (d->hidden % 64 != 0 || d->inter % 16 != 0) return MOE_EUNSUPPORTED;
  // one expert matrix is indexed with 32-bit element offsets
  if ((int64_t)d->inter * d->hidden >= (int64_t(1) << 31) ||
      (int64_t)d->shared_inter * d->hidden >= (int64_t(1) << 31))
    return MOE_EUNSUPPORTED;
  if (d->n_shared > 0 && (d->shared_inter <= 0 || d->shared_inter % 16 != 0)) return MOE_EUNSUPPORTED;
  if (d->lore_rank > MOE_MAX_LORE_RANK || d->lore_rank % 8 != 0) return MOE_EUNSUPPORTED;
  if (d->weight_layout != MOE_LAYOUT_ROWS && d->weight_layout != MOE_LAYOUT_MFMA16)
    return MOE_EINVAL;
  if (d->weight_layout == MOE_LAYOUT_MFMA16 &&
      (d->dtype != MOE_BF16 || d->up_format != MOE_UP_DENSE))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_mode(const moe_dims_t* d, moe_mode_t mode) {
  switch (mode) {
    case MOE_MODE_STANDARD:
    case MOE_MODE_STALL_FREE:
      return d->up_format == MOE_UP_DENSE ? MOE_OK : MOE_EUNSUPPORTED;
    case MOE_MODE_LORE:
      if (d->up_format != MOE_UP_DENSE || d->lore_rank == 0) return MOE_EUNSUPPORTED;
      return MOE_OK;
    case MOE_MODE_FLOE:
      if (d->up_format != MOE_UP_INT2_G64) return MOE_EUNSUPPORTED;
      if (d->floe_keep < 1 || d->floe_keep > d->inter) return MOE_EINVAL;
      if (d->inter > floe_max_inter() || d->hidden > floe_max_hidden()) return MOE_EUNSUPPORTED;
      return MOE_OK;
  }
  return MOE_EINVAL;
}

moe_status_t check_weights(const moe_dims_t* d, const moe_weights_t* w, moe_mode_t mode) {
  if (!w) return MOE_EINVAL;
  if (!ok_ptr(w->w_router) || !ok_ptr(w->w_gate) || !ok_ptr(w->w_down)) return MOE_EINVAL;
  if (mode == MOE_MODE_FLOE) {
    if (!ok_ptr(w->up_q) || !ok_ptr(w->up_scale) || !ok_ptr(w->up_zero)) return MOE_EINVAL;
  } else if (!ok_ptr(w->w_up)) {
    return MOE_EINVAL;
  }
  if (d->n_shared > 0) {
    if (!ok_ptr(w->ws_gate) || !ok_ptr(w->ws_up) || !ok_ptr(w->ws_down)) return MOE_EINVAL;
    if (d->shared_gate && !ok_ptr(w->w_shared_gate)) return MOE_EINVAL;
  }
  if (mode == MOE_MODE_LORE && (!ok_ptr(w->lore_A) || !ok_ptr(w->lore_B))) return MOE_EINVAL;
  return MOE_OK;
}

// Workspace plan for T tokens.
struct Plan {
  size_t ids, w, exact, flags, logits, offsets, moffsets, perm, inv, row_of, pscratch;  // routing + permutation
  size_t counter;                                                     // router -> permutation handoff
  size_t y_perm, y_s, g_s;                                            // FFN outputs
  size_t act, act_s;                                                  // fp32 GEMV activations
  size_t act_b, acts_b, z_b;                                          // bf16 MFMA activations
  size_t u, keep, fa, part;                                           // FloE
  size_t ys_part;                                                     // shared down k-split
  size_t total;
};

// The LDS-tiled grouped GEMM takes the routed experts once segments average
// 64 tokens or more, and the shared experts from 128 tokens on; both need the
// contraction lengths in whole 64-wide stages.
inline bool gemm_routed(const moe_dims_t& d, int T) {
  return (int64_t)T * d.top_k >= 64LL * d.n_experts && d.hidden % 64 == 0 && d.inter % 64 == 0;
}
inline bool gemm_shared(const moe_dims_t& d, int T) {
  return d.n_shared > 0 && T >= 128 && d.hidden % 64 == 0 && d.shared_inter % 64 == 0;
}

Plan make_plan(const moe_dims_t& d, int T, moe_mode_t mode) {
  Plan p{};
  const size_t P = (size_t)T * d.top_k;
  const size_t H = d.hidden, I = d.inter, S = (size_t)d.n_shared * d.shared_inter;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  p.ids = take(P * 4);
  p.w = take(P * 4);
  p.exact = take(P);
  p.flags = take((size_t)T * 4);
  p.logits = take((size_t)T * d.n_experts * 4);
  p.offsets = take((size_t)(d.n_experts + 1) * 4);
  p.moffsets = take((size_t)(d.n_experts + 1) * 4);
  p.perm = take(P * 4);
  p.pscratch = take((size_t)permute_scratch_bytes((int)P, d.n_experts));
  p.inv = take(P * 4);
  p.row_of = take(P * 4);
  p.counter = take(4);
  p.y_perm = take(P * H * 4);
  if (mode == MOE_MODE_FLOE) {
    p.u = take(P * I * 4);
    p.keep = take(P * (size_t)d.floe_keep * 4);
    p.fa = take(P * (size_t)d.floe_keep * 4);
    p.part = take((size_t)floe_slices(d.floe_keep) * P * H * 4);
    // dense shared experts beside the FloE routed experts
    if (S && d.dtype == MOE_BF16) p.acts_b = take((size_t)T * S * 2);
    if (S && d.dtype != MOE_BF16) p.act_s = take((size_t)T * S * 4);
  } else if (d.dtype == MOE_BF16) {
    p.act_b = take(P * I * 2);
    if (S) p.acts_b = take((size_t)T * S * 2);
    if (mode == MOE_MODE_LORE) p.z_b = take(P * (size_t)d.lore_rank * 2);
  } else {
    p.act = take(P * I * 4);
    if (S) p.act_s = take((size_t)T * S * 4);
  }
  if (d.n_shared > 0) {
    p.y_s = take((size_t)T * H * 4);
    p.g_s = take((size_t)T * 4);
  }
  if (mode != MOE_MODE_FLOE && d.dtype == MOE_BF16 && gemm_shared(d, T)) {
    const int ks = gemm_shared_down_ksplit(d, T);
    if (ks > 1) p.ys_part = take((size_t)ks * T * H * 4);
  }
  p.total = o;
  return p;
}

template <typename T>
inline T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Dense or FloE expert FFNs + shared experts (+ the LoRE products when
// `lore`) into the plan's buffers.  bf16 layers run on the matrix cores; fp32
// layers use the vector GEMV kernels.
hipError_t run_ffn(const moe_dims_t& d, int T, const void* x, const moe_weights_t& w,
                   moe_mode_t mode, const int32_t* offsets, const int32_t* moffsets,
                   const int32_t* perm, float* y_perm, float* y_s, int32_t* keep, uint32_t* flags,
                   void* ws, const Plan& p, int lore, const Prof& pf, hipStream_t s,
                   bool y_bf16 = false, bool shared_apart = false,
                   const FloeCombine* floe_cb = nullptr) {
  if (mode == MOE_MODE_FLOE) {
    hipError_t e = hipSuccess;
    if (d.n_shared > 0) {
      // the shared experts are dense: the same kernels as the other modes,
      // shared segments only
      if (d.dtype == MOE_BF16) {
        FfnBuffers sb{};
        sb.acts = at<bf16>(ws, p.acts_b);
        sb.ys = y_s;
        e = launch_ffn_mfma(d, T, x, w, offsets, moffsets, perm, sb, 0, 1, 0, s, 1);
        if (e == hipSuccess) e = launch_ffn_mfma(d, T, x, w, offsets, moffsets, perm, sb, 0, 1, 0, s, 2);
      } else {
        e = launch_dense_ffn(d, T, x, w, offsets, perm, 0, nullptr, y_perm, at<float>(ws, p.act_s),
                             y_s, Prof{}, s);
      }
    }
    if (e == hipSuccess)
      e = launch_floe(d, T, x, w, offsets, perm, at<float>(ws, p.u), keep, at<float>(ws, p.fa),
                      at<float>(ws, p.part), y_perm, flags, pf, s, floe_cb);
    return e;
  }
  if (d.dtype != MOE_BF16)
    return launch_dense_ffn(d, T, x, w, offsets, perm, T * d.top_k, at<float>(ws, p.act), y_perm,
                            d.n_shared > 0 ? at<float>(ws, p.act_s) : nullptr, y_s, pf, s);
  const bool sh = d.n_shared > 0;
  FfnBuffers b{};
  b.act = at<bf16>(ws, p.act_b);
  b.acts = sh ? at<bf16>(ws, p.acts_b) : nullptr;
  b.z = lore ? at<bf16>(ws, p.z_b) : nullptr;
  b.y = y_perm;
  b.ys = y_s;
  const bool g_r = gemm_routed(d, T), g_s = gemm_shared(d, T);
  auto stage = [&](int which) {
    hipError_t r = launch_ffn_mfma(d, T, x, w, offsets, moffsets, perm, b, !g_r, !g_s, lore, s, which);
    if (r == hipSuccess && g_r)
      r = launch_ffn_gemm(d, T, x, w, offsets, perm, false, b.act, y_perm,
                          y_bf16 ? (bf16*)y_perm : nullptr, nullptr, s, which);
    if (r == hipSuccess && g_s && !shared_apart)
      r = launch_ffn_gemm(d, T, x, w, nullptr, nullptr, true, b.acts, y_s, nullptr,
                          p.ys_part ? at<float>(ws, p.ys_part) : nullptr, s, which);
    return r;
  };
  hipError_t e = pf.begin(MOE_KERNEL_EXPERT_GATE_UP, s);
  if (e == hipSuccess) e = stage(1);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_GATE_UP, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_EXPERT_DOWN, s);
  if (e == hipSuccess) e = stage(2);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_EXPERT_DOWN, s);
  return e;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or mode";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status_t moe_workspace_size(const moe_dims_t* dims, int32_t T, moe_mode_t mode, size_t* bytes) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_mode(dims, mode)) != MOE_OK) return st;
  if (!bytes || T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  *bytes = make_plan(*dims, T, mode).total;
  return MOE_OK;
}

moe_status_t moe_route(const moe_dims_t* dims, int32_t T, const void* x, const void* w_router,
                       const uint64_t* resident, int64_t resident_stride, moe_mode_t mode,
                       int32_t* topk_ids, float* topk_w, uint8_t* exact, uint32_t* flags,
                       float* logits, float* mass_opt, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (mode < MOE_MODE_STANDARD || mode > MOE_MODE_FLOE) return MOE_EINVAL;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_ptr(topk_ids) || !ok_ptr(topk_w) || !ok_ptr(exact) ||
      !ok_ptr(flags) || !ok_ptr(logits) || !ok_opt(mass_opt))
    return MOE_EINVAL;
  const bool needs_mask = mode == MOE_MODE_LORE || mode == MOE_MODE_STALL_FREE;
  if (needs_mask && (!ok_ptr(resident) || (resident_stride != 0 && resident_stride != 1)))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_route(*dims, T, x, w_router, resident, resident_stride, mode, topk_ids,
                                 topk_w, exact, flags, logits, mass_opt, nullptr, nullptr,
                                 (hipStream_t)stream));
}

moe_status_t moe_prefetch_mask(const moe_dims_t* dims, int32_t T, const void* x,
                               const void* w_prefetch, const int32_t* delta, uint64_t* mask_out,
                               uint32_t* flags, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(w_prefetch) || !ok_ptr(delta) || !ok_ptr(mask_out) || !ok_ptr(flags))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_prefetch(*dims, T, x, w_prefetch, delta, mask_out, flags,
                                    (hipStream_t)stream));
}

moe_status_t moe_pack_size(int32_t groups, int32_t rows, int32_t cols, size_t* bytes) {
  if (!bytes || groups <= 0 || rows <= 0 || cols <= 0 || cols % 8 != 0) return MOE_EINVAL;
  *bytes = (size_t)groups * (size_t)packed_elems(rows, cols) * 2;
  return MOE_OK;
}

moe_status_t moe_pack_weights(int32_t groups, int32_t rows, int32_t cols, const void* src,
                              void* dst, void* stream) {
  if (groups <= 0 || rows <= 0 || cols <= 0 || cols % 8 != 0) return MOE_EINVAL;
  if (!ok_ptr(src) || !ok_ptr(dst)) return MOE_EINVAL;
  const size_t sb = (size_t)groups * rows * cols * 2;
  const size_t db = (size_t)groups * (size_t)packed_elems(rows, cols) * 2;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + db && d0 < s0 + sb) return MOE_EINVAL;  // overlap
  return hip_status(launch_pack_mfma16(groups, rows, cols, src, dst, (hipStream_t)stream));
}

moe_status_t moe_prefetch_adaptive(const moe_dims_t* dims, int32_t T, const void* x,
                                   const void* w_prefetch, const void* w_delta,
                                   const float* theta, float tau, const int32_t* topk_ids_opt,
                                   int32_t* delta_out, uint64_t* mask_out, uint32_t* flags,
                                   int32_t* delta_star_opt, int32_t* overlap_opt, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (T < 0 || !(tau > 0.f && tau < 1.f)) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(w_prefetch) || !ok_ptr(w_delta) || !ok_ptr(theta) ||
      !ok_ptr(delta_out) || !ok_ptr(mask_out) || !ok_ptr(flags))
    return MOE_EINVAL;
  if (!ok_opt(topk_ids_opt) || !ok_opt(delta_star_opt) || !ok_opt(overlap_opt)) return MOE_EINVAL;
  // the diagnostics need the router's choices, and come together
  if ((delta_star_opt != nullptr) != (overlap_opt != nullptr)) return MOE_EINVAL;
  if ((delta_star_opt != nullptr) != (topk_ids_opt != nullptr)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const float lt = (float)std::log((double)tau / (1.0 - (double)tau));
  return hip_status(launch_prefetch_adaptive(*dims, T, x, w_prefetch, w_delta, theta, lt,
                                             topk_ids_opt, delta_out, mask_out, flags,
                                             delta_star_opt, overlap_opt, (hipStream_t)stream));
}

moe_status_t moe_permute(int32_t T, int32_t k, int32_t E, const int32_t* topk_ids,
                         const uint8_t* exact, int32_t* expert_offsets, int32_t* perm, int32_t* inv,
                         void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || E <= 0) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || T > kMaxTokens) return MOE_EUNSUPPORTED;
  if (!ok_ptr(topk_ids) || !ok_ptr(exact) || !ok_ptr(expert_offsets) || !ok_ptr(perm) ||
      !ok_ptr(inv))
    return MOE_EINVAL;
  const size_t need = (size_t)permute_scratch_bytes(T * k, E);
  if (need > 0 && !ok_ptr(ws)) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  return hip_status(launch_permute(T * k, E, topk_ids, exact, expert_offsets, perm, inv, nullptr,
                                   nullptr, need > 0 ? (int32_t*)ws : nullptr, (hipStream_t)stream));
}

moe_status_t moe_expert_ffn(const moe_dims_t* dims, int32_t T, const void* x,
                            const moe_weights_t* w, moe_mode_t mode, const int32_t* expert_offsets,
                            const int32_t* perm, float* y_perm, float* y_shared, float* shared_gate,
                            int32_t* floe_keep_opt, uint32_t* flags_opt, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_mode(dims, mode)) != MOE_OK) return st;
  if ((st = check_weights(dims, w, mode)) != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(expert_offsets) || !ok_ptr(perm) || !ok_ptr(y_perm) || !ok_ptr(ws))
    return MOE_EINVAL;
  if (dims->n_shared > 0 && (!ok_ptr(y_shared) || !ok_ptr(shared_gate))) return MOE_EINVAL;
  if (!ok_opt(floe_keep_opt) || !ok_opt(flags_opt)) return MOE_EINVAL;
  if (mode == MOE_MODE_FLOE && !flags_opt) return MOE_EINVAL;
  if (mode == MOE_MODE_FLOE && (int64_t)T * dims->top_k > kFloeMaxPairs) return MOE_EUNSUPPORTED;
  const Plan p = make_plan(*dims, T, mode);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  int32_t* keep = floe_keep_opt ? floe_keep_opt : at<int32_t>(ws, p.keep);
  hipError_t e = run_ffn(*dims, T, x, *w, mode, expert_offsets, nullptr, perm, y_perm, y_shared, keep,
                         flags_opt, ws, p, 0, Prof{}, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_shared_gate(*dims, T, x, *w, shared_gate, (hipStream_t)stream);
  return hip_status(e);
}

moe_status_t moe_floe_predict(const moe_dims_t* dims, int32_t T, const void* h_prev,
                              const moe_weights_t* w, const int32_t* topk_ids, int32_t* keep_out,
                              uint32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_mode(dims, MOE_MODE_FLOE)) != MOE_OK) return st;
  if (!w || !ok_ptr(w->up_q) || !ok_ptr(w->up_scale) || !ok_ptr(w->up_zero)) return MOE_EINVAL;
  if (T < 0) return MOE_EINVAL;
  if ((int64_t)T * dims->top_k > kFloeMaxPairs) return MOE_EUNSUPPORTED;
  if (!ok_ptr(h_prev) || !ok_ptr(topk_ids) || !ok_ptr(keep_out) || !ok_ptr(flags) || !ok_ptr(ws))
    return MOE_EINVAL;
  const Plan p = make_plan(*dims, T, MOE_MODE_FLOE);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const int P = T * dims->top_k;
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* perm = at<int32_t>(ws, p.perm);
  hipError_t e = launch_permute(P, dims->n_experts, topk_ids, nullptr, offsets, perm,
                                at<int32_t>(ws, p.inv), at<int32_t>(ws, p.row_of),
                                at<int32_t>(ws, p.moffsets), at<int32_t>(ws, p.pscratch), s);
  if (e == hipSuccess)
    e = launch_floe_predict(*dims, T, h_prev, *w, offsets, perm, at<float>(ws, p.u), keep_out,
                            flags, s);
  return hip_status(e);
}

moe_status_t moe_floe_pack(const moe_dims_t* dims, int32_t T, const int32_t* topk_ids,
                           const int32_t* keep, const void* w_gate, const void* w_down,
                           void* gate_out, void* down_out, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_mode(dims, MOE_MODE_FLOE)) != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if ((int64_t)T * dims->top_k > kFloeMaxPairs) return MOE_EUNSUPPORTED;
  if (!ok_ptr(topk_ids) || !ok_ptr(keep) || !ok_ptr(w_gate) || !ok_ptr(w_down) ||
      !ok_ptr(gate_out) || !ok_ptr(down_out))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_floe_pack(*dims, T, topk_ids, keep, w_gate, w_down, gate_out, down_out,
                                     (hipStream_t)stream));
}

moe_status_t moe_lore_targets(const moe_dims_t* dims, int32_t N, const void* h_cal,
                              const moe_weights_t* w, int32_t expert, float* resid_out, void* ws,
                              size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->up_format != MOE_UP_DENSE) return MOE_EUNSUPPORTED;
  moe_dims_t d1 = *dims;
  d1.top_k = 1;  // every calibration row goes to the one expert
  if ((st = check_weights(&d1, w, MOE_MODE_STANDARD)) != MOE_OK) return st;
  if (N < 0 || expert < 0 || expert >= dims->n_experts) return MOE_EINVAL;
  if (!tokens_fit(*dims, N)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(h_cal) || !ok_ptr(resid_out) || !ok_ptr(ws)) return MOE_EINVAL;
  const Plan p = make_plan(d1, N, MOE_MODE_STANDARD);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (N == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* perm = at<int32_t>(ws, p.perm);
  float* ye = at<float>(ws, p.y_perm);
  float* ys = d1.n_shared > 0 ? at<float>(ws, p.y_s) : nullptr;
  hipError_t e = launch_fit_route(N, d1.n_experts, expert, offsets, perm, s);
  if (e == hipSuccess)
    e = run_ffn(d1, N, h_cal, *w, MOE_MODE_STANDARD, offsets, at<int32_t>(ws, p.moffsets), perm, ye,
                ys, nullptr, nullptr, ws, p, 0, Prof{}, s);
  if (e == hipSuccess) e = launch_fit_resid(ye, ys, (int64_t)N * d1.hidden, resid_out, s);
  return hip_status(e);
}

moe_status_t moe_lore_fit_size(int32_t hidden, int32_t N, int32_t rank, int32_t cols,
                               size_t* bytes) {
  if (!bytes || hidden <= 0 || N <= 0 || rank < 1 || cols < rank || cols > 64 || cols > hidden)
    return MOE_EINVAL;
  *bytes = (size_t)lore_fit_ws_elems(hidden, N, rank, cols) * 4;
  return MOE_OK;
}

moe_status_t moe_lore_fit(const moe_dims_t* dims, int32_t N, const void* h_cal,
                          const float* resid, int32_t rank, int32_t cols, int32_t n_iter,
                          const float* omega, void* lore_A_out, void* lore_B_out,
                          float* sigma_out, float* err_out, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (N <= 0 || rank < 1 || cols < rank || cols > 64 || cols > dims->hidden || n_iter < 0 ||
      n_iter > 1000)
    return MOE_EINVAL;
  if (!tokens_fit(*dims, N)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(h_cal) || !ok_ptr(resid) || !ok_ptr(omega) || !ok_ptr(lore_A_out) ||
      !ok_ptr(lore_B_out) || !ok_ptr(sigma_out) || !ok_ptr(err_out) || !ok_ptr(ws))
    return MOE_EINVAL;
  if (ws_bytes < (size_t)lore_fit_ws_elems(dims->hidden, N, rank, cols) * 4) return MOE_EWORKSPACE;
  return hip_status(launch_lore_fit(*dims, N, h_cal, resid, rank, cols, n_iter, omega, lore_A_out,
                                    lore_B_out, sigma_out, err_out, (float*)ws,
                                    (hipStream_t)stream));
}

moe_status_t moe_lore_surrogate(const moe_dims_t* dims, int32_t T, const void* x,
                                const int32_t* topk_ids, const uint8_t* exact, const void* lore_A,
                                const void* lore_B, float* lore_out, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->lore_rank == 0) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(topk_ids) || !ok_ptr(exact) || !ok_ptr(lore_A) || !ok_ptr(lore_B) ||
      !ok_ptr(lore_out))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_lore(*dims, T, x, topk_ids, exact, lore_A, lore_B, lore_out,
                                (hipStream_t)stream));
}

moe_status_t moe_combine(const moe_dims_t* dims, int32_t T, const float* y_perm, const int32_t* inv,
                         const float* topk_w, const uint8_t* exact, const float* y_shared,
                         const float* shared_gate, const float* lore_out, void* out, void* stream) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (!ok_ptr(y_perm) || !ok_ptr(inv) || !ok_ptr(topk_w) || !ok_ptr(exact) || !ok_ptr(out) ||
      !ok_opt(y_shared) || !ok_opt(shared_gate) || !ok_opt(lore_out))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_combine(*dims, T, y_perm, inv, topk_w, exact, nullptr, y_shared,
                                   shared_gate, lore_out, nullptr, nullptr, nullptr, out,
                                   (hipStream_t)stream));
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;

// Side stream of the shared experts' separate launches: one non-blocking
// stream at the default priority and two events per GPU, made on that GPU's
// first call that needs them and kept until the process ends.  `mu`
// serialises the fork and join of concurrent calls on one GPU: each call's
// side-stream wait must see its own fork record.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

SideStream* side_stream() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream& sd = g_side[dev];
  if (!sd.s) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    sd.fork = f;
    sd.join = j;
    sd.s = st;
  }
  return &sd;
}

// Argument checks shared by moe_layer_forward and its allocation-free
// variant (everything except the workspace).
moe_status_t check_forward(const moe_dims_t* dims, int32_t T, const void* x,
                           const moe_weights_t* w, const uint64_t* resident,
                           int64_t resident_stride, moe_mode_t mode, const void* out,
                           const moe_debug_t* dbg) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_mode(dims, mode)) != MOE_OK) return st;
  if ((st = check_weights(dims, w, mode)) != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  if (mode == MOE_MODE_FLOE && (int64_t)T * dims->top_k > kFloeMaxPairs) return MOE_EUNSUPPORTED;
  if (!ok_ptr(x) || !ok_ptr(out)) return MOE_EINVAL;
  const bool needs_mask = mode == MOE_MODE_LORE || mode == MOE_MODE_STALL_FREE;
  if (needs_mask && (!ok_ptr(resident) || (resident_stride != 0 && resident_stride != 1)))
    return MOE_EINVAL;
  if (dbg) {
    if (!ok_opt(dbg->topk_ids) || !ok_opt(dbg->topk_w) || !ok_opt(dbg->exact) ||
        !ok_opt(dbg->flags) || !ok_opt(dbg->logits) || !ok_opt(dbg->mass) ||
        !ok_opt(dbg->expert_offsets) || !ok_opt(dbg->perm) || !ok_opt(dbg->floe_keep))
      return MOE_EINVAL;
  }
  return MOE_OK;
}

// The forward after its checks, on the workspace `ws` laid out by plan p.
moe_status_t layer_forward_impl(const moe_dims_t* dims, int32_t T, const void* x,
                                const moe_weights_t* w, const uint64_t* resident,
                                int64_t resident_stride, moe_mode_t mode, void* out,
                                const moe_debug_t* dbg, void* ws, const Plan& p, void* stream,
                                bool allow_side) {
  const moe_dims_t& d = *dims;
  hipStream_t s = (hipStream_t)stream;
  const int k = d.top_k, E = d.n_experts, P = T * k;
  int32_t* ids = at<int32_t>(ws, p.ids);
  float* wts = at<float>(ws, p.w);
  uint8_t* exact = at<uint8_t>(ws, p.exact);
  uint32_t* flags = at<uint32_t>(ws, p.flags);
  float* logits = (dbg && dbg->logits) ? dbg->logits : at<float>(ws, p.logits);
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* perm = at<int32_t>(ws, p.perm);
  int32_t* inv = at<int32_t>(ws, p.inv);
  int32_t* row_of = at<int32_t>(ws, p.row_of);
  int32_t* moffsets = at<int32_t>(ws, p.moffsets);
  float* y_perm = at<float>(ws, p.y_perm);
  float* y_s = d.n_shared > 0 ? at<float>(ws, p.y_s) : nullptr;
  float* g_s = d.n_shared > 0 ? at<float>(ws, p.g_s) : nullptr;
  int32_t* keep = (mode == MOE_MODE_FLOE) ? at<int32_t>(ws, p.keep) : nullptr;
  const bool lore = mode == MOE_MODE_LORE;
  // bf16: LoRE products run as extra tiles of the FFN kernels and the combine
  // reads rows; fp32: the combine computes LoRE itself.
  const bool mfma = d.dtype == MOE_BF16 && mode != MOE_MODE_FLOE;

  Prof pf;
  if (dbg) {
    pf.id = dbg->prof_kernel;
    pf.start = (hipEvent_t)dbg->prof_start;
    pf.stop = (hipEvent_t)dbg->prof_stop;
  }
  // Shared experts with launches of their own depend on x alone: they run on
  // the side stream from the start of the call, beside the routing and the
  // routed experts, and join before the combine.
  // (Measured at the Qwen2-57B-shaped 256 tokens: forking both shared GEMMs
  // here beats serial launches by about 3% in STANDARD mode and 16% in LoRE
  // mode, and beats holding the shared down GEMM back until the routed
  // gate/up launch, or running it on the caller's stream after the routed
  // down launch.)
  const bool apart = mfma && gemm_shared(d, T);
  SideStream* sd = (apart && allow_side) ? side_stream() : nullptr;
  std::unique_lock<std::mutex> side_lock;
  hipError_t e = hipSuccess;
  if (sd) {
    side_lock = std::unique_lock<std::mutex>(sd->mu);
    e = hipEventRecord(sd->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
    if (e == hipSuccess) e = pf.begin(MOE_KERNEL_SHARED_FFN, sd->s);
    for (int which = 1; which <= 2 && e == hipSuccess; ++which)
      e = launch_ffn_gemm(d, T, x, *w, nullptr, nullptr, true, at<bf16>(ws, p.acts_b), y_s,
                          nullptr, p.ys_part ? at<float>(ws, p.ys_part) : nullptr, sd->s, which);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_SHARED_FFN, sd->s);
    if (e == hipSuccess) e = hipEventRecord(sd->join, sd->s);
  } else {
    // no separate shared launches: the bracket is empty
    e = pf.begin(MOE_KERNEL_SHARED_FFN, s);
    if (e == hipSuccess) e = pf.end(MOE_KERNEL_SHARED_FFN, s);
  }
  // small batches are permuted by the router's top-k launch itself
  const PermOut po{at<int32_t>(ws, p.counter), offsets, perm, inv, row_of, moffsets};
  bool permuted = false;
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_ROUTE, s);
  if (e == hipSuccess)
    e = launch_route(d, T, x, w->w_router, resident, resident_stride, mode, ids, wts, exact, flags,
                     logits, dbg ? dbg->mass : nullptr,
                     d.shared_gate ? w->w_shared_gate : nullptr, g_s, s, &po, &permuted);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_ROUTE, s);
  if (e == hipSuccess) e = pf.begin(MOE_KERNEL_PERMUTE, s);
  if (e == hipSuccess && !permuted)
    e = launch_permute(P, E, ids, exact, offsets, perm, inv, row_of, moffsets,
                       at<int32_t>(ws, p.pscratch), s);
  if (e == hipSuccess) e = pf.end(MOE_KERNEL_PERMUTE, s);
  // When every expert row comes from the grouped GEMM (no LoRE rows), the
  // rows are kept as bf16: the combine sums them in fp32 and the bytes between
  // the two launches halve.
  const bool y_bf16 = mfma && !lore && gemm_routed(d, T);
  // FloE: the weighted combine is the last step of the FloE launches
  const FloeCombine fcb{row_of, wts, exact, y_s, g_s, out};
  const bool floe = mode == MOE_MODE_FLOE;
  if (e == hipSuccess)
    e = run_ffn(d, T, x, *w, mode, offsets, moffsets, perm, y_perm, y_s, keep, flags, ws, p,
                mfma && lore, pf, s, y_bf16, sd != nullptr, floe ? &fcb : nullptr);
  if (e == hipSuccess && sd) e = hipStreamWaitEvent(s, sd->join, 0);
  if (e == hipSuccess && !floe) e = pf.begin(MOE_KERNEL_COMBINE, s);
  if (e == hipSuccess && !floe) {
    if (mfma)
      e = launch_combine_rows(d, T, y_perm, y_bf16, row_of, wts, exact, y_s, g_s, out, s);
    else
      e = launch_combine(d, T, y_perm, inv, wts, exact, ids, y_s, g_s, nullptr, x,
                         lore ? w->lore_A : nullptr, lore ? w->lore_B : nullptr, out, s);
  }
  if (e == hipSuccess && !floe) e = pf.end(MOE_KERNEL_COMBINE, s);
  if (e == hipSuccess && dbg) {
    auto cp = [&](void* dst, const void* src, size_t bytes) {
      if (dst && e == hipSuccess) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
    };
    cp(dbg->topk_ids, ids, (size_t)P * 4);
    cp(dbg->topk_w, wts, (size_t)P * 4);
    cp(dbg->exact, exact, (size_t)P);
    cp(dbg->flags, flags, (size_t)T * 4);
    cp(dbg->expert_offsets, offsets, (size_t)(E + 1) * 4);
    cp(dbg->perm, perm, (size_t)P * 4);
    if (keep) cp(dbg->floe_keep, keep, (size_t)P * d.floe_keep * 4);
  }
  return hip_status(e);
}

// Scratch memory of moe_layer_forward_noalloc: one array per GPU the library
// runs on, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns, looked up once
// per device on that device's first call and kept here.
constexpr size_t kNoallocBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoallocBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr on a HIP error.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status_t moe_layer_forward(const moe_dims_t* dims, int32_t T, const void* x,
                               const moe_weights_t* w, const uint64_t* resident,
                               int64_t resident_stride, moe_mode_t mode, void* out,
                               const moe_debug_t* dbg, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_forward(dims, T, x, w, resident, resident_stride, mode, out, dbg);
  if (st != MOE_OK) return st;
  if (!ok_ptr(ws)) return MOE_EINVAL;
  const Plan p = make_plan(*dims, T, mode);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  return layer_forward_impl(dims, T, x, w, resident, resident_stride, mode, out, dbg, ws, p,
                            stream, true);
}

moe_status_t moe_layer_forward_noalloc(const moe_dims_t* dims, int32_t T, const void* x,
                                       const moe_weights_t* w, const uint64_t* resident,
                                       int64_t resident_stride, moe_mode_t mode, void* out,
                                       void* stream) {
  moe_status_t st = check_forward(dims, T, x, w, resident, resident_stride, mode, out, nullptr);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(*dims, T, mode);
  if (p.total > kNoallocBytes) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  // No workspace region has to start at zero: the one counter the router's
  // launches share is zeroed by the first of them on every call.
  void* ws = noalloc_scratch();
  if (!ws) return MOE_EHIP;
  return layer_forward_impl(dims, T, x, w, resident, resident_stride, mode, out, nullptr, ws, p,
                            stream, false);
}

}  // extern "C"

// ---- exact execution of missed experts: fetch or host FFN -------------------

namespace {

inline size_t elem_bytes(const moe_dims_t& d) { return d.dtype == MOE_BF16 ? 2 : 4; }

moe_status_t check_cost(const moe_offload_cost_t* c) {
  if (!c) return MOE_EINVAL;
  if (!(c->pcie_bytes_per_s > 0.0) || !(c->gpu_expert_s >= 0.0) || !(c->cpu_expert_s >= 0.0) ||
      !(c->cpu_pair_s >= 0.0) || std::isinf(c->pcie_bytes_per_s))
    return MOE_EINVAL;
  return MOE_OK;
}

// The cost rule over every expert (tokens, resident and cost checked).
// Queue-aware: experts by decreasing pair count, each side's cost raised by
// the time already committed to it.
void offload_decide(const moe_dims_t& d, const int32_t* tokens, uint64_t resident,
                    const moe_offload_cost_t& c, uint8_t* decision) {
  const double eb = (double)elem_bytes(d);
  const double w_bytes = 3.0 * d.inter * (double)d.hidden * eb, h_bytes = d.hidden * eb;
  int order[MOE_MAX_EXPERTS];
  int m = 0;
  for (int e = 0; e < d.n_experts; ++e) {
    decision[e] = MOE_OFFLOAD_NONE;
    if (tokens[e] > 0 && !((resident >> e) & 1ull)) order[m++] = e;
  }
  if (c.queue_aware)
    std::stable_sort(order, order + m, [&](int a, int b) { return tokens[a] > tokens[b]; });
  double link = 0.0, cpu = 0.0;
  for (int i = 0; i < m; ++i) {
    const int e = order[i];
    double fetch, host;
    offload_costs(w_bytes, h_bytes, tokens[e], c.pcie_bytes_per_s, c.gpu_expert_s, c.cpu_expert_s,
                  c.cpu_pair_s, &fetch, &host);
    if (c.queue_aware) {
      fetch += link;
      host += cpu;
    }
    if (fetch < host) {
      decision[e] = MOE_OFFLOAD_FETCH;
      link = fetch;
    } else {
      decision[e] = MOE_OFFLOAD_HOST;
      cpu = host;
    }
  }
}

// Extra device buffers (after the standard plan) and the host workspace.
struct OffloadPlan {
  Plan dev;
  size_t d_y, d_pairs, d_total;
  size_t ids, x, exact, pairs, tok, gexp, gstart, done, tokens, dec, xf, act, y, h_total;
};

OffloadPlan make_offload_plan(const moe_dims_t& d, int T) {
  OffloadPlan p{};
  p.dev = make_plan(d, T, MOE_MODE_STANDARD);
  const size_t P = (size_t)T * d.top_k, H = d.hidden, I = d.inter, E = d.n_experts;
  size_t o = p.dev.total;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  p.d_y = take(P * H * 4);
  p.d_pairs = take(P * 4);
  p.d_total = o;
  o = 0;
  p.ids = take(P * 4);
  p.x = take((size_t)T * H * elem_bytes(d));
  p.exact = take(P);
  p.pairs = take(P * 4);
  p.tok = take(P * 4);
  p.gexp = take(E * 4);
  p.gstart = take((E + 1) * 4);
  p.done = take(E * 4);
  p.tokens = take(E * 4);
  p.dec = take(E);
  p.xf = take(P * H * 4);
  p.act = take(P * I * 4);
  p.y = take(P * H * 4);
  p.h_total = o;
  return p;
}

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

extern "C" {

moe_status_t moe_offload_plan(const moe_dims_t* dims, const int32_t* tokens,
                              const uint64_t* resident, const moe_offload_cost_t* cost,
                              uint8_t* decision_out) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if ((st = check_cost(cost)) != MOE_OK) return st;
  if (!tokens || !resident || !decision_out) return MOE_EINVAL;
  for (int e = 0; e < dims->n_experts; ++e)
    if (tokens[e] < 0) return MOE_EINVAL;
  offload_decide(*dims, tokens, *resident, *cost, decision_out);
  return MOE_OK;
}

moe_status_t moe_offload_workspace_size(const moe_dims_t* dims, int32_t T, size_t* device_bytes,
                                        size_t* host_bytes) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (T < 0 || !device_bytes || !host_bytes) return MOE_EINVAL;
  if (!tokens_fit(*dims, T)) return MOE_EUNSUPPORTED;
  const OffloadPlan p = make_offload_plan(*dims, T);
  *device_bytes = p.d_total;
  *host_bytes = p.h_total;
  return MOE_OK;
}

// host workspace of moe_host_expert_ffn: grouped pairs, counters, scratch
struct HostFfnPlan {
  size_t order, tok, gexp, gstart, done, cnt, xf, act, y, total;
};

HostFfnPlan make_host_ffn_plan(const moe_dims_t& d, int n) {
  HostFfnPlan p{};
  const size_t N = (size_t)std::max(n, 0), E = d.n_experts;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  p.order = take(N * 4);
  p.tok = take(N * 4);
  p.gexp = take(E * 4);
  p.gstart = take((E + 1) * 4);
  p.done = take(E * 4);
  p.cnt = take(E * 4);
  p.xf = take(N * d.hidden * 4);
  p.act = take(N * d.inter * 4);
  p.y = take(N * d.hidden * 4);
  p.total = o;
  return p;
}

inline int host_threads(int32_t t) {
  return t > 0 ? t : (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
}

moe_status_t moe_host_ffn_workspace_size(const moe_dims_t* dims, int32_t n, size_t* bytes) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (n < 0 || !bytes) return MOE_EINVAL;
  *bytes = make_host_ffn_plan(*dims, n).total;
  return MOE_OK;
}

moe_status_t moe_host_expert_ffn(const moe_dims_t* dims, int32_t T, const void* x,
                                 const moe_weights_t* host_w, int32_t n, const int32_t* tok,
                                 const int32_t* expert, int32_t threads, float* y_out,
                                 void* host_ws, size_t host_ws_bytes) {
  moe_status_t st = check_dims(dims);
  if (st != MOE_OK) return st;
  if (dims->up_format != MOE_UP_DENSE || dims->weight_layout != MOE_LAYOUT_ROWS)
    return MOE_EUNSUPPORTED;
  if (T < 0 || n < 0) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (!x || !host_w || !host_w->w_gate || !host_w->w_up || !host_w->w_down || !tok || !expert ||
      !y_out || !host_ws || !aligned16(host_ws))
    return MOE_EINVAL;
  const moe_dims_t& d = *dims;
  const HostFfnPlan p = make_host_ffn_plan(d, n);
  if (host_ws_bytes < p.total) return MOE_EWORKSPACE;
  for (int i = 0; i < n; ++i)
    if (tok[i] < 0 || tok[i] >= T || expert[i] < 0 || expert[i] >= d.n_experts) return MOE_EINVAL;
  // stable grouping of the pairs by expert
  int32_t* cnt = at<int32_t>(host_ws, p.cnt);
  int32_t* gexp = at<int32_t>(host_ws, p.gexp);
  int32_t* gstart = at<int32_t>(host_ws, p.gstart);
  int32_t* order = at<int32_t>(host_ws, p.order);
  int32_t* gtok = at<int32_t>(host_ws, p.tok);
  for (int e = 0; e < d.n_experts; ++e) cnt[e] = 0;
  for (int i = 0; i < n; ++i) ++cnt[expert[i]];
  int ng = 0, q = 0;
  for (int e = 0; e < d.n_experts; ++e) {
    if (!cnt[e]) continue;
    gexp[ng] = e;
    gstart[ng++] = q;
    for (int i = 0; i < n; ++i)
      if (expert[i] == e) order[q++] = i;
  }
  gstart[ng] = q;
  for (int j = 0; j < n; ++j) gtok[j] = tok[order[j]];
  HostFfnArgs a{};
  a.H = d.hidden;
  a.I = d.inter;
  a.n_pairs = n;
  a.n_groups = ng;
  a.threads = host_threads(threads);
  a.tok = gtok;
  a.gexp = gexp;
  a.gstart = gstart;
  a.done = at<int32_t>(host_ws, p.done);
  a.xf = at<float>(host_ws, p.xf);
  a.act = at<float>(host_ws, p.act);
  a.y = at<float>(host_ws, p.y);
  host_expert_ffn(a, d.dtype == MOE_BF16, x, host_w->w_gate, host_w->w_up, host_w->w_down);
  for (int j = 0; j < n; ++j)
    memcpy(y_out + (int64_t)order[j] * d.hidden, a.y + (int64_t)j * d.hidden,
           (size_t)d.hidden * 4);
  return MOE_OK;
}

moe_status_t moe_layer_forward_offload(const moe_dims_t* dims, int32_t T, const void* x,
                                       const moe_weights_t* w, const moe_weights_t* host_w,
                                       const uint64_t* resident,
                                       const moe_offload_cost_t* cost, void* out, void* ws,
                                       size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                                       moe_offload_stats_t* stats, void* stream) {
  const auto t0 = std::chrono::steady_clock::now();
  moe_status_t st = check_forward(dims, T, x, w, nullptr, 0, MOE_MODE_STANDARD, out, nullptr);
  if (st != MOE_OK) return st;
  if (dims->weight_layout != MOE_LAYOUT_ROWS || dims->up_format != MOE_UP_DENSE)
    return MOE_EUNSUPPORTED;
  if ((st = check_cost(cost)) != MOE_OK) return st;
  if (!host_w || !host_w->w_gate || !host_w->w_up || !host_w->w_down || !resident)
    return MOE_EINVAL;
  if (!ok_ptr(ws) || !ok_ptr(host_ws)) return MOE_EINVAL;
  const OffloadPlan op = make_offload_plan(*dims, T);
  if (ws_bytes < op.d_total || host_ws_bytes < op.h_total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;

  const moe_dims_t& d = *dims;
  const Plan& p = op.dev;
  hipStream_t s = (hipStream_t)stream;
  const int k = d.top_k, E = d.n_experts, P = T * k, H = d.hidden, I = d.inter;
  const size_t eb = elem_bytes(d);
  int32_t* ids = at<int32_t>(ws, p.ids);
  float* wts = at<float>(ws, p.w);
  uint8_t* exact = at<uint8_t>(ws, p.exact);
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* perm = at<int32_t>(ws, p.perm);
  int32_t* row_of = at<int32_t>(ws, p.row_of);
  int32_t* moffsets = at<int32_t>(ws, p.moffsets);
  float* y_perm = at<float>(ws, p.y_perm);
  float* y_s = d.n_shared > 0 ? at<float>(ws, p.y_s) : nullptr;
  float* g_s = d.n_shared > 0 ? at<float>(ws, p.g_s) : nullptr;
  int32_t* h_ids = at<int32_t>(host_ws, op.ids);
  uint8_t* h_exact = at<uint8_t>(host_ws, op.exact);
  int32_t* h_pairs = at<int32_t>(host_ws, op.pairs);
  int32_t* h_tok = at<int32_t>(host_ws, op.tok);
  int32_t* h_gexp = at<int32_t>(host_ws, op.gexp);
  int32_t* h_gstart = at<int32_t>(host_ws, op.gstart);
  int32_t* h_tokens = at<int32_t>(host_ws, op.tokens);
  uint8_t* h_dec = at<uint8_t>(host_ws, op.dec);
  float* h_y = at<float>(host_ws, op.y);

  // 1. route, then stage the routed ids and the token rows on the host
  hipError_t e = launch_route(d, T, x, w->w_router, nullptr, 0, MOE_MODE_STANDARD, ids, wts, exact,
                              at<uint32_t>(ws, p.flags), at<float>(ws, p.logits), nullptr,
                              d.shared_gate ? w->w_shared_gate : nullptr, g_s, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_ids, ids, (size_t)P * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(at<void>(host_ws, op.x), x, (size_t)T * H * eb, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return MOE_EHIP;
  const double route_ms = ms_since(t0);

  for (int i = 0; i < E; ++i) h_tokens[i] = 0;
  for (int f = 0; f < P; ++f) {
    const int ex = h_ids[f];
    if (ex < 0 || ex >= E) return MOE_EHIP;  // the router never writes such an id
    ++h_tokens[ex];
  }
  offload_decide(d, h_tokens, *resident, *cost, h_dec);
  int missed = 0, fetched = 0, n_groups = 0, n_host = 0;
  for (int i = 0; i < E; ++i) {
    missed += h_dec[i] != MOE_OFFLOAD_NONE;
    fetched += h_dec[i] == MOE_OFFLOAD_FETCH;
    if (h_dec[i] == MOE_OFFLOAD_HOST) {
      h_gexp[n_groups] = i;
      h_gstart[n_groups] = n_host;
      for (int f = 0; f < P; ++f)
        if (h_ids[f] == i) {
          h_pairs[n_host] = f;
          h_tok[n_host] = f / k;
          ++n_host;
        }
      ++n_groups;
    }
  }
  h_gstart[n_groups] = n_host;
  for (int f = 0; f < P; ++f) h_exact[f] = h_dec[h_ids[f]] != MOE_OFFLOAD_HOST;

  // 2. fetches and the GPU's experts on the stream, the host FFN meanwhile
  if (stats && stats->gpu_start) e = hipEventRecord((hipEvent_t)stats->gpu_start, s);
  const size_t mat = (size_t)I * H * eb;
  for (int i = 0; i < E && e == hipSuccess; ++i) {
    if (h_dec[i] != MOE_OFFLOAD_FETCH) continue;
    const size_t o = (size_t)i * mat;
    e = hipMemcpyAsync((char*)w->w_gate + o, (const char*)host_w->w_gate + o, mat,
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync((char*)w->w_up + o, (const char*)host_w->w_up + o, mat,
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync((char*)w->w_down + o, (const char*)host_w->w_down + o, mat,
                         hipMemcpyHostToDevice, s);
  }
  if (e == hipSuccess) e = hipMemcpyAsync(exact, h_exact, (size_t)P, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = launch_permute(P, E, ids, exact, offsets, perm, at<int32_t>(ws, p.inv), row_of, moffsets,
                       at<int32_t>(ws, p.pscratch), s);
  if (e == hipSuccess)
    e = run_ffn(d, T, x, *w, MOE_MODE_STANDARD, offsets, moffsets, perm, y_perm, y_s, nullptr,
                at<uint32_t>(ws, p.flags), ws, p, 0, Prof{}, s, false);
  if (e == hipSuccess && stats && stats->gpu_stop) e = hipEventRecord((hipEvent_t)stats->gpu_stop, s);
  if (e != hipSuccess) return MOE_EHIP;
  const auto t1 = std::chrono::steady_clock::now();
  double host_ms = 0.0, parallel_ms = 0.0;
  if (n_host > 0) {
    HostFfnArgs a{};
    a.H = H;
    a.I = I;
    a.n_pairs = n_host;
    a.n_groups = n_groups;
    a.threads = host_threads(cost->cpu_threads);
    a.tok = h_tok;
    a.gexp = h_gexp;
    a.gstart = h_gstart;
    a.done = at<int32_t>(host_ws, op.done);
    a.xf = at<float>(host_ws, op.xf);
    a.act = at<float>(host_ws, op.act);
    a.y = h_y;
    host_expert_ffn(a, d.dtype == MOE_BF16, at<void>(host_ws, op.x), host_w->w_gate,
                    host_w->w_up, host_w->w_down);
    host_ms = ms_since(t1);
  }
  if (stats) {
    e = stats->gpu_stop ? hipEventSynchronize((hipEvent_t)stats->gpu_stop) : hipStreamSynchronize(s);
    if (e != hipSuccess) return MOE_EHIP;
    parallel_ms = ms_since(t1);
  }

  // 3. host rows to the GPU, into the expert-output rows, then the combine
  if (n_host > 0) {
    float* d_y = at<float>(ws, op.d_y);
    int32_t* d_pairs = at<int32_t>(ws, op.d_pairs);
    e = hipMemcpyAsync(d_y, h_y, (size_t)n_host * H * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d_pairs, h_pairs, (size_t)n_host * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_offload_scatter(n_host, H, d_pairs, d_y, row_of, y_perm, exact, s);
  }
  if (e == hipSuccess) e = launch_combine_rows(d, T, y_perm, false, row_of, wts, exact, y_s, g_s, out, s);
  if (e != hipSuccess) return MOE_EHIP;
  if (stats) {
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_EHIP;
    stats->missed_experts = missed;
    stats->fetched_experts = fetched;
    stats->host_experts = n_groups;
    stats->host_pairs = n_host;
    stats->route_ms = route_ms;
    stats->host_ms = host_ms;
    stats->parallel_ms = parallel_ms;
    stats->wall_ms = ms_since(t0);
    if (stats->decision) memcpy(stats->decision, h_dec, (size_t)E);
  }
  return MOE_OK;
}

}  // extern "C"
