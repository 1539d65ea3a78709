/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * One MoE layer forward at decode and prefill token counts:
 *   router logits -> softmax -> per-token top-k       [APEX page, Sec. 1;
 *                                                       SPICE page, "MoE inference I/O bottleneck"]
 *   stall-free substitution of non-prefetched experts  [APEX page, Sec. 4.3, Algorithm 1]
 *   residency split + LoRE surrogate y_shared + B_e A_e h
 *                                                      [SPICE page, "LoRE low-rank surrogate"]
 *   token->expert permutation (stable counting sort)
 *   SwiGLU expert FFNs, shared experts                 [FloE page, Sec. 1, forward a^S(x)]
 *   FloE: up-magnitude channel mask + INT2 up weights  [FloE page, Sec. 1]
 *   weighted combine.
 *
 * Conventions shared by every entry point
 *   - Pointers named in a signature are DEVICE pointers unless marked (host).
 *     moe_dims_t, moe_weights_t and moe_debug_t are host structs that hold
 *     device pointers.  Every device pointer must be 16-byte aligned.
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing, never synchronises, and keeps no state between calls; scratch
 *     memory comes from the caller's workspace (moe_workspace_size()).  The
 *     exceptions are named where they are declared: moe_layer_forward_noalloc
 *     (a library-held scratch array), moe_layer_forward_offload (waits for
 *     the routed ids and runs host threads) and moe_host_expert_ffn (host).
 *     moe_layer_forward runs the shared experts of bf16 batches of 128 or
 *     more tokens on a side stream (one non-blocking stream at the default
 *     priority and two events per GPU, created by that GPU's first such call
 *     and kept until the process ends), forked from and joined back into
 *     `stream` inside the call, so the caller still sees one ordered stream
 *     (and a graph captured on it holds both branches).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Calls on one stream are ordered.
 *   - Errors are return codes.  All argument checks run on the host before
 *     anything is enqueued: on any status other than MOE_OK nothing has been
 *     enqueued.  MOE_EHIP reports a failed kernel launch.
 *   - Layouts are row-major (C order).  "bf16" buffers hold bfloat16 bit
 *     patterns, "fp16" buffers IEEE half bit patterns.  dtype (MOE_F32 or
 *     MOE_BF16) applies to x, every dense weight, LoRE factors and out.
 *   - Limits: E <= 64, 1 <= k <= min(8, E), H % 64 == 0, I % 16 == 0,
 *     lore_rank <= 64, T >= 0 (T = 0 enqueues nothing and returns MOE_OK).
 *     Element offsets on the GPU are 32-bit: T * k * max(H, I, n_shared * I_s)
 *     and each expert matrix (I * H, I_s * H) must stay below 2^31, and
 *     T <= 2^22; larger batches are split by the caller (MOE_EUNSUPPORTED).
 *
 * Decisions.  Every ranking orders experts by (-logit, id) -- ties go to the
 * lower expert id -- and FloE channels by (-|u|, channel).  A token whose
 * deciding gap is below dims.tie_margin gets a flag bit (several answers are
 * correct there): 1 route, 2 prefetch, 4 substitution, 8 FloE mask, 16
 * prefetch budget.  Bit 32 marks a stall-free token whose prefetched set held
 * fewer than k experts (see moe_route).
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2
#define MOE_MAX_EXPERTS 64
#define MOE_MAX_TOPK 8
#define MOE_MAX_LORE_RANK 64
#define MOE_FLOE_MAX_DIM 16384 /* MOE_MODE_FLOE: inter and hidden at most this */
/* Scratch bytes per GPU of moe_layer_forward_noalloc (128 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* null pointer where one is required, bad value, misaligned */
  MOE_EUNSUPPORTED = 2, /* shape or mode outside the limits above                    */
  MOE_EWORKSPACE = 3,   /* workspace smaller than moe_workspace_size()               */
  MOE_EHIP = 4          /* a kernel launch failed                                    */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_MODE_STANDARD = 0,   /* every routed expert computed exactly                     */
  MOE_MODE_LORE = 1,       /* non-resident routed experts -> LoRE surrogate [SPICE]     */
  MOE_MODE_STALL_FREE = 2, /* non-prefetched routed experts -> best prefetched [APEX]   */
  MOE_MODE_FLOE = 3        /* INT2 up, top-|u| channel mask on gate/down [FloE]         */
} moe_mode_t;

typedef enum { MOE_UP_DENSE = 0, MOE_UP_INT2_G64 = 1 } moe_up_format_t;

/* Storage of the routed and shared expert matrices (w_gate, w_up, w_down,
 * ws_gate, ws_up, ws_down).  The router, prefetch router, shared gate, LoRE
 * factors and FloE tensors are row-major in either case.
 *   MOE_LAYOUT_ROWS:   row-major, the shapes listed in moe_weights_t.
 *   MOE_LAYOUT_MFMA16: every [R][K] matrix (k contiguous in the row-major
 *     form) packed fragment-major by moe_pack_weights: [ceil(R/16)]
 *     [ceil(K/32)][64][8], fragment (t, s) = rows 16t..+15 by k 32s..+31 as the
 *     16x16x32 matrix-core operand (lane l: row 16t + l%16, k from
 *     32s + 8*(l/16), eight values), zero past R or K.  Each expert's (or
 *     shared expert's) matrix is moe_pack_size(1, R, K) bytes, consecutive.
 *     bf16 and MOE_UP_DENSE only.  The kernels then read every weight
 *     fragment as one contiguous 1 KiB access. */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_MFMA16 = 1 } moe_weight_layout_t;

/* Layer shape (host struct). */
typedef struct {
  int32_t hidden;        /* H                                                     */
  int32_t n_experts;     /* E, routed experts                                     */
  int32_t top_k;         /* k                                                     */
  int32_t inter;         /* I, routed expert intermediate size                    */
  int32_t n_shared;      /* number of always-active shared experts (may be 0)     */
  int32_t shared_inter;  /* I_s                                                   */
  int32_t lore_rank;     /* r (0 when the layer has no LoRE factors)              */
  int32_t renormalize;   /* 1: weights p_e / sum over the chosen set; 0: p_e      */
  int32_t shared_gate;   /* 1: shared output scaled by sigmoid(x . w_sg)          */
  int32_t floe_keep;     /* FloE channels kept per (token, expert) pair, 1..I     */
  moe_dtype_t dtype;
  moe_up_format_t up_format;
  float tie_margin;      /* near-tie threshold for the flags (1e-4)               */
  moe_weight_layout_t weight_layout; /* storage of the expert matrices          */
} moe_dims_t;

/* Layer weights (host struct of device pointers; unused entries may be NULL). */
typedef struct {
  const void* w_router;       /* [E][H] dtype: row e holds expert e's logit weights    */
  const void* w_gate;         /* [E][I][H] dtype: channel i's H inputs contiguous      */
  const void* w_up;           /* [E][I][H] dtype (MOE_UP_DENSE)                        */
  const void* w_down;         /* MOE_UP_DENSE: [E][H][I]; MOE_UP_INT2_G64: [E][I][H]   */
  const uint8_t* up_q;        /* [E][I][H/4] INT2 codes, input h at bits 2*(h%4)       */
  const uint16_t* up_scale;   /* [E][I][H/64] fp16 scale s                             */
  const uint16_t* up_zero;    /* [E][I][H/64] fp16 zero z; weight = (q - z) * s        */
  const void* ws_gate;        /* [n_s][I_s][H] dtype                                   */
  const void* ws_up;          /* [n_s][I_s][H] dtype                                   */
  const void* ws_down;        /* [n_s][H][I_s] dtype                                   */
  const void* w_shared_gate;  /* [H] dtype, required when dims.shared_gate             */
  const void* lore_A;         /* [E][r][H] dtype                                       */
  const void* lore_B;         /* [E][H][r] dtype                                       */
} moe_weights_t;

/* Kernels of moe_layer_forward that the debug hook can bracket with events. */
typedef enum {
  MOE_KERNEL_NONE = 0,
  MOE_KERNEL_ROUTE = 1,
  MOE_KERNEL_PERMUTE = 2,        /* runs inside ROUTE when T*k <= 1024 and E > 16 */
  MOE_KERNEL_EXPERT_GATE_UP = 3, /* routed (+ shared, unless SHARED_FFN runs apart) gate/up */
  MOE_KERNEL_EXPERT_DOWN = 4,    /* routed (+ shared, unless SHARED_FFN runs apart) down  */
  MOE_KERNEL_FLOE_UP = 5,        /* INT2 up projection                                   */
  MOE_KERNEL_FLOE_SELECT = 6,    /* top-|u| channel selection                            */
  MOE_KERNEL_FLOE_GATE = 7,      /* gate on kept channels                                */
  MOE_KERNEL_FLOE_DOWN = 8,      /* down on kept channels                                */
  MOE_KERNEL_COMBINE = 9,        /* weighted combine (+ fused LoRE)                      */
  MOE_KERNEL_SHARED_FFN = 10     /* shared experts' own launches (bf16, T >= 128), run
                                    on a side stream alongside the routing and the routed
                                    experts; elapsed time 0 when the shared experts run
                                    inside the routed launches                          */
} moe_kernel_t;

/* Optional copies of intermediate results from moe_layer_forward (host
 * struct of device pointers; each entry may be NULL).  prof_start/prof_stop
 * are hipEvent_t handles owned by the caller: when prof_kernel names a
 * kernel of this call, they are recorded on `stream` immediately before and
 * after that kernel's launch (so hipEventElapsedTime gives its duration);
 * for MOE_KERNEL_SHARED_FFN on the side stream that runs it. */
typedef struct {
  int32_t* topk_ids;     /* [T][k] final expert per slot, ordered by (-logit, id)  */
  float* topk_w;         /* [T][k] combine weight per slot                          */
  uint8_t* exact;        /* [T][k] 1 = computed exactly, 0 = LoRE surrogate         */
  uint32_t* flags;       /* [T] near-tie flag bits                                  */
  float* logits;         /* [T][E] router logits                                    */
  float* mass;           /* [T] probability mass of the routed top-k                */
  int32_t* expert_offsets; /* [E+1]                                                 */
  int32_t* perm;         /* [T*k] (first offsets[E] entries meaningful)             */
  int32_t* floe_keep;    /* [T][k][floe_keep] kept channels, ascending (FLOE)       */
  void* prof_start;      /* hipEvent_t or NULL                                      */
  void* prof_stop;       /* hipEvent_t or NULL                                      */
  int32_t prof_kernel;   /* moe_kernel_t                                            */
} moe_debug_t;

int moe_abi_version(void);
const char* moe_status_string(moe_status_t status);

/* Bytes of device workspace that moe_layer_forward / moe_expert_ffn /
 * moe_permute need for T tokens in `mode` (host output). */
moe_status_t moe_workspace_size(const moe_dims_t* dims, int32_t T, moe_mode_t mode,
                                size_t* bytes /* host */);

/* Bytes of `groups` consecutive [rows][cols] matrices in MOE_LAYOUT_MFMA16
 * (host output): groups * ceil(rows/16)*16 * ceil(cols/32)*32 * 2.
 * MOE_EINVAL for a non-positive size or cols % 8 != 0. */
moe_status_t moe_pack_size(int32_t groups, int32_t rows, int32_t cols, size_t* bytes /* host */);

/* Packs `groups` consecutive row-major bf16 matrices src [groups][rows][cols]
 * into dst (moe_pack_size bytes) in MOE_LAYOUT_MFMA16, padding with zeros.
 * src and dst must not overlap.  Done once per set of weights: e.g.
 * w_gate with (E, I, H), w_down with (E, H, I), ws_down with (n_s, H, I_s). */
moe_status_t moe_pack_weights(int32_t groups, int32_t rows, int32_t cols, const void* src,
                              void* dst, void* stream);

/* Router: logits l = x W_r, softmax p, top-k by (-l, id) [APEX page, Sec. 1;
 * SPICE page, "MoE inference I/O bottleneck"].
 *   x [T][H] dtype, w_router [E][H] dtype.
 *   resident: uint64 expert bit masks; resident_stride 0 = one mask for all
 *     tokens, 1 = one mask per token.  LORE: exact[t][j] = bit of expert.
 *     STALL_FREE: the token's prefetched set; the final set is the routed set
 *     with each non-prefetched expert replaced by the best-scoring prefetched
 *     one under the original router [APEX page, Sec. 4.3, Algorithm 1].  The
 *     page's prefetched sets hold k + delta >= k experts; a set of fewer than
 *     k is kept whole and the remaining slots take the best experts outside
 *     it by router score (they stall), with flag bit 32.
 *     STANDARD / FLOE: ignored (may be NULL); every slot exact.
 *   Outputs: topk_ids [T][k] int32 ordered by (-l, id); topk_w [T][k] fp32
 *     (p_e, or p_e / sum over the set when dims.renormalize); exact [T][k];
 *     flags [T]; logits [T][E] fp32 (required: the first of the router's two
 *     kernels writes the logits there and the second ranks them); mass_opt
 *     [T] fp32 (SPICE confidence: mass of the routed top-k) may be NULL. */
moe_status_t moe_route(const moe_dims_t* dims, int32_t T, const void* x, const void* w_router,
                       const uint64_t* resident, int64_t resident_stride, moe_mode_t mode,
                       int32_t* topk_ids, float* topk_w, uint8_t* exact, uint32_t* flags,
                       float* logits, float* mass_opt, void* stream);

/* APEX prefetch set: mask_out[t] = bit mask of the top-(k + delta[t]) experts
 * of x W_p^T, W_p [E][H] (a linear prefetch router; softmax keeps the order) [APEX page,
 * Sec. 4.1 and Sec. 4.2].  delta [T] int32 in 0..E-k.  flags [T] is
 * overwritten: bit 2 where the list's last member and the next expert differ
 * by less than dims.tie_margin in logits, else 0. */
moe_status_t moe_prefetch_mask(const moe_dims_t* dims, int32_t T, const void* x,
                               const void* w_prefetch, const int32_t* delta,
                               uint64_t* mask_out, uint32_t* flags, void* stream);

/* APEX adaptive prefetch [APEX page, Sec. 4.2 (ordinal budget model) and
 * Sec. 5.1 (expert overlap)]: per token, s = w_delta . x_t and
 * p_d = sigmoid(theta[d] - s) for budgets d = 0..E-k; delta_out[t] = the least
 * d with p_d >= tau, or E-k when none qualifies; then mask_out[t] = the
 * top-(k + delta_out[t]) experts of x W_p^T exactly as moe_prefetch_mask.
 *   x [T][H] dtype, w_prefetch [E][H] dtype, w_delta [H] dtype, theta
 *   [E-k+1] fp32 (device), tau in (0, 1) (host value; MOE_EINVAL outside).
 *   flags [T] is overwritten: bit 2 as in moe_prefetch_mask, bit 16 where
 *   theta[d] - s sits within dims.tie_margin of logit(tau) at the chosen
 *   budget or the one below it (the budget itself is then a near-tie).
 *   topk_ids_opt [T][k] (the router's choices, moe_route's topk_ids) with
 *   delta_star_opt [T] and overlap_opt [T] int32: delta* = the least budget
 *   whose list holds every routed expert, overlap = how many routed experts
 *   the chosen list holds.  These three are all NULL or all set
 *   (MOE_EINVAL otherwise); routed ids outside 0..E-1 are skipped.
 *   Everything is caller-owned device memory; nothing is allocated. */
moe_status_t moe_prefetch_adaptive(const moe_dims_t* dims, int32_t T, const void* x,
                                   const void* w_prefetch, const void* w_delta,
                                   const float* theta, float tau, const int32_t* topk_ids_opt,
                                   int32_t* delta_out, uint64_t* mask_out, uint32_t* flags,
                                   int32_t* delta_star_opt, int32_t* overlap_opt, void* stream);

/* Stable counting sort of the exact (token, slot) pairs by expert: pair
 * f = t*k + j.  expert_offsets [E+1]; perm [T*k] holds f, grouped by expert,
 * f increasing inside a group (first offsets[E] entries); inv [T*k] = position
 * of pair f in perm, or -1 when not exact.  ws: at least
 * moe_workspace_size(dims with these T, k, E, STANDARD) bytes; it holds the
 * per-chunk bucket histograms when T*k > 1024 and may be NULL below that
 * (MOE_EWORKSPACE when too small). */
moe_status_t moe_permute(int32_t T, int32_t k, int32_t E, const int32_t* topk_ids,
                         const uint8_t* exact, int32_t* expert_offsets, int32_t* perm,
                         int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs for the permuted pairs and the shared experts.
 *   Dense: y_perm[p] = SwiGLU_e(x_t) = (SiLU(x W_g) * (x W_u)) W_d for pair
 *     p = (t, e) [FloE page, Sec. 1, S_t = identity], unweighted, fp32 [T*k][H].
 *   FLOE: u = x W_up with W_up = (q - z) * s; keep the dims.floe_keep channels
 *     of largest |u| (ties -> lower channel); y = sum over kept i of
 *     SiLU(g_i) u_i W_d[i,:] [FloE page, Sec. 1].  floe_keep_opt [T*k][keep]
 *     receives the kept channels of slot f = t*k + j (ascending); flags_opt [T] gets
 *     bit 8 OR-ed in for a near-tie at the mask edge (required in MOE_MODE_FLOE,
 *     ignored otherwise and may be NULL).  MOE_MODE_FLOE: T*k <= 65535.
 *   Shared: y_shared [T][H] fp32 = sum of the shared SwiGLU FFNs (ungated);
 *     shared_gate [T] fp32 = sigmoid(x . w_sg), or 1.  Both may be NULL when
 *     n_shared = 0.
 *   expert_offsets / perm come from moe_permute. */
moe_status_t moe_expert_ffn(const moe_dims_t* dims, int32_t T, const void* x,
                            const moe_weights_t* w, moe_mode_t mode,
                            const int32_t* expert_offsets, const int32_t* perm,
                            float* y_perm, float* y_shared, float* shared_gate,
                            int32_t* floe_keep_opt, uint32_t* flags_opt,
                            void* ws, size_t ws_bytes, void* stream);

/* FloE intra-expert predictor [FloE page, "dual sparsity predictors",
 * intra-expert predictor]: the channel masks of this layer's (token, expert)
 * pairs estimated from the previous layer's hidden state h_prev [T][H]
 * (dtype) through this layer's INT2 up projection, by the same rule as the
 * FloE forward (the dims.floe_keep channels of largest |h_prev W_up|, ties ->
 * lower channel).  topk_ids [T][k] name this layer's experts (ids outside
 * 0..E-1 leave their slot unwritten); keep_out [T][k][floe_keep] receives the
 * kept channels of slot f = t*k + j, ascending; flags [T] gets bit 8 OR-ed in
 * at a near-tie (the caller initialises it).  Reads w->up_q, up_scale,
 * up_zero.  ws: at least moe_workspace_size(dims, T, MOE_MODE_FLOE) bytes.
 * Needs the MOE_MODE_FLOE shape (INT2 up format), T*k <= 65535. */
moe_status_t moe_floe_predict(const moe_dims_t* dims, int32_t T, const void* h_prev,
                              const moe_weights_t* w, const int32_t* topk_ids, int32_t* keep_out,
                              uint32_t* flags, void* ws, size_t ws_bytes, void* stream);

/* FloE compact packing [FloE page, "system co-optimisation": the selected
 * channels' gate and down columns stored aligned and moved as one block]:
 * for slot f = t*k + j with expert e = topk_ids[f] and c < floe_keep,
 * gate_out[f][c][:] = w_gate[e][keep[f][c]][:] and down_out[f][c][:] =
 * w_down[e][keep[f][c]][:] (both weight tensors [E][I][H] dtype, the FloE
 * format); out [T][k][floe_keep][H] dtype each.  A slot with an id outside
 * 0..E-1, or a channel outside 0..I-1, gets zero rows.  T*k <= 65535. */
moe_status_t moe_floe_pack(const moe_dims_t* dims, int32_t T, const int32_t* topk_ids,
                           const int32_t* keep, const void* w_gate, const void* w_down,
                           void* gate_out, void* down_out, void* stream);

/* LoRE fitting, step 1 [SPICE page, "LoRE low-rank surrogate": for each
 * expert, collect its inputs h and outputs y_e and the shared experts'
 * output]: resid_out [N][H] fp32 = y_e(h) - y_shared(h) for the N calibration
 * rows h_cal [N][H] (dtype) and expert `expert`, computed by this library's
 * expert and shared FFN kernels (as in moe_expert_ffn, the SwiGLU product
 * rounded to dtype between the projections; y_shared ungated; 0 when
 * n_shared = 0).  Reads the routed and shared matrices of w (either
 * weight_layout) and requires w->w_router like every dense mode.  ws: at least
 * moe_workspace_size(dims with top_k = 1, N, MOE_MODE_STANDARD) bytes. */
moe_status_t moe_lore_targets(const moe_dims_t* dims, int32_t N, const void* h_cal,
                              const moe_weights_t* w, int32_t expert, float* resid_out, void* ws,
                              size_t ws_bytes, void* stream);

/* Bytes of workspace moe_lore_fit needs (host output); MOE_EINVAL unless
 * 1 <= rank <= cols <= min(64, hidden) and N > 0. */
moe_status_t moe_lore_fit_size(int32_t hidden, int32_t N, int32_t rank, int32_t cols,
                               size_t* bytes /* host */);

/* LoRE fitting, step 2 [SPICE page, "LoRE low-rank surrogate": minimise
 * ||y_e - y_shared - B_e A_e h||^2, solved with an SVD]: the rank-`rank` map
 * W = B A minimising ||R - h W^T||_F on the N calibration rows h_cal [N][H]
 * dtype (full column rank, N >= H) for targets R = resid [N][H] fp32
 * (moe_lore_targets).  With G = h^T h / N and M = R^T h / N the minimiser is
 * W = [M G^-1/2]_r G^-1/2: G^-1/2 by 20 rounds of the coupled Newton-Schulz
 * iteration from a Gershgorin-scaled start (converged to fp32 accuracy for
 * cond(G) up to about 1e2; an orthogonal design, G = I, takes 3), then the
 * truncated SVD U_r S_r V_r^T of M G^-1/2.  Outputs: lore_A_out [rank][H] =
 * V_r^T G^-1/2 and lore_B_out [H][rank] = U_r S_r (dtype; for rank =
 * dims.lore_rank these are expert e's slices of moe_weights_t.lore_A /
 * lore_B), sigma_out [rank] fp32 the singular values of M G^-1/2
 * (descending), err_out [1] fp32 the relative residual
 * ||R - h (B A)^T||_F / ||R||_F of the fp32 factors.  The SVD is a subspace
 * iteration of `n_iter` rounds (Y <- M M^T Y, orthonormalised) on `cols`
 * columns (rank <= cols <= 64) started from omega [H][cols] fp32 (the
 * caller's random draw), then a Rayleigh-Ritz step.  ws: at least
 * moe_lore_fit_size(H, N, rank, cols) bytes.  All buffers device,
 * caller-owned. */
moe_status_t moe_lore_fit(const moe_dims_t* dims, int32_t N, const void* h_cal,
                          const float* resid, int32_t rank, int32_t cols, int32_t n_iter,
                          const float* omega, void* lore_A_out, void* lore_B_out,
                          float* sigma_out, float* err_out, void* ws, size_t ws_bytes,
                          void* stream);

/* LoRE residual [SPICE page, "LoRE low-rank surrogate"]: for each slot with
 * exact[t][j] == 0, lore_out[t][j] = B_e (A_e x_t) with A_e [r][H] and
 * B_e [H][r]; slots with exact == 1 get 0.  lore_out [T][k][H] fp32. */
moe_status_t moe_lore_surrogate(const moe_dims_t* dims, int32_t T, const void* x,
                                const int32_t* topk_ids, const uint8_t* exact,
                                const void* lore_A, const void* lore_B, float* lore_out,
                                void* stream);

/* Weighted combine: out[t] = g_s(t) y_s(t) + sum_j w_tj yhat_tj with
 * yhat = y_perm[inv[t*k+j]] for exact slots and y_s(t) + lore_out[t][j]
 * otherwise.  y_shared / shared_gate / lore_out may be NULL (read as 0, 1, 0).
 * out [T][H] dtype, rounded to nearest even for bf16. */
moe_status_t moe_combine(const moe_dims_t* dims, int32_t T, const float* y_perm,
                         const int32_t* inv, const float* topk_w, const uint8_t* exact,
                         const float* y_shared, const float* shared_gate,
                         const float* lore_out, void* out, void* stream);

/* The whole layer in one call: route (+ substitution / residency split),
 * permute, expert FFNs, shared experts, LoRE surrogate fused into the
 * combine.  x [T][H] dtype -> out [T][H] dtype.  resident / resident_stride
 * as in moe_route.  dbg_opt (host struct, may be NULL) receives copies of
 * intermediates.  ws: moe_workspace_size(dims, T, mode) bytes. */
moe_status_t moe_layer_forward(const moe_dims_t* dims, int32_t T, const void* x,
                               const moe_weights_t* w, const uint64_t* resident,
                               int64_t resident_stride, moe_mode_t mode, void* out,
                               const moe_debug_t* dbg_opt, void* ws, size_t ws_bytes,
                               void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from that GPU's first call until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller still owns x, out, the weights and the masks.
 * MOE_EWORKSPACE when moe_workspace_size(dims, T, mode) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (e.g. 4096 Granite-shaped prefill tokens need
 * 225 MiB; every decode batch of the five workloads fits); MOE_EHIP when the
 * scratch array's device address cannot be obtained.  All calls on one GPU
 * share its array, which keeps the last call's contents: calls on one
 * stream are ordered, but calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  No
 * debug copies. */
moe_status_t moe_layer_forward_noalloc(const moe_dims_t* dims, int32_t T, const void* x,
                                       const moe_weights_t* w, const uint64_t* resident,
                                       int64_t resident_stride, moe_mode_t mode, void* out,
                                       void* stream);

/* ---- Exact execution of missed experts on the host or after a fetch ------
 * [SPICE page, "CPU-GPU collaboration: handling prefetch misses", cost rule
 * and the three-step execution of its Fig. 6]
 *
 * The routed expert matrices live in host memory (host_w) and the GPU holds
 * a slot per expert in w->w_gate / w_up / w_down, of which only the experts
 * set in the `resident` mask hold valid weights.  A routed expert that is not
 * resident is missed; each missed expert is either fetched (its three
 * matrices copied host -> slot, then run on the GPU with the resident ones)
 * or run on the host from host_w, by the cost rule below.  Both are exact:
 * the output equals moe_layer_forward in MOE_MODE_STANDARD up to fp32
 * summation order. */

typedef struct {
  double pcie_bytes_per_s; /* B_pcie: host -> GPU copy rate, bytes/s (> 0)          */
  double gpu_expert_s;     /* T_gpu_e: one expert's FFN on the GPU, seconds (>= 0)  */
  double cpu_expert_s;     /* host FFN time per expert run (its weight reads), s   */
  double cpu_pair_s;       /* host FFN time per (token, expert) pair, s (>= 0)     */
  int32_t cpu_threads;     /* host FFN threads; <= 0: min(16, hardware threads)   */
  int32_t queue_aware;     /* 0: each missed expert on its own; 1: with the load
                              already committed (see moe_offload_plan)         */
} moe_offload_cost_t;

/* Decisions of moe_offload_plan, one byte per expert. */
#define MOE_OFFLOAD_NONE 0  /* resident, or routed by no token        */
#define MOE_OFFLOAD_FETCH 1 /* copied to its GPU slot and run there   */
#define MOE_OFFLOAD_HOST 2  /* run on the host from host_w            */

/* The cost rule, per missed expert e with n_e routed (token, expert) pairs:
 *   fetch cost = W_e / B_pcie + T_gpu_e, W_e = 3 * I * H * sizeof(dtype)
 *   host cost  = T_cpu_e + 2 * n_e * H * sizeof(dtype) / B_pcie,
 *   T_cpu_e    = cpu_expert_s + n_e * cpu_pair_s
 * (the hidden state goes down and the expert's output comes back once per
 * pair); the expert is fetched when the fetch cost is strictly lower, else
 * run on the host.  With cost->queue_aware = 1 the link and the host are
 * treated as queues (the page's "PCIe pressure"): the missed experts are
 * decided in order of decreasing n_e (then id), and each fetch cost also
 * counts the fetch time (W_e / B_pcie + T_gpu_e) of the experts already
 * sent to the GPU, each host cost the host time of those already sent to
 * the host, so the two sides fill up evenly; the first decision is the
 * plain rule.  tokens [E] (host): n_e for every expert.  resident
 * (host): one uint64 mask word, bit e set = expert e is in its GPU slot.
 * decision_out [E] (host): MOE_OFFLOAD_*.  Host-only: no GPU needed, nothing
 * enqueued.  MOE_EINVAL on NULL pointers, negative counts or a cost with
 * B_pcie <= 0 (or infinite) or negative (or NaN) times. */
moe_status_t moe_offload_plan(const moe_dims_t* dims, const int32_t* tokens,
                              const uint64_t* resident, const moe_offload_cost_t* cost,
                              uint8_t* decision_out);

/* Device and host workspace bytes of moe_layer_forward_offload for T tokens.
 * The host workspace must be pinned (hipHostMalloc, or a torch tensor made
 * with pin_memory=True) so that its copies run asynchronously. */
moe_status_t moe_offload_workspace_size(const moe_dims_t* dims, int32_t T,
                                        size_t* device_bytes, size_t* host_bytes);

/* The host half of moe_layer_forward_offload on its own, all buffers in
 * host memory: for n (token, expert) pairs i, y_out[i] = W_d[e] a with
 * a = SiLU(W_g[e] x_t) * (W_u[e] x_t), t = tok[i], e = expert[i], sums in
 * fp32 and a rounded to dtype (bf16 layers) as on the GPU.  x [T][H] dtype;
 * host_w: w_gate, w_up, w_down as in moe_layer_forward_offload; y_out
 * [n][H] fp32.  threads <= 0: min(16, hardware threads).  host_ws: at least
 * moe_host_ffn_workspace_size(dims, n) bytes (pinning not needed).  Each
 * output element is one thread's fixed-order sum, so results do not depend
 * on the thread count.  Requires MOE_UP_DENSE; MOE_EINVAL on a token or
 * expert id out of range.  Runs on the calling thread (and the threads it
 * starts) and returns when done; no GPU needed. */
moe_status_t moe_host_ffn_workspace_size(const moe_dims_t* dims, int32_t n, size_t* bytes);
moe_status_t moe_host_expert_ffn(const moe_dims_t* dims, int32_t T, const void* x,
                                 const moe_weights_t* host_w, int32_t n, const int32_t* tok,
                                 const int32_t* expert, int32_t threads, float* y_out,
                                 void* host_ws, size_t host_ws_bytes);

/* Per-call figures of moe_layer_forward_offload (host struct, optional). */
typedef struct {
  int32_t missed_experts;   /* out: routed experts not resident              */
  int32_t fetched_experts;  /* out: of those, fetched                        */
  int32_t host_experts;     /* out: of those, run on the host                */
  int32_t host_pairs;       /* out: (token, expert) pairs run on the host    */
  double route_ms;          /* out: call start -> routed ids on the host     */
  double host_ms;           /* out: host FFN                                 */
  double parallel_ms;       /* out: GPU work dispatched -> host FFN and GPU
                               expert FFNs both done                         */
  double wall_ms;           /* out: whole call, through its last kernel      */
  uint8_t* decision;        /* in, optional host [E]: receives the plan      */
  void* gpu_start;          /* in, optional hipEvent_t: recorded before the
                               weight fetches                               */
  void* gpu_stop;           /* in, optional hipEvent_t: recorded after the
                               GPU expert FFNs                               */
} moe_offload_stats_t;

/* One layer forward with missed experts executed exactly, in three steps:
 *   1. route (MOE_MODE_STANDARD semantics) and stage the token rows and the
 *      routed ids in the pinned host workspace; plan every missed expert
 *      with moe_offload_plan;
 *   2. enqueue the fetched experts' copies host_w -> GPU slots and the GPU
 *      FFNs of the resident and fetched experts and the shared experts; the
 *      host FFN of the remaining missed pairs runs meanwhile on
 *      cost->cpu_threads threads (fp32 sums, the SwiGLU product rounded to
 *      dtype as on the GPU);
 *   3. copy the host rows to the GPU and combine them with the GPU rows.
 * x, out [T][H] dtype and ws (device bytes of moe_offload_workspace_size)
 * are device buffers; w holds device pointers, and the call writes fetched
 * experts into their slots of w->w_gate / w_up / w_down (it does not set
 * their resident bits: that is the caller's cache policy).  host_w: host
 * pointers w_gate, w_up, w_down, [E][I][H], [E][I][H], [E][H][I] dtype,
 * pinned for asynchronous fetches (its other members are ignored).
 * resident (host): one mask word.  host_ws: pinned host workspace.  Requires
 * MOE_LAYOUT_ROWS and MOE_UP_DENSE.
 *
 * Unlike the other entry points this call waits on `stream`, once, for the
 * routed ids (step 1), and with stats != NULL once more before returning.
 * It returns with steps 2 and 3 still enqueued: host_ws must stay untouched
 * until `stream` has finished them (a later call on the same stream is
 * ordered after them).  MOE_EINVAL / MOE_EUNSUPPORTED / MOE_EWORKSPACE as
 * for moe_layer_forward; MOE_EHIP on a failed launch or copy. */
moe_status_t moe_layer_forward_offload(const moe_dims_t* dims, int32_t T, const void* x,
                                       const moe_weights_t* w, const moe_weights_t* host_w,
                                       const uint64_t* resident,
                                       const moe_offload_cost_t* cost, void* out, void* ws,
                                       size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                                       moe_offload_stats_t* stats, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROUTE_H */
