/*
 * moe.h -- C ABI of libmoe: the forward pass of one sparse Mixture-of-Experts
 * FFN layer on an AMD Instinct MI355X (gfx950).
 *
 * The operation (pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 basic MoE
 * layer, §4.3 auxiliary loss and router z-loss, §5.1 DeepSpeed MoE settings
 * (min_capacity), §6.1 Mixtral expert (bias-free, SiLU), §7.1 DeepSeekMoE shared
 * experts, §8.2 capacity factor; "第7章 Mixture of Experts（MoE）架构" §7.1
 * MoE(x) = sum_i G(x)_i E_i(x), §7.4 balance loss and capacity; "[BEE-30064]
 * 混合專家架構與服務", how routing works):
 *
 *   l[t,e]  = sum_c x[t,c] W_g[e,c] (+ b_g[e])              router, no bias
 *   p[t,:]  = softmax(l[t,:])
 *   idx[t,:] = the k largest logits, descending, ties to the lower expert index
 *   w[t,j]  = p[t,idx[t,j]] / sum_j' p[t,idx[t,j']]          renormalised
 *   cap     = max(ceil(cf * T / E), min_capacity) (cf <= 0: no limit); for each
 *             expert the assignments are kept in ascending token order while
 *             fewer than cap have been kept, the rest are dropped (contribute nothing)
 *   out[t]  = sum_{kept j} w[t,j] (W2_e act(W1_e x[t] + b1_e) + b2_e),  e = idx[t,j]
 *           + sum_{s<S} FFN_{E+s}(x[t])                      shared, weight 1
 *   aux     = E * sum_e f_e P_e,  f_e = c_e/(T k) (c_e counted before capacity),
 *             P_e = mean_t p[t,e]                            unscaled
 *   z       = (1/T) sum_t (log sum_e exp l[t,e])^2           router z-loss, unscaled
 *   act     = GELU(u) = u * Phi(u) (erf form), or SiLU(u) = u / (1 + e^-u);
 *             a NULL b1 or b2 is a bias-free Linear.
 *
 * Conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library allocates no device memory, keeps no state between calls that
 *     affects a result (it caches two per-device lookups: the CU count and,
 *     for moe_forward_noalloc, its fixed scratch array's address) and never
 *     synchronises: moe_forward enqueues its kernels on launch->stream and
 *     returns.  Calls on different streams need distinct workspaces.
 *   - Matrices are row-major.  Weight matrices use the nn.Linear (out, in)
 *     layout.  dtype applies to x, W_g, W1, b1, W2, b2 and out: MOE_F32 is
 *     IEEE float32, MOE_BF16 is bfloat16 (uint16 bit patterns).
 *   - Validation happens on the host before anything is launched; on error
 *     nothing is launched and no output is touched.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Expert activation between the two Linears. */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SILU = 1 } moe_activation_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null required pointer, T/d/h/E <= 0, k < 1, k > E, n_shared < 0,
                               min_capacity < 0, NaN capacity_factor */
  MOE_ERR_UNSUPPORTED = 2,  /* E > MOE_MAX_EXPERTS, k > MOE_MAX_TOPK, n_shared > MOE_MAX_SHARED,
                               d or h not a multiple of 8, pointer not 16-byte aligned, unknown
                               dtype or activation, a row count that overflows int32, or (bf16) x,
                               the hidden rows R x h, one expert's weight or the router weight
                               reaching 4 GiB (the kernels address them through 32-bit buffer
                               ranges); float32: d x 256 bytes or the router weight reaching 4 GiB */
  MOE_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than moe_workspace_bytes(...) */
  MOE_ERR_HIP = 4,          /* a HIP launch reported an error (hipGetLastError) */
  MOE_ERR_SCRATCH = 5       /* moe_forward_noalloc: the problem needs more than
                               MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status_t;

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_MAX_SHARED 8

/* Stage boundaries at which optional timing events are recorded (see
 * moe_launch_t.stage_events): before the router, then after the router, the
 * scan, the scatter (each kept assignment's row in the expert-sorted order;
 * token rows are not copied), expert phase 1 (x W1^T + b1, activation), expert phase 2
 * (h W2^T + b2) and the combine.  With top-k routing the scan and the scatter
 * are one permute kernel: both boundaries are recorded after it (the scatter
 * stage is empty).  Under expert choice the scatter stage is the selection. */
#define MOE_NUM_STAGE_EVENTS 7

typedef struct {
  int32_t T;            /* tokens (rows of x), >= 1 */
  int32_t d;            /* model dimension, multiple of 8 */
  int32_t h;            /* expert hidden dimension, multiple of 8 */
  moe_dtype_t dtype;    /* dtype of x, W_g, W1, b1, W2, b2, out */
  const float* b_g;     /* [E] float32 added to the router logits before softmax and
                           selection, or NULL (no router bias) */
  int32_t* expert_counts; /* [E] out, or NULL: assignments per expert before capacity (c_e) */
  int32_t* expert_kept;   /* [E] out, or NULL: assignments kept after capacity */
  int32_t* slot_pos;      /* [T,k] out, or NULL: row of assignment (t,j) in the
                             expert-sorted buffer (expert e's rows start at
                             sum_{e'<e} kept_e'), or -1 if dropped */
  void* workspace;        /* device scratch of at least moe_workspace_bytes(...) bytes,
                             256-byte aligned; contents need not be initialised */
  size_t workspace_bytes;
  hipStream_t stream;     /* stream all kernels are enqueued on (0 = default stream) */
  hipEvent_t* stage_events; /* NULL, or an array of MOE_NUM_STAGE_EVENTS events recorded on
                               `stream` at the stage boundaries; a NULL entry is skipped
                               (each event recorded costs a few microseconds of the layer) */
  float* z_loss;          /* [1] out, or NULL: router z-loss (1/T) sum_t (log sum_e exp l[t,e])^2,
                             logits including b_g, unscaled (float64 partials, one rounding) */
  int32_t activation;     /* moe_activation_t of every expert, routed and shared;
                             0 = MOE_ACT_GELU (a zero-initialised struct keeps GELU) */
  int32_t min_capacity;   /* >= 0: floor under the capacity when capacity_factor > 0
                             (cap = max(ceil(cf*T/E), min_capacity)); ignored otherwise */
  const float* b_sel;     /* [E] float32, or NULL: a selection-only router bias.  The top-k
                             ranks l[t,e] + b_sel[e] (ties to the lower expert index);
                             the weights, the balance loss's P and the z-loss use l
                             itself.  The DeepSeek-V3 bias of the MoE training guide
                             §4.3/§7.1 and the BEE-30064 page (a bias on the router
                             logits that corrects expert usage), in the reading where
                             only the choice sees it (b_g is the in-logit reading).
                             No effect under expert choice: a per-expert constant does
                             not reorder an expert's tokens. */
  int32_t weights_packed; /* 0: W1 and W2 as declared below ([E+S, N, K] row-major).
                             1: both in the tile-packed layout that moe_pack_weights
                             writes (bf16, d and h multiples of 256 only; else
                             MOE_ERR_UNSUPPORTED).  Same results, bit for bit. */
} moe_launch_t;

/* Bytes of device workspace moe_forward needs for this problem shape (0 if
 * the shape is invalid).  Dominated by the hidden buffer [(T*k + S*T), h]
 * and the expert-output buffer [(T*k + S*T), d] in dtype, plus 64 MB of
 * float32 partial tiles for the bf16 grouped GEMM. */
size_t moe_workspace_bytes(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k,
                           int32_t n_shared, moe_dtype_t dtype);

/* The layer forward described above.
 *   x        [T, d]          input tokens (a batch and sequence flattened, as on the pages)
 *   W_g      [E, d]          router weight
 *   W1       [E+S, h, d]     first expert linear; experts 0..E-1 routed, E..E+S-1 shared
 *   b1       [E+S, h]         or NULL: the first Linear has no bias
 *   W2       [E+S, d, h]     second expert linear
 *   b2       [E+S, d]         or NULL: the second Linear has no bias
 *   E        routed experts, 1..MOE_MAX_EXPERTS
 *   k        experts per token, 1..min(E, MOE_MAX_TOPK)
 *   capacity_factor  <= 0: no capacity limit; else cap = max(ceil(cf*T/E), launch->min_capacity)
 *            (the ceiling in double precision)
 *   n_shared shared experts S, 0..MOE_MAX_SHARED
 *   out      [T, d]          layer output, dtype (bf16: accumulated in float32, rounded once)
 *   topk_idx [T, k] int32    slot j = the (j+1)-th largest logit, + launch->b_sel if given
 *            (before capacity)
 *   topk_w   [T, k] float32  renormalised weights of those slots (before capacity)
 *   aux_loss [1]    float32  E * sum_e f_e P_e
 *   launch   shape, dtype, optional outputs, workspace and stream (required)
 * Returns MOE_OK once everything is enqueued, or an error code (see moe_status_t). */
moe_status_t moe_forward(const void* x, const void* W_g, const void* W1, const void* b1,
                         const void* W2, const void* b2, int32_t E, int32_t k,
                         float capacity_factor, int32_t n_shared, void* out,
                         int32_t* topk_idx, float* topk_w, float* aux_loss,
                         const moe_launch_t* launch);

/* ---- Tile-packed expert weights --------------------------------------------
 * An optional weight layout for the bf16 expert Linears, written once (the
 * weights of a served model do not change) and read by moe_forward,
 * moe_forward_noalloc and moe_forward_expert_choice when
 * launch->weights_packed = 1.  The grouped GEMM streams each expert's weight
 * panel in 256-row x 64-column blocks; packed, every such block is 32 KB of
 * contiguous memory in the order the GEMM's loads take it, instead of 256
 * separate 128-byte pieces 2K bytes apart (measured 9% faster for the second
 * Linear of the DeepSeek-shaped layer, whose weights stream from HBM).
 *
 *   W      [n_mat, N, K] bf16 row-major (nn.Linear layout): W1 with N = h, K = d,
 *          or W2 with N = d, K = h; n_mat = E + S
 *   Wp     [n_mat * N * K] bf16, caller-owned, must not overlap W.  Element
 *          (m, n, kk) goes to block ((m * N/256 + n/256) * K/64 + kk/64), each block
 *          16384 elements: row r = n % 256 at r * 64, its 16-byte chunk
 *          c = (kk % 64) / 8 at chunk position c ^ (r & 7) ^ ((r >> 3) & 1), element
 *          kk % 8 within the chunk.
 *   N, K   multiples of 256; n_mat >= 1; N * K * 2 < 2^32 bytes (one matrix)
 *   stream the copy is enqueued on; returns MOE_OK once it is enqueued, or
 *          MOE_ERR_ARG / MOE_ERR_UNSUPPORTED (NULL, unaligned or overlapping
 *          buffers, a dtype other than bf16, sizes off the multiples above). */
moe_status_t moe_pack_weights(const void* W, int32_t n_mat, int32_t N, int32_t K, moe_dtype_t dtype, void* Wp,
                              hipStream_t stream);

/* ---- Expert-choice routing ------------------------------------------------
 * Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §4.2 (the router scores are
 * transposed to experts x tokens and each expert takes a top-k over tokens
 * with k = its capacity: perfect balance); "第7章 Mixture of Experts（MoE）架构"
 * §7.2 (each expert picks its top-C tokens; a token may be picked by several
 * experts or by none) and §7.1 (the gate weighting an expert's output is the
 * router's softmax).
 *
 *   l, p      as above (b_g included)
 *   tok[e,:]  the C tokens t with the largest l[t,e], ties to the lower token
 *             index, listed in ascending token order
 *   w[e,c]    = p[tok[e,c], e]                                 not renormalised
 *   out[t]    = sum_{(e,c): tok[e,c] = t} w[e,c] FFN_e(x[t])  + shared experts
 *   aux       = E * sum_e f_e P_e with f_e = C / (E C): exactly sum_e P_e, i.e. 1
 *   z         router z-loss as above
 *
 * Bytes of device workspace for moe_forward_expert_choice (0 if the shape is
 * invalid): hidden and expert-output buffers of E*C + S*T rows, plus an
 * expert-major float64 copy of the logits and an int32 [E, T] rank table. */
size_t moe_workspace_bytes_expert_choice(int32_t T, int32_t d, int32_t h, int32_t E, int32_t C,
                                         int32_t n_shared, moe_dtype_t dtype);

/* Tokens per expert for expert-choice routing from a capacity factor: the
 * capacity of "AI-Research-SKILLs MoE 训练实战…全指南" §8.2 (factor x tokens /
 * experts), floored by min_capacity as in its §5.1 DeepSpeed settings, and at
 * most T (an expert cannot take more tokens than there are):
 *   C = min(T, max(ceil(cf * T / E), min_capacity)),
 * the ceiling taken in double precision of the float32 cf (as moe_forward
 * computes its capacity).  Host-only arithmetic, no GPU call.  Returns C
 * (1..T), or -1 when cf is not > 0 (NaN included), T < 1, E < 1 or
 * min_capacity < 0. */
int32_t moe_expert_choice_capacity(float capacity_factor, int32_t T, int32_t E, int32_t min_capacity);

/* The layer forward with expert-choice routing.
 *   x, W_g, W1, b1, W2, b2, n_shared, out   as for moe_forward (b1, b2 may be NULL)
 *   E        routed experts, 1..MOE_MAX_EXPERTS
 *   C        tokens per expert, 1..T (e.g. ceil(capacity_factor * T / E), at most T)
 *   ec_token [E, C] int32 out: expert e's tokens, ascending token order
 *   ec_w     [E, C] float32 out: their weights p[t, e]
 *   aux_loss [1] float32 out, or NULL
 *   launch   as for moe_forward; expert_counts / expert_kept (if given) receive C for
 *            every expert, z_loss and activation apply, slot_pos and min_capacity are
 *            ignored
 * Errors as for moe_forward; C < 1 or C > T is MOE_ERR_ARG, E*C + S*T or E*T
 * above INT32_MAX is MOE_ERR_UNSUPPORTED (k and its limit do not apply). */
moe_status_t moe_forward_expert_choice(const void* x, const void* W_g, const void* W1, const void* b1,
                                       const void* W2, const void* b2, int32_t E, int32_t C,
                                       int32_t n_shared, void* out, int32_t* ec_token, float* ec_w,
                                       float* aux_loss, const moe_launch_t* launch);

/* ---- MXFP8 expert Linears --------------------------------------------------
 * Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §9.2 (FP8 quantization for
 * serving: about 20-30% more throughput than 16-bit, under 1% accuracy loss).
 * The pages fix no encoding; this library uses the OCP microscaling form MXFP8:
 *   codes   uint8 [R, K] E4M3 (bias 7, largest finite 448, S.1111.111 NaN)
 *   scales  uint8 [R, K/32] E8M0: block b of row r is scaled by 2^(byte - 127)
 * along the contracted dimension K.  Quantizing a block of 32 values v:
 *   s = floor(log2 max|v|) - 8 (s = -127 for an all-zero block), byte = s + 127,
 *   code_i = the E4M3 value nearest v_i * 2^-s, ties to even, clamped to +-448.
 * The layer (W8A8): x is quantized along d, the first Linear's activation
 * output H along h, the weights are given quantized along their input
 * dimension; products and sums in float32 on the matrix cores; the router,
 * biases, combine and outputs are bf16 as in moe_forward.
 *
 * bf16 [rows, cols] (cols % 32 == 0, src and codes 16-byte aligned) -> MXFP8,
 * enqueued on `stream`: for quantizing expert weights. */
moe_status_t moe_quantize_mxfp8(const void* src, int32_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream);

/* Workspace bytes for moe_forward_mxfp8 (0 if the shape is invalid: bf16 only,
 * d and h multiples of 256). */
size_t moe_workspace_bytes_mxfp8(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t n_shared);

/* The layer forward with MXFP8 expert Linears.
 *   x [T, d], W_g [E, d], b1 [E+S, h] or NULL, b2 [E+S, d] or NULL, out [T, d]: bf16
 *   W1 [E+S, h, d] codes and W1_scales [E+S, h, d/32]   (quantized along d)
 *   W2 [E+S, d, h] codes and W2_scales [E+S, d, h/32]   (quantized along h)
 *   other arguments and launch fields as for moe_forward; launch->dtype must be
 *   MOE_BF16 (else MOE_ERR_UNSUPPORTED), d and h multiples of 256 (else
 *   MOE_ERR_UNSUPPORTED); code arrays 16-byte, scale arrays 4-byte aligned. */
moe_status_t moe_forward_mxfp8(const void* x, const void* W_g, const uint8_t* W1, const uint8_t* W1_scales,
                               const void* b1, const uint8_t* W2, const uint8_t* W2_scales, const void* b2,
                               int32_t E, int32_t k, float capacity_factor, int32_t n_shared, void* out,
                               int32_t* topk_idx, float* topk_w, float* aux_loss, const moe_launch_t* launch);

/* ---- For callers that cannot allocate ----------------------------------------
 * For code under HIP graph capture, tight serving loops and harnesses that
 * forbid device allocation: moe_forward with every argument and result as
 * above, but its scratch (the hidden and expert-output buffers, routing
 * tables, partial logits and partial GEMM tiles) in a fixed device array of
 * the library instead of launch->workspace (ignored, with
 * launch->workspace_bytes).  The array holds MOE_NOALLOC_SCRATCH_BYTES on
 * every GPU the library runs on, from the code object's load on that GPU
 * until the process ends.  Nothing is allocated or freed by the call (no
 * hipMalloc, hipFree or allocating library routine), and nothing in the
 * array needs to start at zero.
 *
 * The call runs on the calling thread's current device; launch->stream must
 * belong to it.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 *
 * Returns MOE_ERR_SCRATCH, before any GPU call, when the problem's scratch
 * (moe_workspace_bytes' layout with 16 partial GEMM tiles instead of 256)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES: e.g. T = 4096, d = 512, h = 2048,
 * E = 64, k = 1 in float32 fits; the Mixtral-shaped layer (0.8 GB) does not.
 * Other errors as for moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_noalloc(const void* x, const void* W_g, const void* W1, const void* b1,
                                 const void* W2, const void* b2, int32_t E, int32_t k,
                                 float capacity_factor, int32_t n_shared, void* out,
                                 int32_t* topk_idx, float* topk_w, float* aux_loss,
                                 const moe_launch_t* launch);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
