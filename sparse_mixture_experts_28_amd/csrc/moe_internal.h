// Internal declarations shared by the HIP translation units of libmoe.
// Not part of the public ABI (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "moe.h"

namespace moe {

// ------------------------------------------------------------ constants --
constexpr int kRouterTile = 64;     // tokens per router workgroup (= permute rank tile)
constexpr int kRouterThreads = 256; // 4 waves x 16 tokens
constexpr int kWave = 64;

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (n < 64) and does not wait on LDS or export counters
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// ---------------------------------------------------------- bf16 helpers --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x0040u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

// ---------------------------------------------- fast activations (MFMA) --
// For the GEMM epilogues, whose results are rounded to bf16 or quantized.
// SiLU(v) = v / (1 + e^-v) with the hardware exp2 and reciprocal (~1 ulp
// each); e^-v overflows to +inf for v < -88 and the product is then -0, the limit.
__device__ __forceinline__ float silu_fast(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.44269504088896341f));
}

// GELU(v) = v Phi(v) = max(v, 0) - |v| erfc(|v| / sqrt 2) / 2, with
// erfc(u / sqrt 2) = exp2(u Q(u)) for u = min(|v|, 6) and u Q(u) a degree-6
// polynomial fit of log2 erfc(u / sqrt 2) without a constant term (the fit is
// csrc/fit_gelu.py).  Past |v| = 6 the correction term is below 1e-8 and u
// stands in for |v| in it.  Within 2.5e-7 absolute and 4.8e-7 |v| of GELU in
// float32; one exp2 and 9 VALU operations (the epilogue of the first Linear
// is VALU-bound).  The maximum propagates NaN, so NaN gives NaN and +inf
// gives +inf; -inf gives about -6e-9 (the limit is 0; the erf form gives NaN).
__device__ __forceinline__ float gelu_fast(float v) {
  const float u = __builtin_amdgcn_fmed3f(fabsf(v), 0.0f, 6.0f);   // min(|v|, 6); NaN gives 6
  float q = fmaf(u, 3.228566493e-05f, -7.544446853e-04f);
  q = fmaf(u, q, 8.004920557e-03f);
  q = fmaf(u, q, -5.324933678e-02f);
  q = fmaf(u, q, -4.589283466e-01f);
  q = fmaf(u, q, -1.151139259e+00f);
  const float e = __builtin_amdgcn_exp2f(fmaf(q, u, -1.0f));      // erfc(u / sqrt 2) / 2
  return fmaf(-u, e, __builtin_elementwise_maximum(v, 0.0f));
}

// ----------------------------------------------------- workspace layout --
// All regions are carved from one caller-owned device buffer, each aligned to
// 256 bytes.  Row counts: A = routed rows (T*k, the worst case without drops,
// or E*C under expert choice), R = A + S*T rows of the expert hidden / output
// buffers (shared experts at the fixed row offset A + s*T).
struct Workspace {
  int32_t* row_token;   // [A]        token of each row of the expert-sorted order (kept assignments)
  void* hbuf;           // [R, h]     GELU(x W1^T + b1)
  void* ybuf;           // [R, d]     h W2^T + b2
  int32_t* local_rank;  // [T, k]     rank of (t,j) among earlier tokens of its router tile
  int32_t* tile_hist;   // [ntile, E] assignments per (router tile, expert)
  float* p_part;        // [ntile, E] per-tile sums of the softmax probabilities
  double* z_part;       // [ntile]    per-tile sums of the squared log-sum-exp of the logits
  int32_t* counts;      // [E]
  int32_t* kept;        // [E]
  int32_t* slot_pos;    // [T, k]
  int32_t* seg;         // segment table, see SegTable
  double* logits;       // [KS, T, Epad] float64 partial router logits (bf16 path)
  double* ec_logits;    // [E, T]     expert choice: float64 logits, expert-major
  double* ec_m;         // [T]        expert choice: each token's largest logit
  float* ec_z;          // [T]        expert choice: each token's sum of exp(l - m)
  int32_t* ec_pos;      // [E, T]     expert choice: rank of t among e's chosen tokens, -1 if not chosen
  uint8_t* xq;          // [T, d]     MXFP8: x's E4M3 codes (the hidden buffer then holds H's codes and scales)
  uint8_t* xq_scales;   // [T, d/32]  MXFP8: x's E8M0 scales
  float* part;          // [part_cap, BM, 256] float32 partial tiles of the grouped GEMM's split tail
  int part_cap;         // partial tiles the buffer holds (0: no split)
  size_t bytes;
};

// Segment table written by the scan kernel and read by the grouped GEMM and
// the scatter: nseg = E + S segments.  Stored as int32 arrays back to back:
//   rows[nseg]        rows of the segment (kept_e, or T for a shared expert)
//   a_off[nseg]       first row of the segment in its phase-1 row list: the
//                     expert-sorted order (row_token) for routed experts, x for
//                     shared experts
//   o_off[nseg]       first row of the segment in hbuf / ybuf
//   tile_start[nseg+1] prefix sum of ceil(rows / tile_bm) (M tiles of the GEMM)
//   route_off[E]      exclusive scan of kept (first row of expert e in the expert-sorted order)
//   tile_bm[nseg]     M tile height of the segment in the grouped GEMM
struct SegTable {
  int32_t* rows;
  int32_t* a_off;
  int32_t* o_off;
  int32_t* tile_start;
  int32_t* route_off;
  int32_t* tile_bm;
};

__host__ __device__ inline SegTable seg_table(int32_t* base, int nseg, int E) {
  SegTable s;
  s.rows = base;
  s.a_off = base + nseg;
  s.o_off = base + 2 * nseg;
  s.tile_start = base + 3 * nseg;
  s.route_off = base + 4 * nseg + 1;
  s.tile_bm = base + 4 * nseg + 1 + E;
  return s;
}
inline size_t seg_table_ints(int nseg, int E) { return static_cast<size_t>(5 * nseg + 1 + E); }

// The segment table as a kernel that only reads it sees it: in the constant
// address space, so lookups at a uniform index are scalar loads (the scalar
// cache, no vector-memory wait; the table is written by an earlier launch).
typedef const __attribute__((address_space(4))) int32_t cint32_t;
struct SegTableRO {
  cint32_t* rows;
  cint32_t* a_off;
  cint32_t* o_off;
  cint32_t* tile_start;
  cint32_t* tile_bm;
};
__device__ inline SegTableRO seg_table_ro(const int32_t* base, int nseg, int E) {
  cint32_t* c = (cint32_t*)base;
  return SegTableRO{c, c + nseg, c + 2 * nseg, c + 3 * nseg, c + 4 * nseg + 1 + E};
}

// Per-segment tile heights of the MXFP8 GEMM (Problem::gemm_mixed): a
// segment of r rows takes 192-row tiles only when they cut its tiles by more
// than a third, 3 ceil(r / 192) < 2 ceil(r / 128) (r in 129..192, 513..576,
// 897..960, ...).  A 192-row tile takes 1.3-1.4 times as long as a 128-row
// one where the weights stream from HBM, and up to 1.6 times in the second
// Linear of capacity-bound loads (measured), so smaller savings do not pay.
// Empty and short segments keep 128-row tiles.
__host__ __device__ inline int mx_mixed_tile_height(int rows) {
  const int t128 = (rows + 127) / 128, t192 = (rows + 191) / 192;
  return 3 * t192 < 2 * t128 ? 192 : 128;
}

// ------------------------------------------------ grouped-GEMM helpers --
// (shared by the bf16 and MXFP8 grouped GEMMs; the descriptor also by the router)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kGroupM = 8;

// Buffer descriptor over [base, base + bytes): a load past the end reads zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// Logical tile L -> (M tile, N tile): groups of kGroupM consecutive M tiles
// (adjacent rows of the same or neighbouring experts) sweep all N tiles,
// M fastest, so tiles that run together share A and B panels in L2.
__device__ __forceinline__ void tile_of(int L, int total_mt, int ntn, int& mt, int& nt) {
  const int gsz = kGroupM * ntn;
  const int grp = L / gsz;
  const int first_m = grp * kGroupM;
  const int gm = min(kGroupM, total_mt - first_m);
  const int r = L - grp * gsz;
  mt = first_m + r % gm;
  nt = r / gm;
}

// Split of the last partial round of a persistent launch of P workgroups
// over `total` tiles: the `tail` = total mod P tiles of that round are cut
// along K into S pieces each (S = P / tail, at most nk / 4 steps per piece
// and at most part_cap pieces), so the round keeps the whole grid busy.  The
// pieces leave float32 partial tiles; a fix-up kernel sums each tile's S
// pieces in order, so results do not depend on timing.
struct TailPlan {
  int full;   // tiles computed whole
  int tail;   // tiles computed in pieces (0 if no split)
  int S;      // pieces per tail tile
};

__device__ __forceinline__ TailPlan tail_plan(int total, int P, int nk, int part_cap) {
  TailPlan tp{total, 0, 1};
  const int tail = total % P;
  if (tail == 0) return tp;
  int S = min(P / tail, nk / 4);
  S = min(S, part_cap / tail);
  if (S < 2) return tp;
  tp.full = total - tail;
  tp.tail = tail;
  tp.S = S;
  return tp;
}

// Segment of M tile mt: the last segment whose first tile is <= mt (empty
// segments share their successor's first tile and are passed over).
template <typename Ptr>
__device__ __forceinline__ int find_segment(Ptr tile_start, int nseg, int mt) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Logical tile L -> (M tile, N tile) in expert-major order, returning the
// segment: a segment's tiles are contiguous and, within it, its M tiles are
// adjacent for each N tile (M fastest).  Weight-streaming launches (short
// experts) use it: the contiguous run of tiles an XCD takes per round then
// covers few experts, whose weight panels (shared by the expert's M tiles)
// and row panels (shared by its N tiles) stay in that XCD's L2.
template <typename Ptr>
__device__ __forceinline__ int tile_of_expert(int L, Ptr tile_start, int nseg, int ntn, int& mt, int& nt) {
  const int s = find_segment(tile_start, nseg, L / ntn);
  const int t0 = tile_start[s], mts = tile_start[s + 1] - t0;
  const int local = L - t0 * ntn;
  mt = t0 + local % mts;
  nt = local / mts;
  return s;
}

// Compute units of the calling thread's current device (the persistent GEMM
// grids run one workgroup per CU), queried once per device and kept for the
// process; 256 (MI355X) if the query fails.
inline int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int n = dev < kMaxDevices ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct Problem {
  int T, d, h, E, k, S;
  bool mx;       // MXFP8 expert Linears
  int ec_C;      // expert choice: tokens per expert (0: token choice, top-k per token)
  int A;         // routed rows: T * k, or E * ec_C under expert choice
  moe_dtype_t dtype;
  int act;       // moe_activation_t of the experts
  int cap;       // capacity per expert (min_capacity applied); INT32_MAX when unlimited
  int rtile;     // tokens per router tile (router_tile)
  int ntile;     // ceil(T / rtile)
  int gemm_bm;   // M tile of the grouped GEMM (for the tile prefix)
  bool gemm_mixed;   // MXFP8 GEMM: per-segment heights by mx_mixed_tile_height (gemm_bm unused)
  int part_limit;    // float32 partial tiles the workspace reserves for the GEMM's split tail
  bool packed_w;     // W1, W2 in the tile-packed layout (moe_pack_weights)
};

Workspace carve_workspace(const Problem& p, void* base, size_t bytes_available, bool* ok);
size_t workspace_bytes(const Problem& p);

// ------------------------------------------------------ kernel launchers --
// Each returns hipGetLastError() after its launch(es).
hipError_t launch_router(const Problem& p, const void* x, const void* W_g, const float* b_g, const float* b_sel,
                         int32_t* topk_idx, float* topk_w, const Workspace& ws, hipStream_t st);
hipError_t launch_scan(const Problem& p, const Workspace& ws, float* aux_loss, float* z_loss,
                       int32_t* counts_out, int32_t* kept_out, hipStream_t st);
// top-k routing: base ranks, capacity, slot positions, row -> token index, and
// (workgroup 0) counts, aux, z-loss and the segment table, in one launch
hipError_t launch_permute(const Problem& p, const int32_t* topk_idx, const Workspace& ws, float* aux_loss,
                          float* z_loss, int32_t* counts_out, int32_t* kept_out, hipStream_t st);
hipError_t launch_expert_ffn(const Problem& p, const void* x, const void* W1, const void* b1,
                             const void* W2, const void* b2, const Workspace& ws, int phase,
                             hipStream_t st);
hipError_t launch_combine(const Problem& p, const float* topk_w, const Workspace& ws, void* out,
                          hipStream_t st);
// expert choice: each expert's top-C tokens (ec_token, ec_w [E, C]; the GEMM's
// row -> token index; the per-(expert, token) rank table), and the combine
// over the experts that took each token
hipError_t launch_ec_select(const Problem& p, int32_t* ec_token, float* ec_w, const Workspace& ws,
                            hipStream_t st);
hipError_t launch_combine_ec(const Problem& p, const float* ec_w, const Workspace& ws, void* out,
                             hipStream_t st);
// MXFP8: the caller's pre-quantized expert weights and bf16 biases
struct MxWeights {
  const uint8_t* W1;    // [E+S, h, d] E4M3 codes
  const uint8_t* W1s;   // [E+S, h, d/32] E8M0 scales
  const void* b1;       // [E+S, h] bf16 or nullptr
  const uint8_t* W2;    // [E+S, d, h]
  const uint8_t* W2s;   // [E+S, d, h/32]
  const void* b2;       // [E+S, d] bf16 or nullptr
};
// bf16 [rows, cols] -> MXFP8 codes [rows, cols] and scales [rows, cols/32] (cols % 32 == 0)
hipError_t launch_mx_quantize(const uint16_t* src, int rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t st);
hipError_t launch_expert_ffn_mx(const Problem& p, const MxWeights& w, const Workspace& ws, int phase,
                                hipStream_t st);

// Which GEMM kernel serves a problem; the M tile decides the tile prefix.
bool gemm_fast_path(const Problem& p);
// W [n_mat, N, K] bf16 -> the tile-packed layout of include/moe.h (N, K multiples of 256)
hipError_t launch_pack_weights(const void* W, int n_mat, int N, int K, void* Wp, hipStream_t st);
int gemm_m_tile(const Problem& p);
// router logits (bf16, d % 256 == 0, more than 64 experts): expert padding
// and split-K factor, which size the float64 partial-logit workspace
// [KS][T][Epad] (KS = 0 on the one-launch path)
int logit_pad(int E);
int logit_splits(const Problem& p);
// the one-launch router and its tile (32 or 64 tokens; needs T, d, E, dtype)
bool router_fused(const Problem& p);
int router_tile(const Problem& p);
// partial tiles reserved for the grouped GEMM's split tail (one per workgroup of a 256-CU part)
constexpr int kGemmPartCap = 256;
// the same in the fixed scratch of moe_forward_noalloc (16 tiles of 256 x 256 float32: 4 MB)
constexpr int kNoallocPartTiles = 16;

// the top-k layer on a given workspace (moe_api.cpp)
moe_status_t forward_top_k(const void* x, const void* W_g, const void* W1, const void* b1, const void* W2,
                           const void* b2, int32_t E, int32_t k, float capacity_factor, int32_t n_shared, void* out,
                           int32_t* topk_idx, float* topk_w, float* aux_loss, const moe_launch_t* launch,
                           void* ws_base, size_t ws_bytes, int part_limit);
// device address of the current device's copy of the fixed scratch (looked up once per device)
moe_status_t scratch_of_current_device(void** out);

}  // namespace moe
