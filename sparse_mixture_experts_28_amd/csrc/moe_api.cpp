// Host side of the C ABI (include/moe.h): validation, workspace carving and the
// launch sequence router -> scan -> scatter -> expert phase 1 -> phase 2 -> combine
// (expert choice: router -> scan -> per-expert selection -> phase 1 -> phase 2 ->
// combine), all enqueued on the caller's stream with no host synchronisation.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

struct Layout {
  size_t row_token, hbuf, ybuf, local_rank, tile_hist, p_part, z_part, counts, kept, slot_pos, seg, logits, ec_logits,
      ec_m, ec_z, ec_pos, xq, xq_scales, part, total;
  int part_cap;
};

Layout layout_of(const Problem& p) {
  const size_t s = elem_bytes(p.dtype);
  const size_t A = static_cast<size_t>(p.A);
  const size_t R = A + static_cast<size_t>(p.S) * p.T;
  const size_t te = static_cast<size_t>(p.ntile) * p.E;
  const size_t tk = static_cast<size_t>(p.T) * p.k;          // token-choice slots (0 under expert choice)
  const size_t et = p.ec_C > 0 ? static_cast<size_t>(p.E) * p.T : 0;
  const size_t ect = p.ec_C > 0 ? static_cast<size_t>(p.T) : 0;
  Layout L;
  size_t off = 0;
  L.row_token = off;  off += align_up(A * 4);
  L.hbuf = off;       off += align_up(R * p.h * s);
  L.ybuf = off;       off += align_up(R * p.d * s);
  L.local_rank = off; off += align_up(tk * 4);
  L.tile_hist = off;  off += align_up(te * 4);
  L.p_part = off;     off += align_up(te * 4);
  L.z_part = off;     off += align_up(static_cast<size_t>(p.ntile) * 8);
  L.counts = off;     off += align_up(static_cast<size_t>(p.E) * 4);
  L.kept = off;       off += align_up(static_cast<size_t>(p.E) * 4);
  L.slot_pos = off;   off += align_up(tk * 4);
  L.seg = off;        off += align_up(seg_table_ints(p.E + p.S, p.E) * 4);
  L.logits = off;     off += align_up(static_cast<size_t>(logit_splits(p)) * p.T * logit_pad(p.E) * 8);
  L.ec_logits = off;  off += align_up(et * 8);
  L.ec_m = off;       off += align_up(ect * 8);
  L.ec_z = off;       off += align_up(ect * 4);
  L.ec_pos = off;     off += align_up(et * 4);
  // MXFP8: x's codes and scales (H's go into the hidden buffer, R h + R h / 32 <= R h 2 bytes)
  const size_t td = p.mx ? static_cast<size_t>(p.T) * p.d : 0;
  L.xq = off;         off += align_up(td);
  L.xq_scales = off;  off += align_up(td / 32);
  // sized for the tallest tile: moe_workspace_bytes has no capacity factor,
  // and the tile height moe_forward picks can depend on it
  L.part_cap = p.mx || gemm_fast_path(p) ? p.part_limit : 0;   // the MXFP8 path always runs its MFMA kernel
  L.part = off;       off += align_up(static_cast<size_t>(L.part_cap) * 256 * 256 * 4);
  L.total = off;
  return L;
}

}  // namespace

size_t workspace_bytes(const Problem& p) { return layout_of(p).total; }

Workspace carve_workspace(const Problem& p, void* base, size_t bytes_available, bool* ok) {
  const Layout L = layout_of(p);
  Workspace w{};
  *ok = base != nullptr && bytes_available >= L.total && aligned(base, kAlign);
  if (!*ok) return w;
  char* b = static_cast<char*>(base);
  w.row_token = reinterpret_cast<int32_t*>(b + L.row_token);
  w.hbuf = b + L.hbuf;
  w.ybuf = b + L.ybuf;
  w.local_rank = reinterpret_cast<int32_t*>(b + L.local_rank);
  w.tile_hist = reinterpret_cast<int32_t*>(b + L.tile_hist);
  w.p_part = reinterpret_cast<float*>(b + L.p_part);
  w.z_part = reinterpret_cast<double*>(b + L.z_part);
  w.counts = reinterpret_cast<int32_t*>(b + L.counts);
  w.kept = reinterpret_cast<int32_t*>(b + L.kept);
  w.slot_pos = reinterpret_cast<int32_t*>(b + L.slot_pos);
  w.seg = reinterpret_cast<int32_t*>(b + L.seg);
  w.logits = reinterpret_cast<double*>(b + L.logits);
  w.ec_logits = reinterpret_cast<double*>(b + L.ec_logits);
  w.ec_m = reinterpret_cast<double*>(b + L.ec_m);
  w.ec_z = reinterpret_cast<float*>(b + L.ec_z);
  w.ec_pos = reinterpret_cast<int32_t*>(b + L.ec_pos);
  w.xq = reinterpret_cast<uint8_t*>(b + L.xq);
  w.xq_scales = reinterpret_cast<uint8_t*>(b + L.xq_scales);
  w.part = reinterpret_cast<float*>(b + L.part);
  w.part_cap = L.part_cap;
  w.bytes = L.total;
  return w;
}

namespace {

// Shape checks shared by moe_workspace_bytes and moe_forward.
// The kernels read x, the hidden rows, an expert's weight matrix and the
// router weight through buffer resources, whose range (and the offsets into
// it) is 32-bit: each such operand must stay under 4 GiB (bf16; float32 layers
// read only router tiles and the router weight that way).
bool fits_buffer_ranges(long long T, long long d, long long h, long long E, long long rows, int dtype) {
  constexpr long long kRange = 0xffffffffll;
  if (dtype == MOE_BF16)
    return T * d * 2 <= kRange && rows * h * 2 <= kRange && h * d * 2 <= kRange && E * d * 2 <= kRange;
  return 64 * d * 4 <= kRange && E * d * 4 <= kRange;
}

moe_status_t check_shape(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t S, int dtype) {
  if (T < 1 || d < 1 || h < 1 || E < 1 || k < 1 || k > E || S < 0) return MOE_ERR_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || S > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0 || h % 8 != 0) return MOE_ERR_UNSUPPORTED;
  const long long rows = static_cast<long long>(T) * k + static_cast<long long>(S) * T;
  if (rows > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!fits_buffer_ranges(T, d, h, E, rows, dtype)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// cap = max(ceil(cf T / E), min_cap) in double (cf > 0), saturated at INT32_MAX
int capacity_of(float cf, int32_t T, int32_t E, int32_t min_cap) {
  double c = std::ceil(static_cast<double>(cf) * static_cast<double>(T) / static_cast<double>(E));
  if (c < static_cast<double>(min_cap)) c = static_cast<double>(min_cap);
  return c >= static_cast<double>(INT32_MAX) ? INT32_MAX : static_cast<int>(c);
}

// cap = max(ceil(cf T / E), min_cap) in double when cf > 0, else unlimited
Problem make_problem(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t S, moe_dtype_t dt,
                     float cf, int act = MOE_ACT_GELU, int32_t min_cap = 0) {
  Problem p;
  p.T = T;
  p.d = d;
  p.h = h;
  p.E = E;
  p.k = k;
  p.S = S;
  p.dtype = dt;
  p.act = act;
  p.mx = false;
  p.ec_C = 0;
  p.A = T * k;
  p.rtile = router_tile(p);
  p.ntile = (T + p.rtile - 1) / p.rtile;
  p.cap = cf > 0.f ? capacity_of(cf, T, E, min_cap) : INT32_MAX;
  p.gemm_bm = gemm_m_tile(p);
  p.gemm_mixed = false;
  p.part_limit = kGemmPartCap;
  p.packed_w = false;
  return p;
}

// Expert choice: every expert takes exactly C tokens, so C is also its
// capacity and the routed rows are E * C.
moe_status_t check_shape_ec(int32_t T, int32_t d, int32_t h, int32_t E, int32_t C, int32_t S, int dtype) {
  if (T < 1 || d < 1 || h < 1 || E < 1 || C < 1 || C > T || S < 0) return MOE_ERR_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > MOE_MAX_EXPERTS || S > MOE_MAX_SHARED) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0 || h % 8 != 0) return MOE_ERR_UNSUPPORTED;
  const long long rows = static_cast<long long>(E) * C + static_cast<long long>(S) * T;
  if (rows > INT32_MAX || static_cast<long long>(E) * T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!fits_buffer_ranges(T, d, h, E, rows, dtype)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Problem make_problem_ec(int32_t T, int32_t d, int32_t h, int32_t E, int32_t C, int32_t S, moe_dtype_t dt,
                        int act = MOE_ACT_GELU) {
  Problem p;
  p.T = T;
  p.d = d;
  p.h = h;
  p.E = E;
  p.k = 0;
  p.S = S;
  p.dtype = dt;
  p.act = act;
  p.mx = false;
  p.ec_C = C;
  p.A = E * C;
  p.rtile = router_tile(p);
  p.ntile = (T + p.rtile - 1) / p.rtile;
  p.cap = C;
  p.gemm_bm = gemm_m_tile(p);
  p.gemm_mixed = false;
  p.part_limit = kGemmPartCap;
  p.packed_w = false;
  return p;
}

// MXFP8 (bf16 activations, d and h multiples of 256: the MX GEMM's N tiles
// are 256 columns and its K stages 128 bytes).
moe_status_t check_shape_mx(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t S) {
  const moe_status_t sc = check_shape(T, d, h, E, k, S, MOE_BF16);
  if (sc != MOE_OK) return sc;
  if (d % 256 != 0 || h % 256 != 0) return MOE_ERR_UNSUPPORTED;
  const long long rows = static_cast<long long>(T) * k + static_cast<long long>(S) * T + 256;
  const long long widest = d > h ? d : h;
  if (rows * widest >= (1LL << 31) || static_cast<long long>(h) * d >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Tile heights of the MXFP8 GEMM: 256 rows when experts average >= 512 rows
// and the capacity allows as many (compute bound, as in the bf16 GEMM's
// gemm_m_tile); else each segment's own, 128 or 192 rows by the rows the scan
// finds it routed (mx_mixed_tile_height).  Those tiles stream their expert's
// weights, so an expert's tile count is what a height has to keep low, and
// only the routed counts show it: loads are often far from even.
Problem make_problem_mx(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t S, float cf, int act,
                        int32_t min_cap) {
  Problem p = make_problem(T, d, h, E, k, S, MOE_BF16, cf, act, min_cap);
  p.mx = true;
  const long long mean = (static_cast<long long>(p.A) + p.E - 1) / p.E;
  p.gemm_mixed = !(mean >= 512 && p.cap >= 512);
  p.gemm_bm = p.gemm_mixed ? 128 : 256;
  return p;
}

// Records the optional stage events (a NULL entry is skipped) and reports a
// failed launch by stage.
struct StageCheck {
  hipStream_t st;
  hipEvent_t* ev;
  int ei = 0;
  bool operator()(hipError_t e, const char* stage) {
    if (e == hipSuccess && ev != nullptr) {
      if (ev[ei] != nullptr) e = hipEventRecord(ev[ei], st);
      ++ei;
    }
    if (e != hipSuccess) {
      std::fprintf(stderr, "libmoe: %s failed: %s (%s)\n", stage, hipGetErrorName(e), hipGetErrorString(e));
      return false;
    }
    return true;
  }
};

}  // namespace

// The top-k layer on a given workspace (moe_forward: the caller's; moe_forward_noalloc:
// the library's fixed scratch), with part_limit float32 partial tiles for the GEMM's split tail.
moe_status_t forward_top_k(const void* x, const void* W_g, const void* W1, const void* b1, const void* W2,
                           const void* b2, int32_t E, int32_t k, float capacity_factor, int32_t n_shared, void* out,
                           int32_t* topk_idx, float* topk_w, float* aux_loss, const moe_launch_t* launch,
                           void* ws_base, size_t ws_bytes, int part_limit) {
  if (!x || !W_g || !W1 || !W2 || !out || !topk_idx || !topk_w || !aux_loss) return MOE_ERR_ARG;
  if (std::isnan(capacity_factor) || launch->min_capacity < 0) return MOE_ERR_ARG;
  if (launch->activation != MOE_ACT_GELU && launch->activation != MOE_ACT_SILU) return MOE_ERR_UNSUPPORTED;
  const moe_status_t sc = check_shape(launch->T, launch->d, launch->h, E, k, n_shared,
                                      static_cast<int>(launch->dtype));
  if (sc != MOE_OK) return sc;
  const void* a16[] = {x, W_g, W1, b1, W2, b2, out};
  for (const void* q : a16)
    if (q && !aligned(q, 16)) return MOE_ERR_UNSUPPORTED;
  const void* a4[] = {topk_idx, topk_w, aux_loss, launch->z_loss, launch->b_g, launch->b_sel, launch->expert_counts,
                      launch->expert_kept, launch->slot_pos};
  for (const void* q : a4)
    if (q && !aligned(q, 4)) return MOE_ERR_UNSUPPORTED;

  Problem p = make_problem(launch->T, launch->d, launch->h, E, k, n_shared, launch->dtype, capacity_factor,
                           launch->activation, launch->min_capacity);
  p.part_limit = part_limit;
  if (launch->weights_packed != 0) {
    if (launch->weights_packed != 1 || !gemm_fast_path(p)) return MOE_ERR_UNSUPPORTED;
    p.packed_w = true;
  }
  bool ok = false;
  Workspace ws = carve_workspace(p, ws_base, ws_bytes, &ok);
  if (!ok) return MOE_ERR_WORKSPACE;
  if (launch->slot_pos) ws.slot_pos = launch->slot_pos;

  hipStream_t st = launch->stream;
  StageCheck check{st, launch->stage_events};
  // a stale error from an earlier, unrelated HIP call must not be blamed on a launch here
  (void)hipGetLastError();

  if (!check(hipSuccess, "stage event")) return MOE_ERR_HIP;
  if (!check(launch_router(p, x, W_g, launch->b_g, launch->b_sel, topk_idx, topk_w, ws, st), "router launch")) return MOE_ERR_HIP;
  // one permute kernel: the scan and scatter stage boundaries are both recorded after it
  if (!check(launch_permute(p, topk_idx, ws, aux_loss, launch->z_loss, launch->expert_counts, launch->expert_kept, st),
             "permute launch"))
    return MOE_ERR_HIP;
  if (!check(hipSuccess, "stage event")) return MOE_ERR_HIP;
  if (!check(launch_expert_ffn(p, x, W1, b1, W2, b2, ws, 1, st), "expert phase 1 launch")) return MOE_ERR_HIP;
  if (!check(launch_expert_ffn(p, x, W1, b1, W2, b2, ws, 2, st), "expert phase 2 launch")) return MOE_ERR_HIP;
  if (!check(launch_combine(p, topk_w, ws, out, st), "combine launch")) return MOE_ERR_HIP;
  return MOE_OK;
}

// ---------------------------------------------------- fixed device scratch --
// The workspace of moe_forward_noalloc: one array per GPU, allocated when the
// code object is loaded on that GPU and held until the process ends.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in): the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

moe_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    std::fprintf(stderr, "libmoe: no usable current device for the fixed scratch (%s)\n", hipGetErrorName(e));
    return MOE_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      std::fprintf(stderr, "libmoe: hipGetSymbolAddress of the fixed scratch failed on device %d: %s (%s)\n", dev,
                   hipGetErrorName(e), hipGetErrorString(e));
      return MOE_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe

extern "C" {

size_t moe_workspace_bytes(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t n_shared,
                           moe_dtype_t dtype) {
  if (moe::check_shape(T, d, h, E, k, n_shared, static_cast<int>(dtype)) != MOE_OK) return 0;
  return moe::workspace_bytes(moe::make_problem(T, d, h, E, k, n_shared, dtype, 0.f));
}

size_t moe_workspace_bytes_mxfp8(int32_t T, int32_t d, int32_t h, int32_t E, int32_t k, int32_t n_shared) {
  if (moe::check_shape_mx(T, d, h, E, k, n_shared) != MOE_OK) return 0;
  return moe::workspace_bytes(moe::make_problem_mx(T, d, h, E, k, n_shared, 0.f, MOE_ACT_GELU, 0));
}

moe_status_t moe_quantize_mxfp8(const void* src, int32_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream) {
  using namespace moe;
  if (!src || !codes || !scales || rows < 1 || cols < 1) return MOE_ERR_ARG;
  if (cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned(src, 16) || !aligned(codes, 16)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = launch_mx_quantize(static_cast<const uint16_t*>(src), rows, cols, codes, scales, stream);
  if (e != hipSuccess) {
    std::fprintf(stderr, "libmoe: MXFP8 quantize launch failed: %s (%s)\n", hipGetErrorName(e), hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status_t moe_forward_mxfp8(const void* x, const void* W_g, const uint8_t* W1, const uint8_t* W1_scales,
                               const void* b1, const uint8_t* W2, const uint8_t* W2_scales, const void* b2,
                               int32_t E, int32_t k, float capacity_factor, int32_t n_shared, void* out,
                               int32_t* topk_idx, float* topk_w, float* aux_loss, const moe_launch_t* launch) {
  using namespace moe;
  if (launch == nullptr) return MOE_ERR_ARG;
  if (!x || !W_g || !W1 || !W1_scales || !W2 || !W2_scales || !out || !topk_idx || !topk_w || !aux_loss)
    return MOE_ERR_ARG;
  if (std::isnan(capacity_factor) || launch->min_capacity < 0) return MOE_ERR_ARG;
  if (launch->activation != MOE_ACT_GELU && launch->activation != MOE_ACT_SILU) return MOE_ERR_UNSUPPORTED;
  if (launch->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (launch->weights_packed != 0) return MOE_ERR_UNSUPPORTED;   // MX codes have their own layout
  const moe_status_t sc = check_shape_mx(launch->T, launch->d, launch->h, E, k, n_shared);
  if (sc != MOE_OK) return sc;
  const void* a16[] = {x, W_g, W1, W2, out, b1, b2};
  for (const void* q : a16)
    if (q && !aligned(q, 16)) return MOE_ERR_UNSUPPORTED;
  const void* a4[] = {W1_scales, W2_scales, topk_idx, topk_w, aux_loss, launch->z_loss, launch->b_g, launch->b_sel,
                      launch->expert_counts, launch->expert_kept, launch->slot_pos};
  for (const void* q : a4)
    if (q && !aligned(q, 4)) return MOE_ERR_UNSUPPORTED;

  const Problem p = make_problem_mx(launch->T, launch->d, launch->h, E, k, n_shared, capacity_factor,
                                    launch->activation, launch->min_capacity);
  bool ok = false;
  Workspace ws = carve_workspace(p, launch->workspace, launch->workspace_bytes, &ok);
  if (!ok) return MOE_ERR_WORKSPACE;
  if (launch->slot_pos) ws.slot_pos = launch->slot_pos;
  const MxWeights w{W1, W1_scales, b1, W2, W2_scales, b2};

  hipStream_t st = launch->stream;
  StageCheck check{st, launch->stage_events};
  (void)hipGetLastError();
  if (!check(hipSuccess, "stage event")) return MOE_ERR_HIP;
  if (!check(launch_router(p, x, W_g, launch->b_g, launch->b_sel, topk_idx, topk_w, ws, st), "router launch")) return MOE_ERR_HIP;
  // one permute kernel: the scan and scatter stage boundaries are both recorded after it
  if (!check(launch_permute(p, topk_idx, ws, aux_loss, launch->z_loss, launch->expert_counts, launch->expert_kept, st),
             "permute launch"))
    return MOE_ERR_HIP;
  if (!check(hipSuccess, "stage event")) return MOE_ERR_HIP;
  // expert phase 1 stage: quantize x, then the first Linear
  const hipError_t qe = launch_mx_quantize(static_cast<const uint16_t*>(x), p.T, p.d, ws.xq, ws.xq_scales, st);
  if (qe != hipSuccess) {
    std::fprintf(stderr, "libmoe: MXFP8 quantize launch failed: %s (%s)\n", hipGetErrorName(qe), hipGetErrorString(qe));
    return MOE_ERR_HIP;
  }
  if (!check(launch_expert_ffn_mx(p, w, ws, 1, st), "expert phase 1 launch")) return MOE_ERR_HIP;
  if (!check(launch_expert_ffn_mx(p, w, ws, 2, st), "expert phase 2 launch")) return MOE_ERR_HIP;
  if (!check(launch_combine(p, topk_w, ws, out, st), "combine launch")) return MOE_ERR_HIP;
  return MOE_OK;
}

int32_t moe_expert_choice_capacity(float capacity_factor, int32_t T, int32_t E, int32_t min_capacity) {
  if (!(capacity_factor > 0.f) || T < 1 || E < 1 || min_capacity < 0) return -1;
  const int c = moe::capacity_of(capacity_factor, T, E, min_capacity);
  return c < T ? (c < 1 ? 1 : c) : T;
}

size_t moe_workspace_bytes_expert_choice(int32_t T, int32_t d, int32_t h, int32_t E, int32_t C, int32_t n_shared,
                                         moe_dtype_t dtype) {
  if (moe::check_shape_ec(T, d, h, E, C, n_shared, static_cast<int>(dtype)) != MOE_OK) return 0;
  return moe::workspace_bytes(moe::make_problem_ec(T, d, h, E, C, n_shared, dtype));
}

moe_status_t moe_pack_weights(const void* W, int32_t n_mat, int32_t N, int32_t K, moe_dtype_t dtype, void* Wp,
                              hipStream_t stream) {
  using namespace moe;
  if (W == nullptr || Wp == nullptr || n_mat < 1 || N < 1 || K < 1) return MOE_ERR_ARG;
  if (dtype != MOE_BF16 || N % 256 != 0 || K % 256 != 0) return MOE_ERR_UNSUPPORTED;
  // each matrix within one buffer descriptor's 32-bit range (the GEMM's B
  // operand), and a launchable number of 32 KB blocks
  if (static_cast<long long>(N) * K * 2 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  const long long elems = static_cast<long long>(n_mat) * N * K;
  if (elems / 16384 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (!aligned(W, 16) || !aligned(Wp, 16)) return MOE_ERR_UNSUPPORTED;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(W), b0 = reinterpret_cast<uintptr_t>(Wp);
  const uintptr_t len = static_cast<uintptr_t>(elems) * 2u;
  if (a0 < b0 + len && b0 < a0 + len) return MOE_ERR_ARG;   // overlapping buffers
  (void)hipGetLastError();
  const hipError_t e = launch_pack_weights(W, n_mat, N, K, Wp, stream);
  if (e != hipSuccess) {
    std::fprintf(stderr, "libmoe: weight packing launch failed: %s\n", hipGetErrorName(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument (null pointer or size out of range)";
    case MOE_ERR_UNSUPPORTED:
      return "MOE_ERR_UNSUPPORTED: unsupported shape, dtype, activation or pointer alignment";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: the problem needs more scratch than moe_forward_noalloc's fixed buffer";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_forward(const void* x, const void* W_g, const void* W1, const void* b1, const void* W2,
                         const void* b2, int32_t E, int32_t k, float capacity_factor, int32_t n_shared,
                         void* out, int32_t* topk_idx, float* topk_w, float* aux_loss,
                         const moe_launch_t* launch) {
  if (launch == nullptr) return MOE_ERR_ARG;
  return moe::forward_top_k(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w,
                            aux_loss, launch, launch->workspace, launch->workspace_bytes, moe::kGemmPartCap);
}

moe_status_t moe_forward_noalloc(const void* x, const void* W_g, const void* W1, const void* b1, const void* W2,
                                 const void* b2, int32_t E, int32_t k, float capacity_factor, int32_t n_shared,
                                 void* out, int32_t* topk_idx, float* topk_w, float* aux_loss,
                                 const moe_launch_t* launch) {
  using namespace moe;
  if (launch == nullptr) return MOE_ERR_ARG;
  // the scratch size is checked before any HIP call (forward_top_k checks the rest)
  const moe_status_t sc = check_shape(launch->T, launch->d, launch->h, E, k, n_shared,
                                      static_cast<int>(launch->dtype));
  if (sc != MOE_OK) return sc;
  if (std::isnan(capacity_factor) || launch->min_capacity < 0) return MOE_ERR_ARG;
  Problem p = make_problem(launch->T, launch->d, launch->h, E, k, n_shared, launch->dtype, capacity_factor,
                           launch->activation, launch->min_capacity);
  p.part_limit = kNoallocPartTiles;
  if (workspace_bytes(p) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* base = nullptr;
  const moe_status_t ss = scratch_of_current_device(&base);
  if (ss != MOE_OK) return ss;
  return forward_top_k(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w, aux_loss,
                       launch, base, MOE_NOALLOC_SCRATCH_BYTES, kNoallocPartTiles);
}

moe_status_t moe_forward_expert_choice(const void* x, const void* W_g, const void* W1, const void* b1,
                                       const void* W2, const void* b2, int32_t E, int32_t C, int32_t n_shared,
                                       void* out, int32_t* ec_token, float* ec_w, float* aux_loss,
                                       const moe_launch_t* launch) {
  using namespace moe;
  if (launch == nullptr) return MOE_ERR_ARG;
  if (!x || !W_g || !W1 || !W2 || !out || !ec_token || !ec_w) return MOE_ERR_ARG;
  if (launch->activation != MOE_ACT_GELU && launch->activation != MOE_ACT_SILU) return MOE_ERR_UNSUPPORTED;
  const moe_status_t sc = check_shape_ec(launch->T, launch->d, launch->h, E, C, n_shared,
                                         static_cast<int>(launch->dtype));
  if (sc != MOE_OK) return sc;
  const void* a16[] = {x, W_g, W1, b1, W2, b2, out};
  for (const void* q : a16)
    if (q && !aligned(q, 16)) return MOE_ERR_UNSUPPORTED;
  const void* a4[] = {ec_token, ec_w, aux_loss, launch->z_loss, launch->b_g, launch->b_sel, launch->expert_counts,
                      launch->expert_kept};
  for (const void* q : a4)
    if (q && !aligned(q, 4)) return MOE_ERR_UNSUPPORTED;

  Problem p = make_problem_ec(launch->T, launch->d, launch->h, E, C, n_shared, launch->dtype, launch->activation);
  if (launch->weights_packed != 0) {
    if (launch->weights_packed != 1 || !gemm_fast_path(p)) return MOE_ERR_UNSUPPORTED;
    p.packed_w = true;
  }
  bool ok = false;
  Workspace ws = carve_workspace(p, launch->workspace, launch->workspace_bytes, &ok);
  if (!ok) return MOE_ERR_WORKSPACE;

  hipStream_t st = launch->stream;
  StageCheck check{st, launch->stage_events};
  (void)hipGetLastError();
  if (!check(hipSuccess, "stage event")) return MOE_ERR_HIP;
  if (!check(launch_router(p, x, W_g, launch->b_g, nullptr, nullptr, nullptr, ws, st), "router launch")) return MOE_ERR_HIP;
  if (!check(launch_scan(p, ws, aux_loss, launch->z_loss, launch->expert_counts, launch->expert_kept, st),
             "scan launch"))
    return MOE_ERR_HIP;
  if (!check(launch_ec_select(p, ec_token, ec_w, ws, st), "expert-choice selection launch")) return MOE_ERR_HIP;
  if (!check(launch_expert_ffn(p, x, W1, b1, W2, b2, ws, 1, st), "expert phase 1 launch")) return MOE_ERR_HIP;
  if (!check(launch_expert_ffn(p, x, W1, b1, W2, b2, ws, 2, st), "expert phase 2 launch")) return MOE_ERR_HIP;
  if (!check(launch_combine_ec(p, ec_w, ws, out, st), "combine launch")) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // extern "C"
