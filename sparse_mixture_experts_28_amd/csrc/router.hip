// moe_router: router logits, softmax, top-k, renormalisation, per-tile sums of
// the softmax probabilities (the P_e of the balance loss) and of the squared
// log-sum-exp of the logits (the router z-loss) and, for the permute, per-tile
// expert histograms and in-tile token-order ranks.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (router linear, softmax,
// top-k, divide the k scores by their sum) and §4.3 (balance loss from the mean
// router probability; router z-loss, the mean squared log-sum-exp of the logits); "[BEE-30064] 混合專家架構與服務", how routing works
// (bias-free router, top-k, softmax over the k chosen); "第7章 Mixture of
// Experts" tensor-shape trace (the router is a small (B n) x d x N matmul).
//
// One workgroup = 64 tokens = 4 waves x 16 tokens.  Within a wave the logits of
// 16 tokens x (16 * NB) experts live in registers in the layout of the 16x16
// MFMA result: lane (c = lane % 16, g = lane / 16) holds tokens 4g..4g+3 of the
// wave for experts nb*16 + c, nb < NB.  Selection and softmax are 16-lane
// reductions; nothing but the final indices and weights is written to memory.
//
// Logit accuracy.  The top-k choice must agree with exact arithmetic whenever
// the k-th and (k+1)-th logits differ by >= 1e-6.  bf16 products are exact in
// float32; the MFMA sums run in float32 over chunks of 256 elements of d and
// the chunks are added in float64, so the error stays ~1e-7 at d = 7168.  The
// float32 path multiplies in float64 (exact for float32 operands) and
// accumulates in float64.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFlushSteps = 8;  // MFMA k-steps (of 32) per float32 chunk -> 256 elements

struct RouterArgs {
  const void* x;
  const void* W_g;
  const float* b_g;
  const float* b_sel;   // [E] selection-only bias, or nullptr
  int32_t* topk_idx;
  float* topk_w;
  int32_t* local_rank;
  int32_t* tile_hist;
  float* p_part;
  double* z_part;
  // expert-choice mode (ec_logits != nullptr): no top-k; the logits are
  // written expert-major [E][T] with each token's maximum and exponential sum
  double* ec_logits;
  double* ec_m;
  float* ec_z;
  int T, d, E, k, ntile;
};

// squared log-sum-exp of a token's logits from its maximum m and
// z = sum_e exp(l_e - m): (m + log z)^2 in float64
__device__ __forceinline__ double lse_sq(double m, float z) {
  const double lse = m + log(static_cast<double>(z));
  return lse * lse;
}

// Expert-choice mode: token t's logits (lane c of its 16-lane group holds
// experts nb * 16 + c) go to the expert-major table, its maximum and
// exponential sum to per-token arrays (the softmax of a chosen pair is
// rebuilt from them exactly as here).
template <int NB>
__device__ __forceinline__ void write_ec(const RouterArgs& a, const double (&val)[NB], double m, float z, int t,
                                         int c, bool tok_ok) {
  if (!tok_ok) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    if (e < a.E) a.ec_logits[static_cast<size_t>(e) * a.T + t] = val[nb];
  }
  if (c == 0) {
    a.ec_m[t] = m;
    a.ec_z[t] = z;
  }
}

// 16-lane argmax: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax16(double& v, int& i) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    double ov = __shfl_xor(v, m, 16);
    int oi = __shfl_xor(i, m, 16);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// argmax16 carrying a payload (the winner's plain logit when the ranking
// includes the selection-only bias)
__device__ __forceinline__ void argmax16p(double& v, int& i, double& pl) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    double ov = __shfl_xor(v, m, 16);
    int oi = __shfl_xor(i, m, 16);
    double op = __shfl_xor(pl, m, 16);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; pl = op; }
  }
}

__device__ __forceinline__ double max16(double v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmax(v, __shfl_xor(v, m, 16));
  return v;
}

__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m, 16);
  return v;
}

// k rounds of a 16-lane argmax over the not-yet-chosen experts (ties to the
// lower index), ranking the logits plus the selection-only bias when there is
// one; a chosen expert's weight numerator is exp(l - m) of its logit alone.
// Lane j < k ends with the j-th choice and its numerator; every lane with
// their sum.
template <int NB>
__device__ __forceinline__ void select_k(const RouterArgs& a, const double (&val)[NB], double m, int c, int& my_idx,
                                         float& my_e, float& esum) {
  const int E = a.E, k = a.k;
  double key[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    key[nb] = a.b_sel && e < E ? val[nb] + static_cast<double>(a.b_sel[e]) : val[nb];
  }
  uint32_t taken = 0;
  my_idx = 0;
  my_e = 0.f;
  esum = 0.f;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY, bl = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      if (e < E && !((taken >> nb) & 1u) && key[nb] > bv) { bv = key[nb]; bi = e; bl = val[nb]; }
    }
    argmax16p(bv, bi, bl);
    if ((bi & 15) == c) taken |= 1u << (bi >> 4);
    const float ej = __expf(static_cast<float>(bl - m));
    esum += ej;
    if (c == j) { my_idx = bi; my_e = ej; }
  }
}

// Selection, weights, probability partials and ranks for one 64-token tile,
// given the logits acc[nb][v] in the layout described at the top.
template <int NB>
__device__ void route_tile(const RouterArgs& a, double (&acc)[NB][4], int tile0) {
  __shared__ int32_t s_idx[kRouterTile * MOE_MAX_TOPK];
  __shared__ unsigned long long s_mask[16 * NB];
  __shared__ float s_p[4][16 * NB];
  __shared__ double s_z[kRouterTile];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int E = a.E, k = a.k;

  float pp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) pp[nb] = 0.f;

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = wave * 16 + g * 4 + v;   // token within the tile
    const int t = tile0 + r;
    const bool tok_ok = t < a.T;           // uniform across the 16-lane group
    double val[NB];
    double m = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      double l = -INFINITY;
      if (e < E) l = acc[nb][v] + (a.b_g ? static_cast<double>(a.b_g[e]) : 0.0);
      val[nb] = l;
      m = fmax(m, l);
    }
    m = max16(m);
    float ev[NB];
    float zl = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      ev[nb] = (nb * 16 + c < E) ? __expf(static_cast<float>(val[nb] - m)) : 0.f;
      zl += ev[nb];
    }
    const float z = sum16(zl);
    if (tok_ok) {
      const float inv = 1.f / z;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) pp[nb] += ev[nb] * inv;
    }
    if (c == 0) s_z[r] = tok_ok ? lse_sq(m, z) : 0.0;
    if (a.ec_logits) {
      write_ec(a, val, m, z, t, c, tok_ok);
      continue;
    }

    int my_idx;
    float my_e, esum;
    select_k<NB>(a, val, m, c, my_idx, my_e, esum);
    if (c < k) {
      s_idx[r * MOE_MAX_TOPK + c] = tok_ok ? my_idx : -1;
      if (tok_ok) {
        a.topk_idx[static_cast<size_t>(t) * k + c] = my_idx;
        a.topk_w[static_cast<size_t>(t) * k + c] = my_e / esum;
      }
    }
  }

  // probability sums: 4 rows per lane, then the 4 lane groups (fixed order)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float s = pp[nb];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (g == 0) s_p[wave][nb * 16 + c] = s;
  }
  __syncthreads();

  const int ntok = min(kRouterTile, a.T - tile0);
  const int tile = tile0 / kRouterTile;
  const bool ec = a.ec_logits != nullptr;
  // In-tile ranks in token order.  mask[e] has bit r set iff token r of the
  // tile chose e (a token's k experts are distinct, and OR is order-free, so
  // the masks are deterministic); the rank of (r, j) is the number of earlier
  // tokens in its expert's mask, the tile histogram the mask's population.
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();
  if (threadIdx.x < ntok && !ec) {
    const int r = threadIdx.x;
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[s_idx[r * MOE_MAX_TOPK + j]], 1ull << r);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // tile-major layout [ntile][E]: the scan's lanes take consecutive experts
    a.p_part[static_cast<size_t>(tile) * E + e] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
    if (!ec) a.tile_hist[static_cast<size_t>(tile) * E + e] = __popcll(s_mask[e]);
  }
  if (threadIdx.x == blockDim.x - 1) {
    // z-loss partial of the tile, tokens in order
    double zs = 0.0;
    for (int r = 0; r < ntok; ++r) zs += s_z[r];
    a.z_part[tile] = zs;
  }
  for (int i = threadIdx.x; i < (ec ? 0 : ntok * k); i += blockDim.x) {
    const int r = i / k, j = i - r * k;
    const unsigned long long below = (1ull << r) - 1ull;
    a.local_rank[static_cast<size_t>(tile0 + r) * k + j] = __popcll(s_mask[s_idx[r * MOE_MAX_TOPK + j]] & below);
  }
}

// ---- bf16 inputs: 16x16x32 MFMA, float32 chunks summed in float64 ----
template <int NB>
__global__ __launch_bounds__(kRouterThreads) void router_bf16_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int tile0 = blockIdx.x * kRouterTile;
  const int row = tile0 + wave * 16 + c;   // A-operand row of this lane
  const bool row_ok = row < a.T;
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(row_ok ? row : 0) * a.d;
  const uint16_t* W = static_cast<const uint16_t*>(a.W_g);

  double acc[NB][4];
  floatx4 part[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    part[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[nb][v] = 0.0;
  }

  const u32x4 zero = {0u, 0u, 0u, 0u};
  int step = 0;
  for (int k0 = 0; k0 < a.d; k0 += 32) {
    const int kk = k0 + 8 * g;
    const bool k_ok = kk < a.d;
    u32x4 av = (row_ok && k_ok) ? *reinterpret_cast<const u32x4*>(xr + kk) : zero;
    const bf16x8 af = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      u32x4 bv = (e < a.E && k_ok) ? *reinterpret_cast<const u32x4*>(W + static_cast<size_t>(e) * a.d + kk) : zero;
      part[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, bv), part[nb], 0, 0, 0);
    }
    if (++step == kFlushSteps) {
      step = 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[nb][v] += static_cast<double>(part[nb][v]);
        part[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[nb][v] += static_cast<double>(part[nb][v]);

  route_tile<NB>(a, acc, tile0);
}

// ---- float32 inputs: exact float64 products, float64 sums ----
template <int NB>
__global__ __launch_bounds__(kRouterThreads) void router_f32_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int tile0 = blockIdx.x * kRouterTile;
  const float* X = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.W_g);

  const float* xrow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = tile0 + wave * 16 + g * 4 + v;
    xrow[v] = X + static_cast<size_t>(t < a.T ? t : 0) * a.d;
  }
  double acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[nb][v] = 0.0;

  for (int kk = 0; kk < a.d; kk += 4) {
    float4 xv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) xv[v] = *reinterpret_cast<const float4*>(xrow[v] + kk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < a.E) wv = *reinterpret_cast<const float4*>(W + static_cast<size_t>(e) * a.d + kk);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        double s = acc[nb][v];
        s = fma(static_cast<double>(xv[v].x), static_cast<double>(wv.x), s);
        s = fma(static_cast<double>(xv[v].y), static_cast<double>(wv.y), s);
        s = fma(static_cast<double>(xv[v].z), static_cast<double>(wv.z), s);
        s = fma(static_cast<double>(xv[v].w), static_cast<double>(wv.w), s);
        acc[nb][v] = s;
      }
    }
  }
  route_tile<NB>(a, acc, tile0);
}

// ---- bf16 inputs, d % 256 == 0: logits kernel + selection kernel ----
//
// Logits.  A workgroup computes 128 tokens x 64 experts (16 when E <= 16) over one of KS
// contiguous ranges of d (split-K, so that small T or few experts still give
// ~256 workgroups).  Both operands reach LDS by direct loads (buffer_load ...
// lds) in 128-deep stages held in a 3-slot ring, so each workgroup reads its
// x rows and router-weight rows once from L2 (per-wave register loads read
// the weight once per wave and were bound by L2 requests).  Wave w owns
// tokens 32 w .. 32 w + 31 x all experts of the tile: 2 x (tile / 16) blocks of
// the 16x16x32 MFMA, float32 per 256-element chunk of d, chunks added in
// float64.  Output:
// float64 partial logits [KS][T][Epad]; the selection kernel adds the KS
// partials in order.

struct LogitArgs {
  const uint16_t* x;
  const uint16_t* W;
  double* logits;   // [KS][T][Epad]
  int T, d, E, Epad, KS;
};

constexpr int kLgTok = 128, kLgExp = 64, kLgK = 128;   // tile and stage depth (experts: 64, or 16 when E <= 16)
constexpr int kLgCh = kLgK / 8;                        // 16-byte chunks per stage row
// ring slots: as many stages as fit in 144 KB of LDS (3 of 48 KB at 64
// experts, 4 of 36 KB at 16), all but one in flight
template <int EXP>
constexpr int lg_slots() { return EXP == 16 ? 4 : 3; }

// LDS row of 16 chunks (256 bytes): logical chunk c of row r at c ^ (r & 15).
// Measured with an LDS probe on gfx950, the fragment reads (rows 0..15 of a
// block at chunks 4 s .. 4 s + 3 in the four 16-lane quarters) then have no
// bank conflicts.
__device__ __forceinline__ int lgswz(int row, int c) { return c ^ (row & 15); }

__device__ __forceinline__ void lg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt 0 only; direct loads are waited for by vmcnt
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int EXP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void router_logits_kernel(LogitArgs a) {
  constexpr int kStage = (kLgTok + EXP) * kLgCh;     // u32x4 per stage (48 KB at EXP = 64)
  constexpr int kLgLoads = (kLgTok + EXP) / 16;       // 1 KB direct loads per wave per stage
  constexpr int kEB = EXP / 16;                       // expert blocks per wave
  constexpr int NS = lg_slots<EXP>();
  __shared__ u32x4 lds[NS * kStage];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * kLgTok;
  const int e0 = blockIdx.y * EXP;
  const int ks = blockIdx.z;
  const uint32_t rb = static_cast<uint32_t>(a.d) * 2u;   // bytes per row
  const int nrows = min(kLgTok, a.T - tok0);
  const int nexp = min(EXP, a.E - e0);
  // out-of-range token and expert rows read as zero (buffer range check)
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(a.x + static_cast<size_t>(tok0) * a.d, static_cast<uint32_t>(nrows) * rb);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.W + static_cast<size_t>(e0) * a.d, static_cast<uint32_t>(max(nexp, 0)) * rb);
  const int nchunk = a.d / 256;                      // 256-element chunks of d
  const int c0 = ks * nchunk / a.KS, c1 = (ks + 1) * nchunk / a.KS;
  const int nst = (c1 - c0) * (256 / kLgK);          // stages of this split (>= 2)
  const uint32_t kbase = static_cast<uint32_t>(c0) * 512u;

  // direct loads: load i of wave w fills stage rows 16 i + 4 w + lane / 16 at
  // physical chunk lane % 16 (rows 0..127: x, 128..191: router weight)
  const int dr = 4 * wave + (lane >> 4);
  const uint32_t vo = static_cast<uint32_t>(dr) * rb + lgswz(dr, lane & 15) * 16;
  auto issue = [&](int st) {
    u32x4* base = lds + (st % NS) * kStage + (4 * wave) * kLgCh;
    const uint32_t kb = kbase + static_cast<uint32_t>(st) * (kLgK * 2);
#pragma unroll
    for (int i = 0; i < kLgLoads; ++i) {
      if (i < kLgTok / 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (__attribute__((address_space(3))) void*)(base + 16 * i * kLgCh),
                                                 16, vo, static_cast<uint32_t>(16 * i) * rb + kb, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ws, (__attribute__((address_space(3))) void*)(base + 16 * i * kLgCh), 16, vo,
            static_cast<uint32_t>(16 * (i - kLgTok / 16)) * rb + kb, 0, 0);
    }
  };

  const int rr = lane & 15, cg = lane >> 4;
  double acc[2][kEB][4];
  floatx4 part[2][kEB];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int eb = 0; eb < kEB; ++eb) {
      part[tb][eb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[tb][eb][v] = 0.0;
    }

#pragma unroll
  for (int sp = 0; sp < NS - 1; ++sp)
    if (sp < nst) issue(sp);
  for (int st = 0; st < nst; ++st) {
    // stage st landed (the up to NS - 2 stages after it may be in flight);
    // every wave is past stage st-1, whose slot then takes stage st + NS - 1
    if constexpr (NS == 4) {
      if (st + 2 < nst) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kLgLoads));
      else if (st + 1 < nst) __builtin_amdgcn_s_waitcnt(vm_wait_imm(kLgLoads));
      else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    } else {
      if (st + 1 < nst) __builtin_amdgcn_s_waitcnt(vm_wait_imm(kLgLoads));
      else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    lg_barrier();
    if (st + NS - 1 < nst) issue(st + NS - 1);
    const u32x4* sa = lds + (st % NS) * kStage;
#pragma unroll
    for (int s = 0; s < kLgK / 32; ++s) {
      const int ch = lgswz(rr, 4 * s + cg);
      bf16x8 xf[2], wf[kEB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        xf[tb] = __builtin_bit_cast(bf16x8, sa[(32 * wave + 16 * tb + rr) * kLgCh + ch]);
#pragma unroll
      for (int eb = 0; eb < kEB; ++eb)
        wf[eb] = __builtin_bit_cast(bf16x8, sa[(kLgTok + 16 * eb + rr) * kLgCh + ch]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int eb = 0; eb < kEB; ++eb)
          part[tb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[tb], wf[eb], part[tb][eb], 0, 0, 0);
    }
    if (st & 1) {   // a 256-element chunk is complete: add it in float64
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int eb = 0; eb < kEB; ++eb) {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[tb][eb][v] += static_cast<double>(part[tb][eb][v]);
          part[tb][eb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
  }

  // lane (rr, cg) of block (tb, eb) holds tokens 32 w + 16 tb + 4 cg + v, expert 16 eb + rr
  double* out = a.logits + static_cast<size_t>(ks) * a.T * a.Epad;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = tok0 + 32 * wave + 16 * tb + 4 * cg + v;
      if (t < a.T) {
#pragma unroll
        for (int eb = 0; eb < kEB; ++eb) out[static_cast<size_t>(t) * a.Epad + e0 + 16 * eb + rr] = acc[tb][eb][v];
      }
    }
}

// Selection from float64 logits [T, Epad] for one 64-token tile, one token
// per 16-lane group (1024 threads): lane c of token r's group holds experts
// nb * 16 + c.  Same results as route_tile, with 16 waves per tile instead of
// 4 so that few, wide tiles (small T, many experts) still fill the CUs.
constexpr int kSelectThreads = kRouterTile * 16;

// The selection of one 64-token tile on 1024 threads (thread = token r =
// tid / 16, lane c = tid % 16 of its 16-lane group), from the logits lg[nb] of
// experts nb * 16 + c without the router bias (any value for e >= E).
template <int NB>
__device__ __forceinline__ void select_tile(const RouterArgs& a, const double (&lg)[NB], int tile0) {
  __shared__ int32_t s_idx[kRouterTile * MOE_MAX_TOPK];
  __shared__ unsigned long long s_mask[MOE_MAX_EXPERTS];
  __shared__ float s_p[kRouterTile][16 * NB + 1];
  __shared__ double s_z[kRouterTile];

  const int c = threadIdx.x & 15;
  const int r = threadIdx.x >> 4;          // token within the tile
  const int t = tile0 + r;
  const bool tok_ok = t < a.T;             // uniform across the 16-lane group
  const int E = a.E, k = a.k;

  double val[NB];
  double m = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    double l = -INFINITY;
    if (e < E && tok_ok) l = lg[nb] + (a.b_g ? static_cast<double>(a.b_g[e]) : 0.0);
    val[nb] = l;
    m = fmax(m, l);
  }
  m = max16(m);
  float ev[NB];
  float zl = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ev[nb] = (nb * 16 + c < E && tok_ok) ? __expf(static_cast<float>(val[nb] - m)) : 0.f;
    zl += ev[nb];
  }
  const float z = sum16(zl);
  const float inv = tok_ok ? 1.f / z : 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s_p[r][nb * 16 + c] = ev[nb] * inv;
  if (c == 0) s_z[r] = tok_ok ? lse_sq(m, z) : 0.0;
  const bool ec = a.ec_logits != nullptr;
  if (ec) write_ec(a, val, m, z, t, c, tok_ok);

  int my_idx = 0;
  float my_e = 0.f, esum = 0.f;
  if (!ec) select_k<NB>(a, val, m, c, my_idx, my_e, esum);
  if (c < k && !ec) {
    s_idx[r * MOE_MAX_TOPK + c] = tok_ok ? my_idx : -1;
    if (tok_ok) {
      a.topk_idx[static_cast<size_t>(t) * k + c] = my_idx;
      a.topk_w[static_cast<size_t>(t) * k + c] = my_e / esum;
    }
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();

  const int ntok = min(kRouterTile, a.T - tile0);
  const int tile = tile0 / kRouterTile;
  // In-tile ranks in token order, as in route_tile: OR-ed 64-bit token masks
  // per expert (order-free, so deterministic); rank = earlier tokens in the mask.
  if (threadIdx.x < ntok && !ec) {
    const int rr = threadIdx.x;
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[s_idx[rr * MOE_MAX_TOPK + j]], 1ull << rr);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // probability sum over the tile's tokens in token order
    float ps = 0.f;
    for (int rr = 0; rr < ntok; ++rr) ps += s_p[rr][e];
    a.p_part[static_cast<size_t>(tile) * E + e] = ps;
    if (!ec) a.tile_hist[static_cast<size_t>(tile) * E + e] = __popcll(s_mask[e]);
  }
  if (threadIdx.x == blockDim.x - 1) {
    // z-loss partial of the tile, tokens in order
    double zs = 0.0;
    for (int rr = 0; rr < ntok; ++rr) zs += s_z[rr];
    a.z_part[tile] = zs;
  }
  for (int i = threadIdx.x; i < (ec ? 0 : ntok * k); i += blockDim.x) {
    const int rr = i / k, j = i - rr * k;
    const unsigned long long below = (1ull << rr) - 1ull;
    a.local_rank[static_cast<size_t>(tile0 + rr) * k + j] = __popcll(s_mask[s_idx[rr * MOE_MAX_TOPK + j]] & below);
  }
}

template <int NB>
__global__ __launch_bounds__(kSelectThreads) void router_select_kernel(RouterArgs a, const double* logits, int Epad,
                                                                       int KS) {
  const int c = threadIdx.x & 15;
  const int tile0 = blockIdx.x * kRouterTile;
  const int t = tile0 + (threadIdx.x >> 4);
  double lg[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    double l = 0.0;
    if (e < a.E && t < a.T) {
      // the split-K partials, added in split order
      l = logits[static_cast<size_t>(t) * Epad + e];
      for (int q = 1; q < KS; ++q) l += logits[(static_cast<size_t>(q) * a.T + t) * Epad + e];
    }
    lg[nb] = l;
  }
  select_tile<NB>(a, lg, tile0);
}

template <int NB>
hipError_t launch_select(const Problem& p, const RouterArgs& a, const double* logits, int Epad, int KS,
                         hipStream_t st) {
  hipLaunchKernelGGL((router_select_kernel<NB>), dim3(p.ntile), dim3(kSelectThreads), 0, st, a, logits, Epad, KS);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_nb(const Problem& p, const RouterArgs& a, hipStream_t st) {
  dim3 grid(p.ntile), block(kRouterThreads);
  if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(router_bf16_kernel<NB>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(router_f32_kernel<NB>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

// expert padding of the logits: one 16-expert tile when E <= 16 (a quarter of
// the MFMA work and partial-logit traffic of a 64-expert tile), else 64s
int logit_pad(int E) { return E <= 16 ? 16 : (E + kLgExp - 1) / kLgExp * kLgExp; }

// d is split into KS ranges of whole 256-element chunks so the logits launch
// has ~256 workgroups (at most 8 splits, at least one chunk each)
int logit_splits(const Problem& p) {
  const int pad = logit_pad(p.E);
  const long long tiles = static_cast<long long>((p.T + kLgTok - 1) / kLgTok) * (pad / (pad == 16 ? 16 : kLgExp));
  long long ks = (256 + tiles - 1) / tiles;
  if (ks > 8) ks = 8;
  if (ks > p.d / 256) ks = p.d / 256;
  return ks < 1 ? 1 : static_cast<int>(ks);
}

hipError_t launch_router(const Problem& p, const void* x, const void* W_g, const float* b_g, const float* b_sel,
                         int32_t* topk_idx, float* topk_w, const Workspace& ws, hipStream_t st) {
  RouterArgs a;
  a.x = x;
  a.W_g = W_g;
  a.b_g = b_g;
  a.b_sel = p.ec_C > 0 ? nullptr : b_sel;   // no effect on expert choice
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.local_rank = ws.local_rank;
  a.tile_hist = ws.tile_hist;
  a.p_part = ws.p_part;
  a.z_part = ws.z_part;
  a.ec_logits = p.ec_C > 0 ? ws.ec_logits : nullptr;
  a.ec_m = ws.ec_m;
  a.ec_z = ws.ec_z;
  a.T = p.T;
  a.d = p.d;
  a.E = p.E;
  a.k = p.k;
  a.ntile = p.ntile;
  const int nb = (p.E + 15) / 16;
  if (p.dtype == MOE_BF16 && p.d % 256 == 0 && ws.logits != nullptr) {
    LogitArgs la;
    la.x = static_cast<const uint16_t*>(x);
    la.W = static_cast<const uint16_t*>(W_g);
    la.logits = ws.logits;
    la.T = p.T;
    la.d = p.d;
    la.E = p.E;
    la.Epad = logit_pad(p.E);
    la.KS = logit_splits(p);
    if (la.Epad == 16)
      hipLaunchKernelGGL(router_logits_kernel<16>, dim3((p.T + kLgTok - 1) / kLgTok, 1, la.KS), dim3(256), 0, st, la);
    else
      hipLaunchKernelGGL(router_logits_kernel<64>, dim3((p.T + kLgTok - 1) / kLgTok, la.Epad / kLgExp, la.KS),
                         dim3(256), 0, st, la);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nb <= 1) return launch_select<1>(p, a, la.logits, la.Epad, la.KS, st);
    if (nb <= 2) return launch_select<2>(p, a, la.logits, la.Epad, la.KS, st);
    if (nb <= 4) return launch_select<4>(p, a, la.logits, la.Epad, la.KS, st);
    if (nb <= 8) return launch_select<8>(p, a, la.logits, la.Epad, la.KS, st);
    return launch_select<16>(p, a, la.logits, la.Epad, la.KS, st);
  }
  if (nb <= 1) return launch_nb<1>(p, a, st);
  if (nb <= 2) return launch_nb<2>(p, a, st);
  if (nb <= 4) return launch_nb<4>(p, a, st);
  if (nb <= 8) return launch_nb<8>(p, a, st);
  return launch_nb<16>(p, a, st);
}

}  // namespace moe
