// moe_router: router logits, softmax, top-k, renormalisation, per-tile sums of
// the softmax probabilities (the P_e of the balance loss) and, for the permute,
// per-tile expert histograms and in-tile token-order ranks.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (router linear, softmax,
// top-k, divide the k scores by their sum) and §4.3 (balance loss from the mean
// router probability); "[BEE-30064] 混合專家架構與服務", how routing works
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
  int32_t* topk_idx;
  float* topk_w;
  int32_t* local_rank;
  int32_t* tile_hist;
  float* p_part;
  int T, d, E, k, ntile;
};

// 16-lane argmax: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax16(double& v, int& i) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    double ov = __shfl_xor(v, m, 16);
    int oi = __shfl_xor(i, m, 16);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
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

// Selection, weights, probability partials and ranks for one 64-token tile,
// given the logits acc[nb][v] in the layout described at the top.
template <int NB>
__device__ void route_tile(const RouterArgs& a, double (&acc)[NB][4], int tile0) {
  __shared__ int32_t s_idx[kRouterTile * MOE_MAX_TOPK];
  __shared__ unsigned long long s_mask[16 * NB];
  __shared__ float s_p[4][16 * NB];

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

    // k rounds of a 16-lane argmax over the not-yet-chosen experts
    uint32_t taken = 0;
    int my_idx = 0;
    float my_e = 0.f;
    float esum = 0.f;
    for (int j = 0; j < k; ++j) {
      double bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int e = nb * 16 + c;
        if (e < E && !((taken >> nb) & 1u) && val[nb] > bv) { bv = val[nb]; bi = e; }
      }
      argmax16(bv, bi);
      if ((bi & 15) == c) taken |= 1u << (bi >> 4);
      const float ej = __expf(static_cast<float>(bv - m));
      esum += ej;
      if (c == j) { my_idx = bi; my_e = ej; }
    }
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
  // In-tile ranks in token order.  mask[e] has bit r set iff token r of the
  // tile chose e (a token's k experts are distinct, and OR is order-free, so
  // the masks are deterministic); the rank of (r, j) is the number of earlier
  // tokens in its expert's mask, the tile histogram the mask's population.
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0ull;
  __syncthreads();
  if (threadIdx.x < ntok) {
    const int r = threadIdx.x;
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[s_idx[r * MOE_MAX_TOPK + j]], 1ull << r);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // per-expert layout [E][ntile]: the scan reads each expert's tiles contiguously
    a.p_part[static_cast<size_t>(e) * a.ntile + tile] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
    a.tile_hist[static_cast<size_t>(e) * a.ntile + tile] = __popcll(s_mask[e]);
  }
  for (int i = threadIdx.x; i < ntok * k; i += blockDim.x) {
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
// Logits.  A workgroup (4 waves) owns TT = 64 / KS tokens and ES = 16 * NBW
// experts; the KS waves that share 16 tokens split the blocks of P k-steps
// (32 elements each) of d round-robin.  Operands go straight from memory into
// registers (x rows once per expert slice; the router weight from L2), two
// blocks in flight, 16x16x32 MFMA in float32 per block (<= 256 elements),
// blocks added in float64, the KS partials summed in float64 in fixed order.
// Output: float64 logits [T, Epad].
constexpr uint32_t kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

struct LogitArgs {
  const uint16_t* x;
  const uint16_t* W;
  double* logits;   // [T, Epad]
  int T, d, E, Epad;
};

template <int NBW, int KS>
__global__ __launch_bounds__(256) void router_logits_kernel(LogitArgs a) {
  constexpr int ES = 16 * NBW;
  constexpr int TT = 64 / KS;
  constexpr int P = NBW == 1 ? 8 : (NBW == 2 ? 4 : 2);   // k-steps per block
  __shared__ double red[4][ES][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tg = wave / KS, kw = wave % KS;
  const int c = lane & 15, g = lane >> 4;
  const int tile0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * ES;
  const uint32_t rb = static_cast<uint32_t>(a.d) * 2u;   // bytes per row
  const int nrows = min(TT, a.T - tile0);
  const int nexp = min(ES, a.E - e0);
  // out-of-range token rows and expert rows read as zero (buffer range check)
  const __amdgpu_buffer_rsrc_t xs = rsrc(a.x + static_cast<size_t>(tile0) * a.d, static_cast<uint32_t>(nrows) * rb);
  const __amdgpu_buffer_rsrc_t ws = rsrc(a.W + static_cast<size_t>(e0) * a.d, static_cast<uint32_t>(max(nexp, 0)) * rb);
  const uint32_t xo = static_cast<uint32_t>(tg * 16 + c) * rb + g * 16;
  uint32_t wo[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wo[nb] = static_cast<uint32_t>(nb * 16 + c) * rb + g * 16;

  const int nblk = a.d / (32 * P);
  double acc[NBW][4];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[nb][v] = 0.0;

  u32x4 xa[2][P], wa[2][P][NBW];
  auto load = [&](int blk, int buf) {
    const uint32_t kb = static_cast<uint32_t>(blk) * (P * 64);
#pragma unroll
    for (int q = 0; q < P; ++q) {
      xa[buf][q] = __builtin_amdgcn_raw_buffer_load_b128(xs, xo, kb + q * 64, 0);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) wa[buf][q][nb] = __builtin_amdgcn_raw_buffer_load_b128(ws, wo[nb], kb + q * 64, 0);
    }
  };
  auto compute = [&](int buf) {
    floatx4 part[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) part[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        part[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[buf][q]),
                                                            __builtin_bit_cast(bf16x8, wa[buf][q][nb]), part[nb], 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[nb][v] += static_cast<double>(part[nb][v]);
  };
  // blocks kw, kw + KS, ...: two in flight, buffers alternate (unrolled by two
  // so that every register index is a compile-time constant)
  int blk = kw;
  if (blk < nblk) load(blk, 0);
  while (blk < nblk) {
    if (blk + KS < nblk) load(blk + KS, 1);
    compute(0);
    blk += KS;
    if (blk >= nblk) break;
    if (blk + KS < nblk) load(blk + KS, 0);
    compute(1);
    blk += KS;
  }

  // lane (c, g) holds tokens tg*16 + 4g + v and experts nb*16 + c
  if constexpr (KS == 1) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tile0 + tg * 16 + 4 * g + v;
        if (t < a.T) a.logits[static_cast<size_t>(t) * a.Epad + e0 + nb * 16 + c] = acc[nb][v];
      }
  } else {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][nb * 16 + c][4 * g + v] = acc[nb][v];
    __syncthreads();
    // 16 tokens per token group: sum the KS partials in wave order
    for (int i = threadIdx.x; i < TT * ES; i += blockDim.x) {
      const int tl = i / ES, e = i - tl * ES;
      const int grp = tl / 16, r = tl - grp * 16;
      double sum = 0.0;
#pragma unroll
      for (int q = 0; q < KS; ++q) sum += red[grp * KS + q][e][r];
      const int t = tile0 + tl;
      if (t < a.T) a.logits[static_cast<size_t>(t) * a.Epad + e0 + e] = sum;
    }
  }
}

// Selection from float64 logits [T, Epad] for one 64-token tile, one token
// per 16-lane group (1024 threads): lane c of token r's group holds experts
// nb * 16 + c.  Same results as route_tile, with 16 waves per tile instead of
// 4 so that few, wide tiles (small T, many experts) still fill the CUs.
constexpr int kSelectThreads = kRouterTile * 16;

template <int NB>
__global__ __launch_bounds__(kSelectThreads) void router_select_kernel(RouterArgs a, const double* logits, int Epad) {
  __shared__ int32_t s_idx[kRouterTile * MOE_MAX_TOPK];
  __shared__ unsigned long long s_mask[MOE_MAX_EXPERTS];
  __shared__ float s_p[kRouterTile][16 * NB + 1];

  const int c = threadIdx.x & 15;
  const int r = threadIdx.x >> 4;          // token within the tile
  const int tile0 = blockIdx.x * kRouterTile;
  const int t = tile0 + r;
  const bool tok_ok = t < a.T;             // uniform across the 16-lane group
  const int E = a.E, k = a.k;

  double val[NB];
  double m = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    double l = -INFINITY;
    if (e < E && tok_ok) l = logits[static_cast<size_t>(t) * Epad + e] + (a.b_g ? static_cast<double>(a.b_g[e]) : 0.0);
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

  // k rounds of a 16-lane argmax over the not-yet-chosen experts
  uint32_t taken = 0;
  int my_idx = 0;
  float my_e = 0.f;
  float esum = 0.f;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      if (e < E && !((taken >> nb) & 1u) && val[nb] > bv) { bv = val[nb]; bi = e; }
    }
    argmax16(bv, bi);
    if ((bi & 15) == c) taken |= 1u << (bi >> 4);
    const float ej = __expf(static_cast<float>(bv - m));
    esum += ej;
    if (c == j) { my_idx = bi; my_e = ej; }
  }
  if (c < k) {
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
  if (threadIdx.x < ntok) {
    const int rr = threadIdx.x;
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[s_idx[rr * MOE_MAX_TOPK + j]], 1ull << rr);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // probability sum over the tile's tokens in token order
    float ps = 0.f;
    for (int rr = 0; rr < ntok; ++rr) ps += s_p[rr][e];
    a.p_part[static_cast<size_t>(e) * a.ntile + tile] = ps;
    a.tile_hist[static_cast<size_t>(e) * a.ntile + tile] = __popcll(s_mask[e]);
  }
  for (int i = threadIdx.x; i < ntok * k; i += blockDim.x) {
    const int rr = i / k, j = i - rr * k;
    const unsigned long long below = (1ull << rr) - 1ull;
    a.local_rank[static_cast<size_t>(tile0 + rr) * k + j] = __popcll(s_mask[s_idx[rr * MOE_MAX_TOPK + j]] & below);
  }
}

template <int NBW, int KS>
hipError_t launch_logits(const Problem& p, const LogitArgs& la, hipStream_t st) {
  constexpr int ES = 16 * NBW;
  constexpr int TT = 64 / KS;
  dim3 grid((p.T + TT - 1) / TT, (p.E + ES - 1) / ES);
  hipLaunchKernelGGL((router_logits_kernel<NBW, KS>), grid, dim3(256), 0, st, la);
  return hipGetLastError();
}

template <int NBW>
hipError_t launch_logits_ks(const Problem& p, const LogitArgs& la, hipStream_t st) {
  constexpr int ES = 16 * NBW;
  const long long slices = (p.E + ES - 1) / ES;
  // smallest token tile (most split of d) that still gives >= 512 workgroups
  if (static_cast<long long>((p.T + 63) / 64) * slices >= 512) return launch_logits<NBW, 1>(p, la, st);
  if (static_cast<long long>((p.T + 31) / 32) * slices >= 512) return launch_logits<NBW, 2>(p, la, st);
  return launch_logits<NBW, 4>(p, la, st);
}

template <int NB>
hipError_t launch_select(const Problem& p, const RouterArgs& a, const double* logits, int Epad, hipStream_t st) {
  hipLaunchKernelGGL((router_select_kernel<NB>), dim3(p.ntile), dim3(kSelectThreads), 0, st, a, logits, Epad);
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

hipError_t launch_router(const Problem& p, const void* x, const void* W_g, const float* b_g,
                         int32_t* topk_idx, float* topk_w, const Workspace& ws, hipStream_t st) {
  RouterArgs a;
  a.x = x;
  a.W_g = W_g;
  a.b_g = b_g;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.local_rank = ws.local_rank;
  a.tile_hist = ws.tile_hist;
  a.p_part = ws.p_part;
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
    const int nbw = nb <= 1 ? 1 : (nb <= 2 ? 2 : 4);
    la.Epad = ((p.E + 16 * nbw - 1) / (16 * nbw)) * 16 * nbw;
    hipError_t e = nbw == 1 ? launch_logits_ks<1>(p, la, st)
                 : nbw == 2 ? launch_logits_ks<2>(p, la, st)
                            : launch_logits_ks<4>(p, la, st);
    if (e != hipSuccess) return e;
    if (nb <= 1) return launch_select<1>(p, a, la.logits, la.Epad, st);
    if (nb <= 2) return launch_select<2>(p, a, la.logits, la.Epad, st);
    if (nb <= 4) return launch_select<4>(p, a, la.logits, la.Epad, st);
    if (nb <= 8) return launch_select<8>(p, a, la.logits, la.Epad, st);
    return launch_select<16>(p, a, la.logits, la.Epad, st);
  }
  if (nb <= 1) return launch_nb<1>(p, a, st);
  if (nb <= 2) return launch_nb<2>(p, a, st);
  if (nb <= 4) return launch_nb<4>(p, a, st);
  if (nb <= 8) return launch_nb<8>(p, a, st);
  return launch_nb<16>(p, a, st);
}

}  // namespace moe
