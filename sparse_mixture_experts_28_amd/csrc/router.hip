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

// 16-lane reductions through DPP row moves instead of LDS permutes (a
// ds_bpermute per value and step costs an LDS round trip on the selection's
// critical path).  The four steps exchange between lanes i and i ^ 1, i ^ 2
// (quad_perm), then between the two quads of each half row (row_half_mirror:
// lane i and 7 - i) and the two halves of the row (row_mirror: lane i and
// 15 - i).  After the first two steps a quad's lanes hold equal values, so
// the mirrors pair the same partial results as the exchanges i ^ 4 and i ^ 8,
// with each lane's own value on the same side of the operation: the results
// are those of the plain butterfly, bit for bit.  A DPP row is 16 lanes, the
// token's lane group.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = static_cast<unsigned>(dpp_i<CTRL>(static_cast<int>(static_cast<unsigned>(b))));
  const unsigned hi = static_cast<unsigned>(dpp_i<CTRL>(static_cast<int>(static_cast<unsigned>(b >> 32))));
  return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}

// one argmax step: the other lane's (value, index, payload) wins if its value
// is larger, or equal with a lower index
template <int CTRL>
__device__ __forceinline__ void argmax_step(double& v, int& i, double& pl) {
  const double ov = dpp_d<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  const double op = dpp_d<CTRL>(pl);
  const bool take = (ov > v) | ((ov == v) & (oi < i));   // selects, not an exec-masked branch
  v = take ? ov : v;
  i = take ? oi : i;
  pl = take ? op : pl;
}

// 16-lane argmax carrying a payload (the winner's plain logit when the
// ranking includes the selection-only bias): larger value wins, equal values
// go to the lower index
__device__ __forceinline__ void argmax16p(double& v, int& i, double& pl) {
  argmax_step<kDppXor1>(v, i, pl);
  argmax_step<kDppXor2>(v, i, pl);
  argmax_step<kDppHalfMirror>(v, i, pl);
  argmax_step<kDppMirror>(v, i, pl);
}

__device__ __forceinline__ double max16(double v) {
  v = fmax(v, dpp_d<kDppXor1>(v));
  v = fmax(v, dpp_d<kDppXor2>(v));
  v = fmax(v, dpp_d<kDppHalfMirror>(v));
  return fmax(v, dpp_d<kDppMirror>(v));
}

__device__ __forceinline__ double sum16d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  return v + dpp_d<kDppMirror>(v);
}

// sum over a wave: the 16-lane butterfly by DPP, then the exchanges across
// lane groups (i ^ 16, i ^ 32); every lane ends with the same value
__device__ __forceinline__ double wave_sum64(double v) {
  v = sum16d(v);
  v += __shfl_xor(v, 16, kWave);
  return v + __shfl_xor(v, 32, kWave);
}

__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

// k rounds of a 16-lane argmax over the not-yet-chosen experts (ties to the
// lower index), ranking the logits plus the selection-only bias when there is
// one; a chosen expert's weight numerator is exp(l - m) of its logit alone.
// Lane j < k ends with the j-th choice and its numerator; every lane with
// their sum.
//
// The choice is total: a NaN key ranks as -inf, and every not-yet-chosen
// expert is a candidate even when its key is -inf, so each round returns an
// expert in [0, E) (k <= E leaves one untaken).  A token whose logits are NaN
// (a NaN in its row of x, in W_g or in a bias) then gets valid indices and
// NaN weights, and the other tokens are unaffected.
template <int NB>
__device__ __forceinline__ void select_k(const RouterArgs& a, const double (&val)[NB], const double (&bsel)[NB],
                                         double m, int c, int& my_idx, float& my_e, float& esum) {
  const int E = a.E, k = a.k;
  double key[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    const double kv = a.b_sel && e < E ? val[nb] + bsel[nb] : val[nb];
    key[nb] = kv == kv ? kv : -INFINITY;
  }
  constexpr int kNone = 0x7fffffff;
  uint32_t taken = 0;
  my_idx = 0;
  my_e = 0.f;
  esum = 0.f;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY, bl = -INFINITY;
    int bi = kNone;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      // experts ascend with nb: the first untaken one is this lane's candidate
      // until a strictly larger key replaces it
      // (selects, not a branch: as an if-block the compiler emitted an
      // exec-masked branch per expert)
      const bool take = (e < E) & !((taken >> nb) & 1u) & ((bi == kNone) | (key[nb] > bv));
      bv = take ? key[nb] : bv;
      bi = take ? e : bi;
      bl = take ? val[nb] : bl;
    }
    argmax16p(bv, bi, bl);
    if ((bi & 15) == c) taken |= 1u << (bi >> 4);
    const float ej = __expf(static_cast<float>(bl - m));
    esum += ej;
    if (c == j) { my_idx = bi; my_e = ej; }
  }
}

// The lane's router offsets (b_g, 0 without one) and selection-only biases
// (b_sel) of experts nb * 16 + c, loaded together once per tile rather than
// one dependent load per expert and token.
// (The loads are unconditional at a clamped index inside a branch that is
// uniform across the workgroup, so they are all in flight before the first
// wait; lanes past E then take 0.)
template <int NB>
__device__ __forceinline__ void lane_bias(const float* b, int c, int E, double (&out)[NB]) {
  float v[NB];
  if (b != nullptr) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) v[nb] = b[min(nb * 16 + c, E - 1)];
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) v[nb] = 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) out[nb] = nb * 16 + c < E ? static_cast<double>(v[nb]) : 0.0;
}

template <int NB>
__device__ __forceinline__ void lane_biases(const RouterArgs& a, int c, double (&bg)[NB], double (&bs)[NB]) {
  lane_bias<NB>(a.b_g, c, a.E, bg);
  lane_bias<NB>(a.b_sel, c, a.E, bs);
}

// Selection, weights, probability partials and ranks for one tile of RT
// tokens (RT = 32 or 64; 4 waves, wave w holding tokens 16 w .. 16 w + 15 of
// the tile, so waves past RT / 16 hold none), given the logits acc[nb][v] in
// the layout described at the top.
//
// Its LDS tables live in `smem` (route_tile_smem<RT, NB>() bytes, 8-byte
// aligned), so a kernel whose main loop fills one LDS object by direct loads
// can hand it a part of that object: a second LDS object would make the
// compiler wait for every direct load in flight before each read of the first.
template <int RT, int NB>
constexpr int route_tile_smem() { return RT * 8 + 16 * NB * 8 + 4 * 16 * NB * 4 + RT * MOE_MAX_TOPK * 4; }

//
// VW = 1 (16-token tiles only): the tile's selection is spread over the four
// waves, wave w holding in acc[nb][0] the logits of tokens 4 g + w (its
// 16-lane group g), so each wave selects four tokens instead of wave 0
// selecting all sixteen.
template <int RT, int NB, int VW = 4>
__device__ void route_tile(const RouterArgs& a, double (&acc)[NB][4], int tile0, unsigned char* smem) {
  static_assert(RT == 16 || RT == 32 || RT == 64, "router tiles are 16, 32 or 64 tokens");
  static_assert(VW == 4 || (VW == 1 && RT == 16), "spread selection is for 16-token tiles");
  double* s_z = reinterpret_cast<double*>(smem);                                        // [RT]
  unsigned long long* s_mask = reinterpret_cast<unsigned long long*>(smem + RT * 8);      // [16 NB]
  float (*s_p)[16 * NB] = reinterpret_cast<float (*)[16 * NB]>(smem + RT * 8 + 16 * NB * 8);   // [4][16 NB]
  int32_t* s_idx = reinterpret_cast<int32_t*>(smem + RT * 8 + 16 * NB * 8 + 4 * 16 * NB * 4);  // [RT * MOE_MAX_TOPK]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int E = a.E, k = a.k;

  float pp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) pp[nb] = 0.f;
  double bg[NB], bs[NB];
  lane_biases<NB>(a, c, bg, bs);

#pragma unroll
  for (int v = 0; v < VW; ++v) {
    const int r = VW == 1 ? g * 4 + wave : wave * 16 + g * 4 + v;   // token within the tile
    const int t = tile0 + r;
    const bool in_tile = r < RT;           // uniform across the wave
    const bool tok_ok = in_tile && t < a.T;   // uniform across the 16-lane group
    double val[NB];
    double m = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      double l = -INFINITY;
      if (e < E) l = acc[nb][v] + bg[nb];
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
    if (c == 0 && in_tile) s_z[r] = tok_ok ? lse_sq(m, z) : 0.0;
    if (a.ec_logits) {
      write_ec(a, val, m, z, t, c, tok_ok);
      continue;
    }

    int my_idx;
    float my_e, esum;
    select_k<NB>(a, val, bs, m, c, my_idx, my_e, esum);
    if (c < k && in_tile) {
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

  const int ntok = min(RT, a.T - tile0);
  const int tile = tile0 / RT;
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
  if (threadIdx.x < kWave) {
    // z-loss partial of the tile: a fixed butterfly over the tile's tokens
    const double zs = wave_sum64(threadIdx.x < ntok ? s_z[threadIdx.x] : 0.0);
    if (threadIdx.x == 0) a.z_part[tile] = zs;
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

  __shared__ __align__(8) unsigned char smem[route_tile_smem<kRouterTile, NB>()];
  route_tile<kRouterTile, NB>(a, acc, tile0, smem);
}

// ---- float32 inputs: exact float64 products, float64 sums ----
// RT = 64: wave w holds tokens 16 w .. 16 w + 15 over all of d.  RT = 16 (at
// most 64 experts, few tokens): the four waves share the tile's 16 tokens and
// take every fourth group of four columns of d; their float64 sums are added
// in LDS in wave order, so small batches still fill the GPU.
template <int RT, int NB>
__global__ __launch_bounds__(kRouterThreads) void router_f32_kernel(RouterArgs a) {
  static_assert(RT == 64 || (RT == 16 && NB <= 4), "float32 router tiles");
  constexpr int KW = RT == 16 ? 4 : 1;   // waves sharing a token block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int tile0 = blockIdx.x * RT;
  const int tb = KW == 1 ? wave : 0, kw = KW == 1 ? 0 : wave;
  const float* X = static_cast<const float*>(a.x);
  const uint32_t rb = static_cast<uint32_t>(a.d) * 4u;   // bytes per row
  // buffer loads: token rows past T and router rows past E read zero (range
  // check); the lane offsets stay fixed over the loop and the column offset is
  // scalar, so no address registers are rewritten while loads are in flight
  const __amdgpu_buffer_rsrc_t xs =
      make_rsrc(X + static_cast<size_t>(tile0) * a.d, static_cast<uint32_t>(min(RT, a.T - tile0)) * rb);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.W_g, static_cast<uint32_t>(a.E) * rb);
  uint32_t xo[4], wo[NB];
#pragma unroll
  for (int v = 0; v < 4; ++v) xo[v] = static_cast<uint32_t>(tb * 16 + g * 4 + v) * rb;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wo[nb] = static_cast<uint32_t>(nb * 16 + c) * rb;
  double acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[nb][v] = 0.0;

  // The loads of later groups of four columns are issued before this group's
  // products (a group past d re-reads column 0 and is never folded).
  auto load = [&](int kk, float4 (&xv)[4], float4 (&wv)[NB]) {
    const uint32_t ko = static_cast<uint32_t>(kk < a.d ? kk : 0) * 4u;
#pragma unroll
    for (int v = 0; v < 4; ++v) xv[v] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xs, xo[v], ko, 0));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      wv[nb] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ws, wo[nb], ko, 0));
  };
  auto fold = [&](const float4 (&xv)[4], const float4 (&wv)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        double s = acc[nb][v];
        s = fma(static_cast<double>(xv[v].x), static_cast<double>(wv[nb].x), s);
        s = fma(static_cast<double>(xv[v].y), static_cast<double>(wv[nb].y), s);
        s = fma(static_cast<double>(xv[v].z), static_cast<double>(wv[nb].z), s);
        s = fma(static_cast<double>(xv[v].w), static_cast<double>(wv[nb].w), s);
        acc[nb][v] = s;
      }
  };
  // four column groups in registers: group i is folded while groups i+1 ..
  // i+3 are in flight (one group ahead left each fold waiting for its loads:
  // at the switch-shaped layer the kernel took 45 us against ~6 us of float64
  // arithmetic).  Only groups inside d are folded.
  float4 x0[4], w0[NB], x1[4], w1[NB], x2[4], w2[NB], x3[4], w3[NB];
  constexpr int GS = 4 * KW;                   // columns between a wave's groups
  int kk = __builtin_amdgcn_readfirstlane(4 * kw);   // wave-uniform: the loop exits are scalar branches
  load(kk, x0, w0);
  load(kk + GS, x1, w1);
  load(kk + 2 * GS, x2, w2);
  // (the scheduling barriers keep each group's loads ahead of the products
  // that precede them in program order; without them the loads sank below the
  // products and each fold waited for every load in flight)
  for (; kk < a.d; kk += 4 * GS) {
    load(kk + 3 * GS, x3, w3);
    __builtin_amdgcn_sched_barrier(0);
    fold(x0, w0);
    if (kk + GS >= a.d) break;
    load(kk + 4 * GS, x0, w0);
    __builtin_amdgcn_sched_barrier(0);
    fold(x1, w1);
    if (kk + 2 * GS >= a.d) break;
    load(kk + 5 * GS, x1, w1);
    __builtin_amdgcn_sched_barrier(0);
    fold(x2, w2);
    if (kk + 3 * GS >= a.d) break;
    load(kk + 6 * GS, x2, w2);
    __builtin_amdgcn_sched_barrier(0);
    fold(x3, w3);
  }
  __shared__ __align__(8) unsigned char smem[route_tile_smem<RT, NB>()];
  if constexpr (KW > 1) {
    // wave w adds the four waves' sums of tokens 4 g + w in wave order and
    // selects those four tokens (route_tile's spread layout)
    __shared__ double red[KW * NB * 4 * 64];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((wave * NB + nb) * 4 + v) * 64 + lane] = acc[nb][v];
    __syncthreads();
    double sel[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      double s = red[((0 * NB + nb) * 4 + wave) * 64 + lane];
      for (int w = 1; w < KW; ++w) s += red[((w * NB + nb) * 4 + wave) * 64 + lane];
      sel[nb][0] = s;
    }
    route_tile<RT, NB, 1>(a, sel, tile0, smem);
  } else {
    route_tile<RT, NB>(a, acc, tile0, smem);
  }
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
  // start at different even stages per token tile and wrap, spreading the
  // concurrent reads over d (the split's chunk order changes, chunks stay whole)
  const int s0 = (2 * static_cast<int>(blockIdx.x)) % nst;

  // direct loads: load i of wave w fills stage rows 16 i + 4 w + lane / 16 at
  // physical chunk lane % 16 (rows 0..127: x, 128..191: router weight)
  const int dr = 4 * wave + (lane >> 4);
  const uint32_t vo = static_cast<uint32_t>(dr) * rb + lgswz(dr, lane & 15) * 16;
  auto issue = [&](int st) {
    u32x4* base = lds + (st % NS) * kStage + (4 * wave) * kLgCh;
    const int sc = st + s0 < nst ? st + s0 : st + s0 - nst;
    const uint32_t kb = kbase + static_cast<uint32_t>(sc) * (kLgK * 2);
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

// ---- bf16 inputs, d % 256 == 0, E <= 64: one fused launch ----
//
// A workgroup owns RT tokens (32 or 64, so that a launch has ~256
// workgroups) and every expert (padded to EXP = 16 or 64), over all of d, so
// the selection follows in the same workgroup with the logits in registers:
// no partial logits leave the CU.  x rows and router-weight rows reach LDS
// by direct loads in 128-deep stages through an NS-slot ring (NS - 1 stages
// in flight, up to ~100 KB per CU, so the stream of x is not bound by the
// memory latency); x is read once, the router weight (<= 64 rows) from L2.
// Wave w takes token block tb = w % TB (TB = RT / 16) and, when RT = 32, half
// of each stage's four 32-deep k-steps (kq = w / TB); the two halves' float64
// sums are added in LDS (kq 0 then kq 1) before the selection, which runs on
// waves 0 .. TB-1 in the layout of route_tile.  float32 MFMA sums over each
// 256-element chunk of d, chunks added in float64, as in the other paths.
template <int RT, int EXP>
constexpr int fused_slots() {
  return (144 * 1024) / ((RT + EXP) * kLgK * 2) > 12 ? 12 : (144 * 1024) / ((RT + EXP) * kLgK * 2);
}

// wait until at most s stages of L direct loads each are in flight (s uniform)
template <int L, int S>
__device__ __forceinline__ void wait_stages(int s) {
  if constexpr (S > 0) {
    if (s >= S) {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(S * L));
      return;
    }
    wait_stages<L, S - 1>(s);
  } else {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  }
}

template <int RT, int EXP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void router_fused_kernel(RouterArgs a) {
  constexpr int TB = RT / 16;                 // token blocks of 16
  constexpr int KQ = 4 / TB;                  // waves per token block
  constexpr int NB = EXP / 16;                // expert blocks of 16
  constexpr int kRows = RT + EXP;             // stage rows: tokens, then router-weight rows
  constexpr int kStage = kRows * kLgCh;       // u32x4 per stage
  constexpr int kLoads = kRows / 16;          // 1 KB direct loads per wave per stage
  constexpr int NS = fused_slots<RT, EXP>();
  static_assert(NS >= 3 && NS * (kLoads) < 64, "ring");
  __shared__ u32x4 lds[NS * kStage];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tb = wave % TB, kq = wave / TB;
  const int tile0 = blockIdx.x * RT;
  const uint32_t rb = static_cast<uint32_t>(a.d) * 2u;   // bytes per row
  const int nrows = min(RT, a.T - tile0);
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  // out-of-range token and expert rows read as zero (buffer range check)
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(X + static_cast<size_t>(tile0) * a.d, static_cast<uint32_t>(nrows) * rb);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.W_g, static_cast<uint32_t>(a.E) * rb);
  const int nst = a.d / kLgK;                 // stages (even: d % 256 == 0)

  // direct loads: load i of wave w fills stage rows 16 i + 4 w + lane / 16 at
  // physical chunk lane % 16 (rows 0..RT-1: x, then the router weight)
  const int dr = 4 * wave + (lane >> 4);
  const uint32_t vo = static_cast<uint32_t>(dr) * rb + lgswz(dr, lane & 15) * 16;
  // Workgroups start at different even stages of d and wrap around, so the
  // launch's concurrent row segments spread over d (and the memory channels)
  // instead of all reading the same columns; each 256-element chunk stays
  // whole, and a token's chunk order is fixed by its tile.
  const int s0 = (2 * static_cast<int>(blockIdx.x)) % nst;
  auto issue = [&](int st) {
    u32x4* base = lds + (st % NS) * kStage + (4 * wave) * kLgCh;
    const int sc = st + s0 < nst ? st + s0 : st + s0 - nst;
    const uint32_t kb = static_cast<uint32_t>(sc) * (kLgK * 2);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      if (i < RT / 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (__attribute__((address_space(3))) void*)(base + 16 * i * kLgCh),
                                                 16, vo, static_cast<uint32_t>(16 * i) * rb + kb, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (__attribute__((address_space(3))) void*)(base + 16 * i * kLgCh),
                                                 16, vo, static_cast<uint32_t>(16 * (i - RT / 16)) * rb + kb, 0, 0);
    }
  };

  const int rr = lane & 15, cg = lane >> 4;
  double acc[NB][4];
  floatx4 part[NB];
#pragma unroll
  for (int eb = 0; eb < NB; ++eb) {
    part[eb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[eb][v] = 0.0;
  }

#pragma unroll
  for (int sp = 0; sp < NS - 1; ++sp)
    if (sp < nst) issue(sp);
  for (int st = 0; st < nst; ++st) {
    // stage st landed (up to NS - 2 later stages may be in flight); every
    // wave is past stage st-1, whose slot then takes stage st + NS - 1
    wait_stages<kLoads, NS - 2>(min(NS - 2, nst - 1 - st));
    lg_barrier();
    if (st + NS - 1 < nst) issue(st + NS - 1);
    const u32x4* sa = lds + (st % NS) * kStage;
#pragma unroll
    for (int q = 0; q < kLgK / 32 / KQ; ++q) {
      const int s = q * KQ + kq;   // this wave's k-steps of the stage
      const int ch = lgswz(rr, 4 * s + cg);
      const bf16x8 xf = __builtin_bit_cast(bf16x8, sa[(16 * tb + rr) * kLgCh + ch]);
#pragma unroll
      for (int eb = 0; eb < NB; ++eb) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, sa[(RT + 16 * eb + rr) * kLgCh + ch]);
        part[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wf, part[eb], 0, 0, 0);
      }
    }
    if (st & 1) {   // a 256-element chunk is complete: add it in float64
#pragma unroll
      for (int eb = 0; eb < NB; ++eb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[eb][v] += static_cast<double>(part[eb][v]);
        part[eb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  if constexpr (KQ > 1) {
    // add the second half's sums into the first (the ring is free: every wave
    // is past its last stage once all have passed this barrier)
    lg_barrier();
    double* red = reinterpret_cast<double*>(lds);
    if (kq == 1) {
#pragma unroll
      for (int eb = 0; eb < NB; ++eb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((tb * NB + eb) * 4 + v) * 64 + lane] = acc[eb][v];
    }
    lg_barrier();
    if (kq == 0) {
#pragma unroll
      for (int eb = 0; eb < NB; ++eb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[eb][v] += red[((tb * NB + eb) * 4 + v) * 64 + lane];
    }
    __syncthreads();
  }
  // lane (rr, cg) holds tokens 16 tb + 4 cg + v of the tile, experts 16 eb + rr:
  // the layout of route_tile (waves TB .. 3 hold no tokens there); its tables
  // go to the start of the ring, free once every wave is past the barrier above
  // (RT = 64) or the reduction's __syncthreads (RT = 32)
  if constexpr (KQ == 1) lg_barrier();
  static_assert(route_tile_smem<RT, NB>() <= NS * kStage * 16, "route_tile tables fit in the ring");
  route_tile<RT, NB>(a, acc, tile0, reinterpret_cast<unsigned char*>(lds));
}

// ---- bf16 inputs, d % 256 == 0, E <= 16, T <= 16384: 16-token tiles ----
//
// One workgroup per 16 tokens (Mixtral shape: 512 workgroups, two per CU),
// the four waves splitting d into interleaved 256-element chunks.  Each lane
// loads its MFMA fragments straight into registers: 16 bytes of its token row
// (the A operand) and of its expert's router row (the B operand; rows past E
// read zero through the buffer range check, with no memory traffic), a whole
// chunk (8 k-steps) ahead of the MFMAs, so ~8 KB per wave and ~128 KB per CU
// are in flight with no barrier in the loop.  float32 sums per chunk, added in
// float64; the four waves' sums are added in LDS in wave order, each wave
// taking a quarter of the tokens, whose selection it then runs (route_tile's
// spread layout: the per-token chain of softmax, top-k and log-sum-exp is a
// quarter as long as on one wave).
__global__ __launch_bounds__(256) void router_t16_kernel(RouterArgs a) {
  constexpr int RT = 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rr = lane & 15, cg = lane >> 4;
  const int tile0 = blockIdx.x * RT;
  const uint32_t rb = static_cast<uint32_t>(a.d) * 2u;
  const int nrows = min(RT, a.T - tile0);
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(X + static_cast<size_t>(tile0) * a.d, static_cast<uint32_t>(nrows) * rb);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.W_g, static_cast<uint32_t>(a.E) * rb);
  const uint32_t vo = static_cast<uint32_t>(rr) * rb + static_cast<uint32_t>(cg) * 16u;
  const int nch = a.d / 256;

  u32x4 xa0[8], wb0[8], xa1[8], wb1[8];
  auto load = [&](u32x4 (&xa)[8], u32x4 (&wb)[8], int c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t so = static_cast<uint32_t>(c) * 512u + static_cast<uint32_t>(s) * 64u;
      xa[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xs, vo, so, 0));
      wb[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, vo, so, 0));
    }
  };
  double acc[1][4] = {{0.0, 0.0, 0.0, 0.0}};
  auto chunk = [&](const u32x4 (&xa)[8], const u32x4 (&wb)[8]) {
    floatx4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[s]), __builtin_bit_cast(bf16x8, wb[s]),
                                                     part, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[0][v] += static_cast<double>(part[v]);
  };
  // wave w takes chunks w, w + 4, ...: two at a time, the next pair's loads
  // issued before the current pair's MFMAs
  int c = wave;
  if (c < nch) load(xa0, wb0, c);
  if (c + 4 < nch) load(xa1, wb1, c + 4);
  for (; c < nch; c += 8) {
    chunk(xa0, wb0);
    if (c + 8 < nch) load(xa0, wb0, c + 8);
    if (c + 4 < nch) {
      chunk(xa1, wb1);
      if (c + 12 < nch) load(xa1, wb1, c + 12);
    }
  }
  // wave w adds the four waves' sums of tokens 4 g + w in wave order and
  // selects those four tokens (route_tile's spread layout)
  __shared__ double red[4][4][64];
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[0][v];
  __syncthreads();
  double sel[1][4];
  sel[0][0] = ((red[0][wave][lane] + red[1][wave][lane]) + red[2][wave][lane]) + red[3][wave][lane];
  __shared__ __align__(8) unsigned char smem[route_tile_smem<RT, 1>()];
  route_tile<RT, 1, 1>(a, sel, tile0, smem);
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

  double bg[NB], bs[NB];
  lane_biases<NB>(a, c, bg, bs);
  double val[NB];
  double m = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    double l = -INFINITY;
    if (e < E && tok_ok) l = lg[nb] + bg[nb];
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
  if (!ec) select_k<NB>(a, val, bs, m, c, my_idx, my_e, esum);
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
  // probability sums over the tile's tokens: thread (q, e), q < G = 1024 / E,
  // adds tokens q, q + G, ... in order; then the G partials in order
  __shared__ float s_ps[kSelectThreads];
  {
    const int G = kSelectThreads / E, e = threadIdx.x % E, q = threadIdx.x / E;
    float ps = 0.f;
    if (q < G)
      for (int rr = q; rr < ntok; rr += G) ps += s_p[rr][e];
    s_ps[threadIdx.x] = ps;
    __syncthreads();
    if (threadIdx.x < E) {
      float tot = 0.f;
      for (int qq = 0; qq < G; ++qq) tot += s_ps[qq * E + threadIdx.x];
      a.p_part[static_cast<size_t>(tile) * E + threadIdx.x] = tot;
      if (!ec) a.tile_hist[static_cast<size_t>(tile) * E + threadIdx.x] = __popcll(s_mask[threadIdx.x]);
    }
  }
  if (threadIdx.x < kWave) {
    // z-loss partial of the tile: a fixed butterfly over the tile's tokens
    const double zs = wave_sum64(threadIdx.x < ntok ? s_z[threadIdx.x] : 0.0);
    if (threadIdx.x == 0) a.z_part[tile] = zs;
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
  // the split-K partials, added in split order; every expert's load of a
  // split is issued before any is added (a load-and-add loop per expert waited
  // for each load in turn: NB memory round trips per split instead of one)
  const bool tok_ok = t < a.T;
  double lg[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + c;
    lg[nb] = e < a.E && tok_ok ? logits[static_cast<size_t>(t) * Epad + e] : 0.0;
  }
  for (int q = 1; q < KS; ++q) {
    const double* lq = logits + static_cast<size_t>(q) * a.T * Epad;
    double v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int e = nb * 16 + c;
      v[nb] = e < a.E && tok_ok ? lq[static_cast<size_t>(t) * Epad + e] : 0.0;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) lg[nb] += v[nb];
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
  if (p.dtype == MOE_BF16) {
    hipLaunchKernelGGL(router_bf16_kernel<NB>, grid, block, 0, st, a);
  } else {
    if constexpr (NB <= 4) {
      if (p.rtile == 16) {
        hipLaunchKernelGGL((router_f32_kernel<16, NB>), grid, block, 0, st, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((router_f32_kernel<64, NB>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

// The one-launch router serves bf16 layers with d a multiple of 256 and at
// most 64 experts (each workgroup holds every expert's logits); more experts
// take the split logits kernel and the selection kernel.
bool router_fused(const Problem& p) { return p.dtype == MOE_BF16 && p.d % 256 == 0 && p.E <= kLgExp; }

// Tokens per router tile (and per-tile permute table row): 16 on the bf16
// path with at most 16 experts (T <= 16384); else, when 64-token tiles would
// give the launch fewer than 256 workgroups, 32 on the other one-launch bf16
// path and 16 on the float32 path (at most 64 experts); else 64.  (16-token
// selection tiles for more than 64 experts were measured at the DeepSeek
// shape: selection 28 -> 21 us, but the permute, whose workgroups each read
// the whole [tiles, E] count table, 13 -> 27 us.)
// The 16-token bf16 kernel (at most 16 experts): its workgroups each read
// every tile's expert counts in the permute, so it is kept to T <= 16384.
bool router_t16(const Problem& p) { return router_fused(p) && p.E <= 16 && p.T <= 16384; }

int router_tile(const Problem& p) {
  const bool few = (p.T + 63) / 64 < 256;
  if (router_t16(p)) return 16;
  if (router_fused(p) && few) return 32;
  // float32 with at most 64 experts: 16-token tiles, the four waves splitting d
  if (p.dtype == MOE_F32 && p.E <= 64 && few) return 16;
  return kRouterTile;
}

// expert padding of the logits: one 16-expert tile when E <= 16 (a quarter of
// the MFMA work and partial-logit traffic of a 64-expert tile), else 64s
int logit_pad(int E) { return E <= 16 ? 16 : (E + kLgExp - 1) / kLgExp * kLgExp; }

// d is split into KS ranges of whole 256-element chunks so the logits launch
// has ~256 workgroups (at most 8 splits, at least one chunk each)
int logit_splits(const Problem& p) {
  if (router_fused(p)) return 0;   // no partial logits
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
  if (router_fused(p)) {
    const dim3 grid(p.ntile), block(256);
    if (p.rtile == 16) {
      hipLaunchKernelGGL(router_t16_kernel, grid, block, 0, st, a);
    } else if (p.rtile == 32) {
      if (p.E <= 16) hipLaunchKernelGGL((router_fused_kernel<32, 16>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((router_fused_kernel<32, 64>), grid, block, 0, st, a);
    } else {
      if (p.E <= 16) hipLaunchKernelGGL((router_fused_kernel<64, 16>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((router_fused_kernel<64, 64>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  }
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
