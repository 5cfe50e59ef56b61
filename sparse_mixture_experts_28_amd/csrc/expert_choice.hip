// moe_expert_choice: expert-choice routing.  Every expert takes the C tokens
// with the largest router logits (ties to the lower token index) and weights
// each by the token's softmax probability of that expert.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §4.2 (the router scores are
// transposed to experts x tokens and each expert takes a top-k over tokens,
// k = its capacity; perfect balance, no token dropped for capacity) and
// "第7章 Mixture of Experts" §7.2 (each expert picks its top-C tokens; a token
// may be picked by several experts or by none) and §7.1 (the gate G(x) that
// weights an expert's output is the router's softmax).
//
// One workgroup per expert; the column of T float64 logits is staged in LDS
// when T <= 16384 (128 KB), else re-read from L2.
//  1. min and max of the column; 1024 buckets of equal width over [min, max]
//     (bucket index = floor((l - min) * 1024 / (max - min)), clamped: a
//     monotone function of l, so every token of a higher bucket has a larger
//     logit); one LDS histogram pass.  Router logits are spread in value, so
//     the histogram's atomics rarely collide.
//  2. The bucket b* holding the C-th largest logit and `need`, how many of its
//     tokens are taken, follow from a scan of the bins from the top.
//  3. The tokens of b* (usually a few dozen) are ranked exactly, by logit and
//     then token index, and marked taken or not in the rank table.  If b*
//     holds more than 1024 tokens (many equal logits), a most-significant-
//     digit radix select over order-preserving 64-bit keys restricted to b*
//     finds the exact threshold key instead, ties again to the lower index.
//  4. The taken tokens (bucket > b*, or marked in b*) are listed in token
//     order by rounds of 1024 consecutive tokens (one per thread, coalesced),
//     ballots and per-wave counts giving each its rank within the round.
// Integer histograms and counts only: the result does not depend on timing.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEcThreads = 1024;
constexpr int kEcWaves = kEcThreads / kWave;

// Order-preserving key of a float64: larger value -> larger unsigned key.
// -0.0 is folded onto +0.0 first so equal values have equal keys.
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v + 0.0));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive count of `flag` over the block's threads in thread order, and the
// block's total.  s_wave[kEcWaves] must not be in use by another count: the
// caller alternates two buffers between consecutive calls (one barrier each).
__device__ __forceinline__ int block_excl_count(bool flag, int* s_wave, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t b = __ballot(flag);
  if (lane == 0) s_wave[wave] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kEcWaves; ++w) {
    const int c = s_wave[w];
    before += w < wave ? c : 0;
    all += c;
  }
  total = all;
  return before + __popcll(b & ((1ull << lane) - 1ull));
}

struct EcArgs {
  const double* logits;   // [E][T]
  const double* m;        // [T]
  const float* z;         // [T]
  int T, C;
  int32_t* ec_token;      // [E][C]
  float* ec_w;            // [E][C]
  int32_t* pos;           // [E][T]; also marks the boundary bucket's tokens during the selection
  int32_t* row_token;     // [E * C]: the GEMM's row -> token index
};

constexpr int kEcLdsTokens = 16384;
constexpr int kBins = 1024;
constexpr int kList = 1024;                       // boundary tokens ranked directly
constexpr int32_t kMarkTaken = -2, kMarkLeft = -3;

__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmin(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmax(v, __shfl_xor(v, m, kWave));
  return v;
}

// Wave 0 scans n bins from the top (lane l: bins n-1-(n/64)l .. descending) and
// returns, in s_sel, the bin holding the need-th largest counted item, how many
// items of that bin are still needed, and the bin's count.
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int need, int* s_sel) {
  if (threadIdx.x >= kWave) return;
  constexpr int per = NB / kWave;
  const int l = threadIdx.x;
  int own = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) own += static_cast<int>(hist[NB - 1 - per * l - i]);
  int incl = own;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (l >= off) incl += o;
  }
  int above = incl - own;
  if (above < need && need <= incl) {
    for (int i = 0; i < per; ++i) {
      const int hi = static_cast<int>(hist[NB - 1 - per * l - i]);
      if (above < need && need <= above + hi) {
        s_sel[0] = NB - 1 - per * l - i;
        s_sel[1] = need - above;
        s_sel[2] = hi;
      }
      above += hi;
    }
  }
}

template <bool kStaged>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(EcArgs a) {
  __shared__ double s_val[kStaged ? kEcLdsTokens : 1];
  __shared__ uint32_t s_hist[kBins];
  __shared__ int32_t s_list_t[kList];
  __shared__ double s_list_v[kList];
  __shared__ double s_red[2][kEcWaves];
  __shared__ int s_cnt[2][kEcWaves];
  __shared__ int s_sel[3];
  __shared__ int s_nlist;
  const int e = blockIdx.x;
  const int T = a.T, C = a.C;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const double* col = a.logits + static_cast<size_t>(e) * T;
  int32_t* pos = a.pos + static_cast<size_t>(e) * T;
  // -0.0 is folded onto +0.0 so that equal logits compare and bucket alike
  auto val = [&](int t) -> double {
    if constexpr (kStaged) return s_val[t];
    else return col[t] + 0.0;
  };

  // 1. stage, min and max: eight tokens a thread per round, their loads
  // issued together (at a clamped index: a load under the t < T condition
  // would be waited for at once)
  double lo = INFINITY, hi = -INFINITY;
  constexpr int kStageU = 8;
  for (int t0 = threadIdx.x; t0 < T; t0 += kStageU * kEcThreads) {
    double v[kStageU];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) v[u] = col[min(t0 + u * kEcThreads, T - 1)];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int t = t0 + u * kEcThreads;
      if (t < T) {
        const double x = v[u] + 0.0;
        if constexpr (kStaged) s_val[t] = x;
        lo = fmin(lo, x);
        hi = fmax(hi, x);
      }
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_red[0][wave] = lo;
    s_red[1][wave] = hi;
  }
  for (int i = threadIdx.x; i < kBins; i += kEcThreads) s_hist[i] = 0u;
  if (threadIdx.x == 0) s_nlist = 0;
  __syncthreads();
  double vmin = s_red[0][0], vmax = s_red[1][0];
#pragma unroll
  for (int w = 1; w < kEcWaves; ++w) {
    vmin = fmin(vmin, s_red[0][w]);
    vmax = fmax(vmax, s_red[1][w]);
  }
  const double range = vmax - vmin;
  const double scale = static_cast<double>(kBins) / range;
  // equal logits everywhere, or a range that does not scale: one bucket
  const bool bucketed = range > 0.0 && isfinite(range) && isfinite(scale);
  auto bucket = [&](double v) -> int {
    if (!bucketed || !(v >= vmin)) return 0;   // a NaN logit goes to the lowest bucket
    const int b = static_cast<int>((v - vmin) * scale);
    return b < kBins - 1 ? b : kBins - 1;
  };

  // 2. histogram and the boundary bucket
  for (int t = threadIdx.x; t < T; t += kEcThreads) atomicAdd(&s_hist[bucket(val(t))], 1u);
  __syncthreads();
  find_bin<kBins>(s_hist, C, s_sel);
  __syncthreads();
  const int bstar = s_sel[0];
  int need = s_sel[1];
  const int nb = s_sel[2];

  // 3. the boundary bucket's tokens
  const bool listed = nb <= kList;
  uint64_t kstar = 0;
  bool all_ties = true;
  if (listed) {
    for (int t = threadIdx.x; t < T; t += kEcThreads) {
      const double v = val(t);
      if (bucket(v) == bstar) {
        const int i = atomicAdd(&s_nlist, 1);   // list order is irrelevant: ranks below are exact
        s_list_t[i] = t;
        s_list_v[i] = v;
      }
    }
    __syncthreads();
    if (threadIdx.x < nb) {
      const int ti = s_list_t[threadIdx.x];
      const double vi = s_list_v[threadIdx.x];
      int rank = 0;
      for (int j = 0; j < nb; ++j) {
        const double vj = s_list_v[j];
        rank += vj > vi || (vj == vi && s_list_t[j] < ti);
      }
      pos[ti] = rank < need ? kMarkTaken : kMarkLeft;
    }
    __syncthreads();   // the marks are read back by other threads below
  } else {
    // exact radix select among the boundary bucket's tokens
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += kEcThreads) s_hist[i] = 0u;
      __syncthreads();
      for (int t = threadIdx.x; t < T; t += kEcThreads) {
        const double v = val(t);
        const uint64_t k = order_key(v);
        if (bucket(v) == bstar && (k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      find_bin<256>(s_hist, need, s_sel);
      __syncthreads();
      prefix |= static_cast<uint64_t>(s_sel[0]) << shift;
      mask |= 0xFFull << shift;
      need = s_sel[1];
      all_ties = s_sel[1] == s_sel[2];   // after the last pass: every key equal to K* is taken
      __syncthreads();
    }
    kstar = prefix;
  }

  // 4. taken tokens in token order, 1024 consecutive tokens per round
  int taken_before = 0, eq_before = 0, buf = 0;
  for (int t0 = 0; t0 < T; t0 += kEcThreads) {
    const int t = t0 + threadIdx.x;
    const bool valid = t < T;
    const double v = valid ? val(t) : 0.0;
    const int b = valid ? bucket(v) : -1;
    bool take = valid && b > bstar;
    if (listed) {
      if (valid && b == bstar) take = pos[t] == kMarkTaken;
    } else {
      const uint64_t k = order_key(v);
      const bool in = valid && b == bstar;
      if (all_ties) {
        take = take || (in && k >= kstar);
      } else {
        const bool eq = in && k == kstar;
        int eq_round;
        const int eq_rank = eq_before + block_excl_count(eq, s_cnt[buf], eq_round);
        buf ^= 1;
        eq_before += eq_round;
        take = take || (in && (k > kstar || (eq && eq_rank < need)));
      }
    }
    int taken_round;
    const int slot = taken_before + block_excl_count(take, s_cnt[buf], taken_round);
    buf ^= 1;
    taken_before += taken_round;
    if (valid) {
      int32_t p = -1;
      // exactly C tokens are taken; the bound keeps every write inside the
      // [E, C] outputs regardless
      if (take && slot < C) {
        p = slot;
        const size_t row = static_cast<size_t>(e) * C + slot;
        a.ec_token[row] = t;
        a.row_token[row] = t;
        // the softmax probability, formed as the router forms it
        a.ec_w[row] = __expf(static_cast<float>(v - a.m[t])) * (1.f / a.z[t]);
      }
      pos[t] = p;
    }
  }
}

}  // namespace

hipError_t launch_ec_select(const Problem& p, int32_t* ec_token, float* ec_w, const Workspace& ws,
                            hipStream_t st) {
  EcArgs a;
  a.logits = ws.ec_logits;
  a.m = ws.ec_m;
  a.z = ws.ec_z;
  a.T = p.T;
  a.C = p.ec_C;
  a.ec_token = ec_token;
  a.ec_w = ec_w;
  a.pos = ws.ec_pos;
  a.row_token = ws.row_token;
  if (p.T <= kEcLdsTokens)
    hipLaunchKernelGGL(ec_select_kernel<true>, dim3(p.E), dim3(kEcThreads), 0, st, a);
  else
    hipLaunchKernelGGL(ec_select_kernel<false>, dim3(p.E), dim3(kEcThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
