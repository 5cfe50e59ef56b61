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
// One workgroup per expert.  The C-th largest logit of the expert's column is
// found exactly by a most-significant-digit radix select over order-preserving
// 64-bit keys of the float64 logits (8 passes of 8 bits; each pass counts the
// keys that still match the prefix found so far in a 256-bin LDS histogram).
// With K* that key and `need` the number of tokens equal to K* still to take,
// a token is taken iff its key > K*, or its key == K* and fewer than `need`
// equal keys precede it in token order.  A block-wide scan over contiguous
// token chunks lists the taken tokens in ascending token order.  Integer
// histograms and scans only: the result does not depend on timing.
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

// Exclusive prefix sum of one int per thread over the 1024-thread block, in
// thread order; also returns the block total.  Uses s_tmp[kEcWaves + 1].
__device__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) s_tmp[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kEcWaves; ++w) {
      const int x = s_tmp[w];
      s_tmp[w] = run;
      run += x;
    }
    s_tmp[kEcWaves] = run;
  }
  __syncthreads();
  const int excl = s_tmp[wave] + incl - v;
  total = s_tmp[kEcWaves];
  __syncthreads();   // s_tmp may be reused by the caller's next scan
  return excl;
}

struct EcArgs {
  const double* logits;   // [E][T]
  const double* m;        // [T]
  const float* z;         // [T]
  int T, C;
  int32_t* ec_token;      // [E][C]
  float* ec_w;            // [E][C]
  int32_t* pos;           // [E][T]
  int32_t* row_token;     // [E * C]: the GEMM's row -> token index
};

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(EcArgs a) {
  __shared__ uint32_t s_hist[256];
  __shared__ int s_scan[kEcWaves + 1];
  __shared__ int s_digit, s_need;
  const int e = blockIdx.x;
  const int T = a.T, C = a.C;
  const double* col = a.logits + static_cast<size_t>(e) * T;

  // 1. radix select of the C-th largest key
  uint64_t prefix = 0, mask = 0;
  int need = C;   // keys still to take among those matching the prefix
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kEcThreads) s_hist[i] = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += kEcThreads) {
      const uint64_t k = order_key(col[t]);
      if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane l owns bins 255 - 4l .. 252 - 4l (descending); find the bin in
      // which the need-th largest matching key falls
      const int l = threadIdx.x;
      uint32_t h[4];
      int own = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = s_hist[255 - 4 * l - i];
        own += static_cast<int>(h[i]);
      }
      int incl = own;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (l >= off) incl += o;
      }
      int above = incl - own;   // matching keys in higher bins
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hi = static_cast<int>(h[i]);
        if (above < need && need <= above + hi) {
          s_digit = 255 - 4 * l - i;
          s_need = need - above;
        }
        above += hi;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(s_digit) << shift;
    mask |= 0xFFull << shift;
    need = s_need;
    __syncthreads();   // s_digit / s_need / s_hist are rewritten next pass
  }
  const uint64_t kstar = prefix;

  // 2. taken tokens in token order: thread i owns tokens [i*chunk, (i+1)*chunk)
  const int chunk = (T + kEcThreads - 1) / kEcThreads;
  const int t0 = min(T, static_cast<int>(threadIdx.x) * chunk);
  const int t1 = min(T, t0 + chunk);
  int n_eq = 0;
  for (int t = t0; t < t1; ++t) n_eq += order_key(col[t]) == kstar;
  int total;
  const int eq_before = block_exclusive_scan(n_eq, s_scan, total);
  int n_take = 0;
  {
    int eq_seen = eq_before;
    for (int t = t0; t < t1; ++t) {
      const uint64_t k = order_key(col[t]);
      if (k > kstar) ++n_take;
      else if (k == kstar) n_take += (eq_seen++ < need);
    }
  }
  int c = block_exclusive_scan(n_take, s_scan, total);
  int eq_seen = eq_before;
  for (int t = t0; t < t1; ++t) {
    const double l = col[t];
    const uint64_t k = order_key(l);
    const bool take = k > kstar || (k == kstar && eq_seen++ < need);
    int32_t slot = -1;
    // exactly C tokens are taken (C - need keys above K*, need equal to it);
    // the bound keeps every write inside the [E, C] outputs regardless
    if (take && c < C) {
      slot = c++;
      const size_t row = static_cast<size_t>(e) * C + slot;
      a.ec_token[row] = t;
      a.row_token[row] = t;
      // the softmax probability, formed as the router forms it
      a.ec_w[row] = __expf(static_cast<float>(l - a.m[t])) * (1.f / a.z[t]);
    }
    a.pos[static_cast<size_t>(e) * T + t] = slot;
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
  hipLaunchKernelGGL(ec_select_kernel, dim3(p.E), dim3(kEcThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
