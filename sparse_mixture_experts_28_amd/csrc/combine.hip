// moe_combine: out[t] = sum over kept slots j of w[t,j] * Y[slot_pos[t,j]]
//                     + sum over shared experts s of Y_shared[s][t].
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (the k expert outputs are
// weighted by the renormalised router scores and summed) and §7.1 (shared
// experts are added to the routed output with weight 1); "第7章 Mixture of
// Experts" §7.1 (MoE(x) = sum_i G(x)_i E_i(x)) and §7.4 (an overflowed token's
// slot contributes nothing; the residual outside the layer carries it).
//
// A gather, not a scatter: one wave per token reads its k expert rows and its
// shared rows, accumulates in float32 in slot order then shared order, and
// rounds once.  No atomics, so the result is bitwise reproducible.
//
// Expert choice ("第7章 Mixture of Experts" §7.2; the guide's §4.2): a token's
// routed rows are those of the experts that took it, 0 to E of them, added in
// ascending expert order with the weights the selection recorded.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void acc_bf16x8(float (&a)[8], u32x4 v, float w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] = fmaf(w, __uint_as_float(v[i] << 16), a[2 * i]);
    a[2 * i + 1] = fmaf(w, __uint_as_float(v[i] & 0xffff0000u), a[2 * i + 1]);
  }
}

__device__ __forceinline__ void acc_f32x4(float4& a, float4 v, float w) {
  a.x = fmaf(w, v.x, a.x);
  a.y = fmaf(w, v.y, a.y);
  a.z = fmaf(w, v.z, a.z);
  a.w = fmaf(w, v.w, a.w);
}

// Accumulates 16-byte column c of rows[0 .. B) times w[0 .. B), in that order:
// all B loads are issued before the first is used, so a token's rows arrive
// together rather than one memory latency each.
template <int B, typename V, typename A>
__device__ __forceinline__ void gather_batch(A& a, const V* __restrict__ y, const int32_t* rows, const float* w, int c,
                                             int vec_per_row) {
  V v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) v[j] = y[static_cast<size_t>(rows[j]) * vec_per_row + c];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    if constexpr (sizeof(V) == 16 && sizeof(A) == 32) acc_bf16x8(a, v[j], w[j]);
    else acc_f32x4(a, v[j], w[j]);
  }
}

// rows[0 .. n) in order, in batches of 8 and one last batch of n mod 8
template <typename V, typename A>
__device__ __forceinline__ void gather_rows(A& a, const V* __restrict__ y, const int32_t* rows, const float* w, int n,
                                            int c, int vec_per_row) {
  int j = 0;
  for (; j + 8 <= n; j += 8) gather_batch<8>(a, y, rows + j, w + j, c, vec_per_row);
  switch (n - j) {
    case 1: gather_batch<1>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 2: gather_batch<2>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 3: gather_batch<3>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 4: gather_batch<4>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 5: gather_batch<5>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 6: gather_batch<6>(a, y, rows + j, w + j, c, vec_per_row); break;
    case 7: gather_batch<7>(a, y, rows + j, w + j, c, vec_per_row); break;
    default: break;
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float (&a)[8]) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(a[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(a[2 * i + 1])) << 16);
  return o;
}

// Top-k, one wave per token (grid-stride over tokens).  Lane j < k reads
// slot j's row and weight, and the wave broadcasts them (uniform values);
// the shared-expert rows follow with weight 1.  Each lane then takes CU
// 16-byte column chunks at a time and issues the loads of all the token's
// rows for them before adding any (ROWS x CU loads in flight per lane), in
// slot order then shared order, a dropped slot (row -1) skipped.  No
// workgroup barrier and no serial list building: a wave moves on to its next
// token as soon as its stores are issued.
template <int ROWS, typename V, typename A>
__device__ __forceinline__ void combine_token_wave(const Problem& p, const V* __restrict__ y,
                                                   const int32_t* __restrict__ slot_pos,
                                                   const float* __restrict__ topk_w, V* __restrict__ out,
                                                   int vec_per_row, int t, int lane) {
  constexpr int CU = ROWS >= 8 ? 1 : 8 / ROWS;
  int my_pos = -1;
  float my_w = 0.f;
  if (lane < p.k) {
    my_pos = slot_pos[static_cast<size_t>(t) * p.k + lane];
    my_w = topk_w[static_cast<size_t>(t) * p.k + lane];
  } else if (lane < p.k + p.S) {
    my_pos = p.A + (lane - p.k) * p.T + t;   // shared expert lane - k, weight 1
    my_w = 1.0f;
  }
  int row[ROWS];
  float wt[ROWS];
#pragma unroll
  for (int j = 0; j < ROWS; ++j) {
    row[j] = __builtin_amdgcn_readfirstlane(__shfl(my_pos, j, kWave));
    wt[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __shfl(my_w, j, kWave))));
  }
  for (int c0 = lane; c0 < vec_per_row; c0 += kWave * CU) {
    V v[ROWS][CU];
#pragma unroll
    for (int j = 0; j < ROWS; ++j)
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int c = c0 + kWave * u;
        if (row[j] >= 0 && c < vec_per_row) v[j][u] = y[static_cast<size_t>(row[j]) * vec_per_row + c];
      }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int c = c0 + kWave * u;
      if (c >= vec_per_row) break;
      A a{};
#pragma unroll
      for (int j = 0; j < ROWS; ++j) {
        if (row[j] < 0) continue;
        if constexpr (sizeof(V) == 16 && sizeof(A) == 32) acc_bf16x8(a, v[j][u], wt[j]);
        else acc_f32x4(a, v[j][u], wt[j]);
      }
      if constexpr (sizeof(A) == 32) out[static_cast<size_t>(t) * vec_per_row + c] = pack_bf16x8(a);
      else out[static_cast<size_t>(t) * vec_per_row + c] = a;
    }
  }
}

template <int ROWS, typename V, typename A>
__global__ __launch_bounds__(256) void combine_wave_kernel(Problem p, const V* __restrict__ y,
                                                           const int32_t* __restrict__ slot_pos,
                                                           const float* __restrict__ topk_w, V* __restrict__ out,
                                                           int vec_per_row) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nw = gridDim.x * (blockDim.x / kWave);
  for (int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave); t < p.T; t += nw)
    combine_token_wave<ROWS, V, A>(p, y, slot_pos, topk_w, out, vec_per_row, t, lane);
}

// Expert choice: the rows of token t, in ascending expert order.  Wave 0 reads
// pos[e][t] for every expert (lane l: experts 4l .. 4l+3, E <= 256) and packs
// the takers with a lane prefix count; the shared-expert rows follow with
// weight 1.  Returns the number of rows.
__device__ int ec_token_rows(const Problem& p, const int32_t* __restrict__ pos, const float* __restrict__ ec_w,
                             int t, int32_t* s_row, float* s_w, int* s_n) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    int32_t c4[4];
    int own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * l + i;
      c4[i] = e < p.E ? pos[static_cast<size_t>(e) * p.T + t] : -1;
      own += c4[i] >= 0;
    }
    int incl = own;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (l >= off) incl += o;
    }
    int at = incl - own;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c4[i] >= 0) {
        const int row = (4 * l + i) * p.ec_C + c4[i];
        s_row[at] = row;
        s_w[at] = ec_w[row];
        ++at;
      }
    }
    // the last lane's count is the number of takers; the shared rows follow
    const int taken = __shfl(incl, kWave - 1, kWave);
    if (l < p.S) {
      s_row[taken + l] = p.A + l * p.T + t;
      s_w[taken + l] = 1.0f;
    }
    if (l == kWave - 1) *s_n = taken + p.S;
  }
  __syncthreads();
  return *s_n;
}

__global__ __launch_bounds__(256) void combine_ec_bf16_kernel(Problem p, const u32x4* __restrict__ y,
                                                              const int32_t* __restrict__ pos,
                                                              const float* __restrict__ ec_w,
                                                              u32x4* __restrict__ out, int vec_per_row) {
  __shared__ int32_t s_row[MOE_MAX_EXPERTS + MOE_MAX_SHARED];
  __shared__ float s_w[MOE_MAX_EXPERTS + MOE_MAX_SHARED];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int n = ec_token_rows(p, pos, ec_w, t, s_row, s_w, &s_n);
  for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    gather_rows(a, y, s_row, s_w, n, c, vec_per_row);
    out[static_cast<size_t>(t) * vec_per_row + c] = pack_bf16x8(a);
  }
}

__global__ __launch_bounds__(256) void combine_ec_f32_kernel(Problem p, const float4* __restrict__ y,
                                                             const int32_t* __restrict__ pos,
                                                             const float* __restrict__ ec_w,
                                                             float4* __restrict__ out, int vec_per_row) {
  __shared__ int32_t s_row[MOE_MAX_EXPERTS + MOE_MAX_SHARED];
  __shared__ float s_w[MOE_MAX_EXPERTS + MOE_MAX_SHARED];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int n = ec_token_rows(p, pos, ec_w, t, s_row, s_w, &s_n);
  for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    gather_rows(a, y, s_row, s_w, n, c, vec_per_row);
    out[static_cast<size_t>(t) * vec_per_row + c] = a;
  }
}

}  // namespace

hipError_t launch_combine_ec(const Problem& p, const float* ec_w, const Workspace& ws, void* out,
                             hipStream_t st) {
  const int elem = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = p.d * elem / 16;
  // at least one wave: wave 0 gathers the token's expert list
  const int threads = vec_per_row >= 256 ? 256 : (vec_per_row >= 128 ? 128 : 64);
  if (p.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_ec_bf16_kernel, dim3(p.T), dim3(threads), 0, st, p,
                       static_cast<const u32x4*>(ws.ybuf), ws.ec_pos, ec_w, static_cast<u32x4*>(out),
                       vec_per_row);
  else
    hipLaunchKernelGGL(combine_ec_f32_kernel, dim3(p.T), dim3(threads), 0, st, p,
                       static_cast<const float4*>(ws.ybuf), ws.ec_pos, ec_w, static_cast<float4*>(out),
                       vec_per_row);
  return hipGetLastError();
}

hipError_t launch_combine(const Problem& p, const float* topk_w, const Workspace& ws, void* out,
                          hipStream_t st) {
  const int elem = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = p.d * elem / 16;
  // grid-stride waves: about eight per SIMD of a 256-CU part
  const int waves = p.T < 8192 ? p.T : 8192;
  const dim3 grid((waves + 3) / 4), block(256);
  const int rows = p.k + p.S;
#define MOE_COMBINE(ROWS_)                                                                                      \
  do {                                                                                                          \
    if (p.dtype == MOE_BF16)                                                                                    \
      hipLaunchKernelGGL((combine_wave_kernel<ROWS_, u32x4, float[8]>), grid, block, 0, st, p,                  \
                         static_cast<const u32x4*>(ws.ybuf), ws.slot_pos, topk_w, static_cast<u32x4*>(out),      \
                         vec_per_row);                                                                          \
    else                                                                                                        \
      hipLaunchKernelGGL((combine_wave_kernel<ROWS_, float4, float4>), grid, block, 0, st, p,                   \
                         static_cast<const float4*>(ws.ybuf), ws.slot_pos, topk_w, static_cast<float4*>(out),    \
                         vec_per_row);                                                                          \
  } while (0)
  if (rows <= 2) MOE_COMBINE(2);
  else if (rows <= 4) MOE_COMBINE(4);
  else if (rows <= 8) MOE_COMBINE(8);
  else MOE_COMBINE(16);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
