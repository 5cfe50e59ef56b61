// moe_permute: turn the router's per-tile histograms and in-tile ranks into a
// deterministic, capacity-limited, expert-sorted copy of the token rows.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (the mask of tokens routed
// to each expert, gathered per expert), §8.2 and "第7章 Mixture of Experts"
// §7.4 (capacity = factor x tokens / experts, overflow tokens dropped or passed
// by the residual outside the layer); §4.3 of the guide (balance loss
// E * sum f_i P_i); "第7章" tensor-shape trace (the token -> expert reordering
// is the real cost of the layer).
//
// scan    (1 workgroup): for every expert, an exclusive scan of its per-tile
//         counts over the tiles in token order gives each tile's base rank;
//         the total is c_e, kept_e = min(c_e, cap); an exclusive scan of kept
//         over experts gives the segment offsets; the balance loss is
//         finalised from c and the per-tile probability sums (float64, fixed
//         order); the grouped-GEMM segment table is written.
// scatter (1 workgroup per token): rank = tile base + in-tile rank; the
//         assignment is kept iff rank < cap; the token row is read once and
//         written to every kept slot (16-byte vectors).
//
// No atomics anywhere: every result is a fixed function of the inputs.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void scan_kernel(Problem p, int32_t* tile_hist, const float* p_part,
                                                   int32_t* counts, int32_t* kept, int32_t* seg_base,
                                                   float* aux_loss, int32_t* counts_out,
                                                   int32_t* kept_out) {
  __shared__ int32_t s_kept[MOE_MAX_EXPERTS];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ double s_P[MOE_MAX_EXPERTS];
  const int E = p.E;
  const int nseg = p.E + p.S;
  SegTable st = seg_table(seg_base, nseg, E);

  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    double psum = 0.0;
    for (int tile = 0; tile < p.ntile; ++tile) {
      const size_t i = static_cast<size_t>(tile) * E + e;
      const int h = tile_hist[i];
      tile_hist[i] = run;       // becomes the tile's base rank for expert e
      run += h;
      psum += static_cast<double>(p_part[i]);
    }
    const int kp = min(run, p.cap);
    counts[e] = run;
    kept[e] = kp;
    if (counts_out) counts_out[e] = run;
    if (kept_out) kept_out[e] = kp;
    s_kept[e] = kp;
    s_cnt[e] = run;
    s_P[e] = psum / static_cast<double>(p.T);
  }
  __syncthreads();

  if (threadIdx.x == 0) {
    // aux = E * sum_e f_e P_e, f_e = c_e / (T k)
    const double tk = static_cast<double>(p.T) * static_cast<double>(p.k);
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += (static_cast<double>(s_cnt[e]) / tk) * s_P[e];
    *aux_loss = static_cast<float>(static_cast<double>(E) * s);

    // segment table: routed experts then shared experts
    int off = 0;
    int tiles = 0;
    const int bm = p.gemm_bm;
    const int routed_rows = p.T * p.k;
    for (int e = 0; e < nseg; ++e) {
      int rows, a_off, o_off;
      if (e < E) {
        rows = s_kept[e];
        a_off = off;
        o_off = off;
        st.route_off[e] = off;
        off += rows;
      } else {
        rows = p.T;
        a_off = 0;
        o_off = routed_rows + (e - E) * p.T;
      }
      st.rows[e] = rows;
      st.a_off[e] = a_off;
      st.o_off[e] = o_off;
      st.tile_start[e] = tiles;
      tiles += (rows + bm - 1) / bm;
    }
    st.tile_start[nseg] = tiles;
  }
}

template <typename Vec>
__global__ __launch_bounds__(256) void scatter_kernel(Problem p, const Vec* __restrict__ x,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ local_rank,
                                                      const int32_t* __restrict__ tile_base,
                                                      const int32_t* __restrict__ seg_base,
                                                      int32_t* __restrict__ slot_pos,
                                                      Vec* __restrict__ xperm, int vec_per_row) {
  __shared__ int32_t s_pos[MOE_MAX_TOPK];
  const int t = blockIdx.x;
  const int k = p.k;
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    const int e = topk_idx[static_cast<size_t>(t) * k + j];
    const int tile = t / kRouterTile;
    const int rank = tile_base[static_cast<size_t>(tile) * p.E + e] + local_rank[static_cast<size_t>(t) * k + j];
    SegTable st = seg_table(const_cast<int32_t*>(seg_base), p.E + p.S, p.E);
    const int pos = rank < p.cap ? st.route_off[e] + rank : -1;
    slot_pos[static_cast<size_t>(t) * k + j] = pos;
    s_pos[j] = pos;
  }
  __syncthreads();
  const Vec* src = x + static_cast<size_t>(t) * vec_per_row;
  for (int c = threadIdx.x; c < vec_per_row; c += blockDim.x) {
    const Vec v = src[c];
    for (int j = 0; j < k; ++j) {
      const int pos = s_pos[j];
      if (pos >= 0) xperm[static_cast<size_t>(pos) * vec_per_row + c] = v;
    }
  }
}

}  // namespace

hipError_t launch_scan(const Problem& p, const Workspace& ws, float* aux_loss, int32_t* counts_out,
                       int32_t* kept_out, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, st, p, ws.tile_hist, ws.p_part, ws.counts,
                     ws.kept, ws.seg, aux_loss, counts_out, kept_out);
  return hipGetLastError();
}

hipError_t launch_scatter(const Problem& p, const void* x, const int32_t* topk_idx, const Workspace& ws,
                          hipStream_t st) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int elem = p.dtype == MOE_BF16 ? 2 : 4;
  const int vec_per_row = p.d * elem / 16;
  const int threads = vec_per_row >= 256 ? 256 : (vec_per_row >= 128 ? 128 : 64);
  hipLaunchKernelGGL(scatter_kernel<u32x4>, dim3(p.T), dim3(threads), 0, st, p,
                     static_cast<const u32x4*>(x), topk_idx, ws.local_rank, ws.tile_hist, ws.seg,
                     ws.slot_pos, static_cast<u32x4*>(ws.xperm), vec_per_row);
  return hipGetLastError();
}

}  // namespace moe
