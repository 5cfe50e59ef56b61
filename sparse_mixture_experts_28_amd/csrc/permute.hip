// moe_permute: turn the router's per-tile histograms and in-tile ranks into a
// deterministic, capacity-limited, expert-sorted order of the token rows.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (the mask of tokens routed
// to each expert, gathered per expert), §8.2 and "第7章 Mixture of Experts"
// §7.4 (capacity = factor x tokens / experts, overflow tokens dropped or passed
// by the residual outside the layer); §4.3 of the guide (balance loss
// E * sum f_i P_i); "第7章" tensor-shape trace (the token -> expert reordering
// is the real cost of the layer).
//
// scan    (1 workgroup of 1024): for every expert, an exclusive scan of its
//         per-tile counts over the tiles in token order gives each tile's base rank;
//         the total is c_e, kept_e = min(c_e, cap); an exclusive scan of kept
//         over experts gives the segment offsets; the balance loss is
//         finalised from c and the per-tile probability sums, the router
//         z-loss from the per-tile sums of squared log-sum-exp (both float64,
//         fixed order); the grouped-GEMM segment table is written.
// scatter (1 thread per assignment): rank = tile base + in-tile rank; the
//         assignment is kept iff rank < cap; its row in the expert-sorted
//         order and that row's token are recorded.  No token row is copied:
//         the expert GEMM gathers x rows through row_token.
//
// No atomics anywhere: every result is a fixed function of the inputs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// Thread t works on expert e = t % E over the tiles of chunk c = t / E (C
// chunks of consecutive tiles); per-chunk totals are scanned over c in LDS in
// fixed order, so bases, counts and the probability sums are deterministic.
// The per-tile tables are tile-major [ntile][E], so the lanes of a wave
// (consecutive experts) read and write consecutive words.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(Problem p, int32_t* tile_hist, const float* p_part,
                                                            const double* z_part, int32_t* counts, int32_t* kept,
                                                            int32_t* seg_base, float* aux_loss, float* z_loss,
                                                            int32_t* counts_out, int32_t* kept_out) {
  __shared__ int32_t s_sum[kScanThreads];
  __shared__ double s_psum[kScanThreads];
  __shared__ int32_t s_kept[MOE_MAX_EXPERTS];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ double s_P[MOE_MAX_EXPERTS];
  const int E = p.E;
  const int nseg = p.E + p.S;
  SegTable st = seg_table(seg_base, nseg, E);
  const int C = max(1, kScanThreads / E);
  const int tpc = (p.ntile + C - 1) / C;
  const int t = threadIdx.x;
  const int e = t % E, c = t / E;
  const bool active = c < C;
  const int tb = c * tpc, te = min(p.ntile, tb + tpc);

  // 1. chunk totals
  int sum = 0;
  double psum = 0.0;
  const int32_t* hcol = tile_hist + e;   // tile i of expert e at i * E
  const float* pcol = p_part + e;
  const bool ec = p.ec_C > 0;   // expert choice: every expert takes exactly ec_C tokens
  if (active) {
#pragma unroll 8
    for (int tile = tb; tile < te; ++tile) {
      if (!ec) sum += hcol[static_cast<size_t>(tile) * E];
      psum += static_cast<double>(pcol[static_cast<size_t>(tile) * E]);
    }
    s_sum[c * E + e] = sum;
    s_psum[c * E + e] = psum;
  }
  __syncthreads();
  // 2. per expert: exclusive scan of the chunk totals (in place), totals
  if (t < E) {
    int run = 0;
    double pr = 0.0;
    for (int q = 0; q < C; ++q) {
      const int v = s_sum[q * E + t];
      s_sum[q * E + t] = run;
      run += v;
      pr += s_psum[q * E + t];
    }
    if (ec) run = p.ec_C;
    const int kp = min(run, p.cap);
    counts[t] = run;
    kept[t] = kp;
    if (counts_out) counts_out[t] = run;
    if (kept_out) kept_out[t] = kp;
    s_kept[t] = kp;
    s_cnt[t] = run;
    s_P[t] = pr / static_cast<double>(p.T);
  }
  __syncthreads();
  // 3. tile bases within the chunk (token choice only)
  if (active && !ec) {
    int run = s_sum[c * E + e];
    int32_t* wcol = tile_hist + e;
#pragma unroll 8
    for (int tile = tb; tile < te; ++tile) {
      const int h = wcol[static_cast<size_t>(tile) * E];
      wcol[static_cast<size_t>(tile) * E] = run;   // becomes the tile's base rank for expert e
      run += h;
    }
  }

  // 4. aux = E * sum_e f_e P_e, f_e = c_e / (T k): a fixed-order tree over experts;
  // z = (1/T) sum_t lse_t^2: contiguous runs of tiles per thread, then a fixed-order tree
  __shared__ double s_aux[MOE_MAX_EXPERTS];
  __shared__ double s_z[kScanThreads];
  {
    const int zc = (p.ntile + kScanThreads - 1) / kScanThreads;
    const int zb = t * zc, ze = min(p.ntile, zb + zc);
    double zs = 0.0;
    for (int tile = zb; tile < ze; ++tile) zs += z_part[tile];
    s_z[t] = zs;
  }
  // f_e = c_e / (all assignments): T k, or E C under expert choice
  const double tk = static_cast<double>(p.A);
  if (t < MOE_MAX_EXPERTS) s_aux[t] = t < E ? (static_cast<double>(s_cnt[t]) / tk) * s_P[t] : 0.0;
  // 5. segment table: one thread per segment (routed experts, then shared)
  constexpr int kSegSlots = 512;   // >= MOE_MAX_EXPERTS + MOE_MAX_SHARED
  __shared__ int32_t s_rows[kSegSlots];
  __shared__ int32_t s_tiles[kSegSlots];
  int my_rows = 0, my_tiles = 0, my_bm = p.gemm_bm;
  if (t < nseg) {
    my_rows = t < E ? s_kept[t] : p.T;
    if (p.gemm_mixed) my_bm = mx_mixed_tile_height(my_rows);
    my_tiles = (my_rows + my_bm - 1) / my_bm;
  }
  if (t < kSegSlots) {
    s_rows[t] = t < E ? my_rows : 0;     // only routed rows are packed in the sorted buffer
    s_tiles[t] = my_tiles;
  }
  __syncthreads();
  for (int w = MOE_MAX_EXPERTS / 2; w > 0; w >>= 1) {
    if (t < w) s_aux[t] += s_aux[t + w];
    __syncthreads();
  }
  if (t == 0 && aux_loss) *aux_loss = static_cast<float>(static_cast<double>(E) * s_aux[0]);
  for (int w = kScanThreads / 2; w > 0; w >>= 1) {
    if (t < w) s_z[t] += s_z[t + w];
    __syncthreads();
  }
  if (t == 0 && z_loss) *z_loss = static_cast<float>(s_z[0] / static_cast<double>(p.T));
  // inclusive scans of routed rows and of M tiles over the segments
  for (int off = 1; off < kSegSlots; off <<= 1) {
    int ar = 0, at = 0;
    if (t < kSegSlots && t >= off) {
      ar = s_rows[t - off];
      at = s_tiles[t - off];
    }
    __syncthreads();
    if (t < kSegSlots) {
      s_rows[t] += ar;
      s_tiles[t] += at;
    }
    __syncthreads();
  }
  if (t < nseg) {
    const int routed_rows = p.A;
    const int excl_rows = s_rows[t] - (t < E ? my_rows : 0);
    st.rows[t] = my_rows;
    st.a_off[t] = t < E ? excl_rows : 0;
    st.o_off[t] = t < E ? excl_rows : routed_rows + (t - E) * p.T;
    st.tile_start[t] = s_tiles[t] - my_tiles;
    st.tile_bm[t] = my_bm;
    if (t < E) st.route_off[t] = excl_rows;
    if (t == nseg - 1) st.tile_start[nseg] = s_tiles[t];
  }
}

// One thread per assignment (t, j): its rank among expert e's assignments in
// token order is the tile base plus the in-tile rank; kept iff rank < cap.
// Writes the assignment's row in the expert-sorted order (slot_pos, -1 if
// dropped) and that row's token (row_token), which the expert GEMM gathers
// its phase-1 rows through.  Every kept row gets exactly one writer.
__global__ __launch_bounds__(256) void scatter_kernel(Problem p, const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ local_rank,
                                                      const int32_t* __restrict__ tile_base,
                                                      const int32_t* __restrict__ seg_base,
                                                      int32_t* __restrict__ slot_pos,
                                                      int32_t* __restrict__ row_token) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.T * p.k) return;
  const int t = i / p.k;
  const int e = topk_idx[i];
  const int rank = tile_base[static_cast<size_t>(t / kRouterTile) * p.E + e] + local_rank[i];
  SegTable st = seg_table(const_cast<int32_t*>(seg_base), p.E + p.S, p.E);
  const int pos = rank < p.cap ? st.route_off[e] + rank : -1;
  slot_pos[i] = pos;
  if (pos >= 0) row_token[pos] = t;
}

}  // namespace

hipError_t launch_scan(const Problem& p, const Workspace& ws, float* aux_loss, float* z_loss, int32_t* counts_out,
                       int32_t* kept_out, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, p, ws.tile_hist, ws.p_part, ws.z_part,
                     ws.counts, ws.kept, ws.seg, aux_loss, z_loss, counts_out, kept_out);
  return hipGetLastError();
}

hipError_t launch_scatter(const Problem& p, const int32_t* topk_idx, const Workspace& ws, hipStream_t st) {
  const int n = p.T * p.k;
  hipLaunchKernelGGL(scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, topk_idx, ws.local_rank,
                     ws.tile_hist, ws.seg, ws.slot_pos, ws.row_token);
  return hipGetLastError();
}

}  // namespace moe
