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
// permute (top-k routing; one workgroup per router tile): each workgroup
//         adds the per-tile expert counts of the tiles before its own (its
//         tile's base rank per expert) and of all tiles (c_e), so no workgroup
//         waits for another; kept_e = min(c_e, cap) and an exclusive scan of
//         kept over experts give the segment offsets; then each assignment of
//         the tile: rank = tile base + in-tile rank, kept iff rank < cap, its
//         row in the expert-sorted order and that row's token are recorded.
//         No token row is copied: the expert GEMM gathers x rows through
//         row_token.  Workgroup 0 also writes the counts, finalises the
//         balance loss from c and the per-tile probability sums and the router
//         z-loss from the per-tile sums of squared log-sum-exp (both float64,
//         fixed order), and writes the grouped-GEMM segment table.
// scan    (expert choice; 1 workgroup of 1024): the same finalisation with
//         every expert taking exactly C tokens (the selection kernel then
//         lists them).
//
// Every result is a fixed function of the inputs: the only atomics are
// integer additions into LDS (exact in any order); float sums run in a fixed order.
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
    int q = 0;
    // eight chunks' reads issued together, then used in chunk order
    for (; q + 8 <= C; q += 8) {
      int v[8];
      double w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u] = s_sum[(q + u) * E + t];
        w[u] = s_psum[(q + u) * E + t];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s_sum[(q + u) * E + t] = run;
        run += v[u];
        pr += w[u];
      }
    }
    for (; q < C; ++q) {
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

constexpr int kPermThreads = 512;
static_assert(kPermThreads >= kRouterTile * MOE_MAX_TOPK, "one assignment of a router tile a thread");
constexpr int kSegSlots = 512;   // >= MOE_MAX_EXPERTS + MOE_MAX_SHARED

// Fixed butterfly sums over a wave (the same tree on every call: deterministic).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// In-place inclusive scan of v[0 .. kSegSlots) by one wave (lane l owns
// entries 8 l .. 8 l + 7: a serial prefix, then a scan of the lane totals);
// the caller publishes the result with a barrier.
__device__ __forceinline__ void wave_scan_incl(int32_t* v, int lane) {
  static_assert(kSegSlots == 8 * kWave, "eight entries a lane");
  int x[8], run = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    run += v[8 * lane + i];
    x[i] = run;
  }
  int incl = run;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  const int base = incl - run;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[8 * lane + i] = base + x[i];
}

// Workgroup 0's per-thread partial sums for the balance loss and the z-loss,
// loaded at the start of the kernel so their loads overlap the count
// table's: thread (q, e), q < G = min(64, 512 / E), adds the probability sums
// of tiles q, q + G, ... of expert e in order (independent loads, all in
// flight: one batch for up to 16 G tiles); lane l of wave 1 adds the z-loss
// sums of tiles l, l + 64, ... in order.
struct FinalPartials {
  double ps;   // P_e partial of thread (q, e)
  double zs;   // z-loss partial of a wave-1 lane
};

__device__ FinalPartials final_partials(const Problem& p, const float* __restrict__ p_part,
                                        const double* __restrict__ z_part) {
  const int E = p.E;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  FinalPartials fp{0.0, 0.0};
  const int G = min(64, kPermThreads / E), e = t % E, q = t / E;
  if (q < G) {
    // sixteen, then eight loads issued together, then added in order
    int j = q;
    for (; j + 15 * G < p.ntile; j += 16 * G) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = p_part[static_cast<size_t>(j + u * G) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) fp.ps += static_cast<double>(v[u]);
    }
    for (; j + 7 * G < p.ntile; j += 8 * G) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p_part[static_cast<size_t>(j + u * G) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) fp.ps += static_cast<double>(v[u]);
    }
    for (; j < p.ntile; j += G) fp.ps += static_cast<double>(p_part[static_cast<size_t>(j) * E + e]);
  }
  if (wave == 1) {
#pragma unroll 4
    for (int j = lane; j < p.ntile; j += kWave) fp.zs += z_part[j];
  }
  return fp;
}

// Workgroup 0's finalisation: counts, kept, the balance loss, the router
// z-loss and the grouped-GEMM segment table, from s_cnt (c_e), s_off
// (exclusive scan of kept over the experts) and the partial sums above.
// Float64 sums in a fixed order: the G partials of an expert in order, a
// fixed butterfly over the lanes of a wave.
__device__ void finalize_tables(const Problem& p, const FinalPartials& fp, const int32_t* s_cnt,
                                const int32_t* s_off, int32_t* counts, int32_t* kept, int32_t* seg_base,
                                float* aux_loss, float* z_loss, int32_t* counts_out, int32_t* kept_out) {
  __shared__ double s_term[MOE_MAX_EXPERTS];
  __shared__ int32_t s_tiles[kSegSlots];
  const int E = p.E, nseg = p.E + p.S;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  __shared__ double s_ppart[kPermThreads];
  s_ppart[t] = fp.ps;
  __syncthreads();
  if (t < E) {
    const int G = min(64, kPermThreads / E);
    double ps = 0.0;
    for (int q = 0; q < G; ++q) ps += s_ppart[q * E + t];
    s_term[t] = (static_cast<double>(s_cnt[t]) / static_cast<double>(p.A)) * (ps / static_cast<double>(p.T));
  }
  const int my_kept = t < E ? min(s_cnt[t], p.cap) : 0;
  if (t < E) {
    counts[t] = s_cnt[t];
    kept[t] = my_kept;
    if (counts_out) counts_out[t] = s_cnt[t];
    if (kept_out) kept_out[t] = my_kept;
  }
  // segment rows and M tiles (routed experts, then shared)
  int my_rows = 0, my_tiles = 0, my_bm = p.gemm_bm;
  if (t < nseg) {
    my_rows = t < E ? my_kept : p.T;
    if (p.gemm_mixed) my_bm = mx_mixed_tile_height(my_rows);
    my_tiles = (my_rows + my_bm - 1) / my_bm;
  }
  s_tiles[t] = my_tiles;
  __syncthreads();
  if (wave == 0) wave_scan_incl(s_tiles, lane);
  __syncthreads();
  if (wave == 0) {
    // aux = E sum_e f_e P_e
    double a = 0.0;
    for (int e = lane; e < E; e += kWave) a += s_term[e];
    a = wave_sum(a);
    if (lane == 0 && aux_loss) *aux_loss = static_cast<float>(static_cast<double>(E) * a);
  } else if (wave == 1) {
    // z = (1/T) sum of the tiles' sums of squared log-sum-exp
    const double z = wave_sum(fp.zs);
    if (lane == 0 && z_loss) *z_loss = static_cast<float>(z / static_cast<double>(p.T));
  }
  if (t < nseg) {
    const SegTable st = seg_table(seg_base, nseg, E);
    const int excl_rows = t < E ? s_off[t] : 0;
    st.rows[t] = my_rows;
    st.a_off[t] = excl_rows;
    st.o_off[t] = t < E ? excl_rows : p.A + (t - E) * p.T;
    st.tile_start[t] = s_tiles[t] - my_tiles;
    st.tile_bm[t] = my_bm;
    if (t < E) st.route_off[t] = excl_rows;
    if (t == nseg - 1) st.tile_start[nseg] = s_tiles[t];
  }
}

// One workgroup per router tile of p.rtile tokens.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(Problem p, const int32_t* __restrict__ topk_idx,
                                                               const int32_t* __restrict__ local_rank,
                                                               const int32_t* __restrict__ tile_hist,
                                                               const float* __restrict__ p_part,
                                                               const double* __restrict__ z_part, int32_t* counts,
                                                               int32_t* kept, int32_t* seg_base, float* aux_loss,
                                                               float* z_loss, int32_t* counts_out, int32_t* kept_out,
                                                               int32_t* __restrict__ slot_pos,
                                                               int32_t* __restrict__ row_token) {
  __shared__ int32_t s_base[MOE_MAX_EXPERTS];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS];
  const int E = p.E, k = p.k;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int tile = blockIdx.x;
  // this tile's assignments (at most 64 tokens x 8 = 512, one a thread): their
  // expert and in-tile rank are loaded first, so the load overlaps the count
  // table's
  const int tok0 = tile * p.rtile;
  const int n_asg = min(p.rtile, p.T - tok0) * k;
  int my_ex = 0, my_lr = 0;
  if (t < n_asg) {
    const size_t a = static_cast<size_t>(tok0) * k + t;
    my_ex = topk_idx[a];
    my_lr = local_rank[a];
  }
  // workgroup 0 also starts the loads of the loss partials
  FinalPartials fp{0.0, 0.0};
  if (tile == 0) fp = final_partials(p, p_part, z_part);
  // 1. per expert, the counts of the tiles before this one (its base rank)
  // and of all tiles (c_e): the [ntile, E] table read in order by all threads
  // (coalesced, every load independent), added into LDS with integer atomics
  // (order-free, so the sums are exact and deterministic)
  if (t < E) {
    s_base[t] = 0;
    s_cnt[t] = 0;
  }
  __syncthreads();
  {
    const int n = p.ntile * E, before_end = tile * E;
    auto add = [&](int i, int h) {
      if (h != 0) {
        const int ex = i % E;
        atomicAdd(&s_cnt[ex], h);
        if (i < before_end) atomicAdd(&s_base[ex], h);
      }
    };
    // eight loads issued together, then their atomics
    int i = t;
    for (; i + 7 * kPermThreads < n; i += 8 * kPermThreads) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = tile_hist[i + u * kPermThreads];
#pragma unroll
      for (int u = 0; u < 8; ++u) add(i + u * kPermThreads, h[u]);
    }
    for (; i < n; i += kPermThreads) add(i, tile_hist[i]);
  }
  __syncthreads();
  // 2. segment offsets: exclusive scan of kept over the experts (wave 0,
  // four experts per lane)
  if (wave == 0) {
    int kp[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = 4 * lane + i;
      kp[i] = ex < E ? min(s_cnt[ex], p.cap) : 0;
      own += kp[i];
    }
    int incl = own;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    int run = incl - own;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = 4 * lane + i;
      if (ex < E) s_off[ex] = run;
      run += kp[i];
    }
  }
  __syncthreads();
  // 3. this tile's assignments (their expert and in-tile rank were loaded at
  // the start)
  if (t < n_asg) {
    const size_t a = static_cast<size_t>(tok0) * k + t;
    const int rank = s_base[my_ex] + my_lr;
    const int pos = rank < p.cap ? s_off[my_ex] + rank : -1;
    slot_pos[a] = pos;
    if (pos >= 0) row_token[pos] = tok0 + t / k;
  }
  if (tile == 0)
    finalize_tables(p, fp, s_cnt, s_off, counts, kept, seg_base, aux_loss, z_loss, counts_out, kept_out);
}

}  // namespace

hipError_t launch_scan(const Problem& p, const Workspace& ws, float* aux_loss, float* z_loss, int32_t* counts_out,
                       int32_t* kept_out, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, p, ws.tile_hist, ws.p_part, ws.z_part,
                     ws.counts, ws.kept, ws.seg, aux_loss, z_loss, counts_out, kept_out);
  return hipGetLastError();
}

hipError_t launch_permute(const Problem& p, const int32_t* topk_idx, const Workspace& ws, float* aux_loss,
                          float* z_loss, int32_t* counts_out, int32_t* kept_out, hipStream_t st) {
  hipLaunchKernelGGL(permute_kernel, dim3(p.ntile), dim3(kPermThreads), 0, st, p, topk_idx, ws.local_rank, ws.tile_hist,
                     ws.p_part, ws.z_part, ws.counts, ws.kept, ws.seg, aux_loss, z_loss, counts_out, kept_out,
                     ws.slot_pos, ws.row_token);
  return hipGetLastError();
}

}  // namespace moe
