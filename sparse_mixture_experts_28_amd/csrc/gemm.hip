// moe_grouped_gemm: the expert FFNs over the ragged expert segments.
//   phase 1: H[seg rows] = GELU(A[seg rows] W1_e^T + b1_e)   (A = expert-sorted tokens,
//                                                              or x for a shared expert)
//   phase 2: Y[seg rows] = H[seg rows] W2_e^T + b2_e
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (each expert is
// Linear(d, 4d) -> GELU -> Linear(4d, d), with bias, applied to the tokens
// routed to it) and §7.1 (shared experts see every token); "[BEE-30064]
// 混合專家架構與服務" (compute grows with the active parameters, memory with the
// total); "第7章 Mixture of Experts" §7.3 (one shared plus many fine-grained
// routed experts).
//
// Both operands are K-contiguous (A rows and nn.Linear weight rows), so
// C = A B^T is the "NT" product that MFMA prefers.  All tiles are 256 columns
// wide with K steps of 64; accumulation is float32 on the 32x32x16 bf16 MFMA;
// the epilogue adds the bias and (phase 1) applies GELU(erf) in float32 and
// rounds once to bf16.
//
// Two bf16 kernels, chosen by the average rows per expert:
//  * 256-row tiles, 8 waves (compute-bound regime, e.g. 8 experts of ~2k rows):
//    two waves per SIMD, 128 x 64 wave tiles, two 64 KB LDS stages filled by
//    direct global->LDS loads one K step ahead.
//  * 128-row tiles, 4 waves (weight-streaming regime: many experts of ~100-400
//    rows): a 3-stage LDS ring filled two K steps ahead so ~96 KB per CU stay
//    in flight.
// Shared pieces: operands are read with buffer loads whose range check returns
// zero past a segment's last row (ragged tails need no clamping); LDS rows use
// a 16-byte-chunk XOR swizzle that makes the MFMA operand reads conflict-free;
// the grid is persistent (one workgroup per CU); workgroup b runs on XCD b % 8
// and the logical tile order gives each XCD a contiguous run of tiles grouped
// 8 M-tiles x N, so concurrently running tiles share A and B panels in that
// XCD's L2.
//
// Fallback (any shape, float32 or bf16): 64 x 64 SIMT tiles, float32 accumulation.
#include "moe_internal.h"

// Pin the MFMA / LDS-read / global-load interleave of the K steps.
#ifndef MOE_GEMM_SCHED
#define MOE_GEMM_SCHED 1
#endif

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const void* a_routed;  // phase 1: xperm; phase 2: hbuf
  const void* a_shared;  // phase 1: x;     phase 2: hbuf
  int a_by_o_off;        // phase 2: the A row offset of a segment is its output row offset
  const void* W;         // [nseg][N][K]
  const void* bias;      // [nseg][N]
  void* C;               // [rows][N]
  const int32_t* seg;    // segment table
  int nseg, E, N, K;
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier for the direct-load kernels.  __syncthreads() also waits
// for every outstanding global load (its fence emits vmcnt(0)), which would
// drain the global->LDS loads kept in flight across stages.  This barrier
// waits only for this wave's own LDS operations (lgkmcnt(0)); callers wait for
// the loads of a stage (vmcnt) themselves before the barrier that publishes it.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

// segment s containing global M-tile mt: tile_start[s] <= mt < tile_start[s+1]
__device__ __forceinline__ int find_segment(const int32_t* tile_start, int nseg, int mt) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// -------------------------------------------------------------- MFMA path --
constexpr int kBN = 256, kBK = 64;
constexpr int kGroupM = 8;
constexpr int kCh = kBK / 8;                   // 16-byte chunks per tile row
constexpr int kRsrcWord3 = 0x00020000;         // raw buffer, 32-bit data format (gfx9 family)

// LDS layout of a tile row of 64 bf16 (8 chunks of 16 bytes): logical chunk c
// of row r is stored at chunk c ^ (r & 7) ^ ((r >> 3) & 1).  A ds_read_b128
// of 16 consecutive rows at one logical chunk then touches 16 distinct
// 16-byte bank groups whether the LDS serves 8 or 16 lanes per cycle, and so
// does a ds_write_b128 of 2 rows x 8 chunks.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// ------------------------------------------------------ 8-wave MFMA path --
// 256 x 256 x 64 tile, 8 waves (2 per SIMD) in a 2 (M) x 4 (N) grid, wave tile
// 128 x 64 = 4 x 2 blocks of the 32x32x16 MFMA (128 float accumulators per
// lane).  With two waves per SIMD, one wave's MFMAs cover the other's LDS and
// memory waits.  Operand fragments are double-buffered in registers across
// the four 16-deep k-steps of a tile step.  Tiles reach LDS directly
// (buffer_load ... lds writes 64 lanes x 16 bytes contiguously at a
// wave-uniform LDS address), without passing through registers.
template <bool GELU>
__global__ __launch_bounds__(512) void gemm_bf16_w8_kernel(GemmArgs g) {
  constexpr int BM = 256;
  constexpr int kStage = (BM + kBN) * kCh;     // u32x4 per LDS stage (64 KB)
  __shared__ u32x4 lds[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const SegTable st = seg_table(const_cast<int32_t*>(g.seg), g.nseg, g.E);
  const int total_mt = uniform(st.tile_start[g.nseg]);
  const int ntn = g.N / kBN;
  const int total = total_mt * ntn;
  const int nk = g.K / kBK;
  const uint32_t row_bytes = static_cast<uint32_t>(g.K) * 2u;

  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  const uint16_t* Wb = static_cast<const uint16_t*>(g.W);
  const uint16_t* Bias = static_cast<const uint16_t*>(g.bias);
  uint16_t* C = static_cast<uint16_t*>(g.C);

  // direct loads: wave w, load i fills LDS rows 64 i + 8 w + lane / 8 at physical
  // chunk lane % 8, so the lane fetches the logical chunk that lands there
  const int dr_row = 8 * wave + (lane >> 3);
  const int dr_ch = (lane & 7) ^ (dr_row & 7) ^ ((dr_row >> 3) & 1);
  const int rd_row = lane & 31;

  for (int it = 0;; ++it) {
    const int L = it * gridDim.x + xcd * per_xcd + slot;
    if (L >= total) break;
    const int gsz = kGroupM * ntn;
    const int grp = L / gsz;
    const int first_m = grp * kGroupM;
    const int gm = min(kGroupM, total_mt - first_m);
    const int r = L - grp * gsz;
    const int mt = first_m + r % gm;
    const int nt = r / gm;

    const int s = uniform(find_segment(st.tile_start, g.nseg, mt));
    const int rows = uniform(st.rows[s]);
    const int m0 = (mt - uniform(st.tile_start[s])) * BM;
    const int a_off = uniform(g.a_by_o_off ? st.o_off[s] : st.a_off[s]);
    const int o_off = uniform(st.o_off[s]);
    const uint16_t* A = static_cast<const uint16_t*>(s < g.E ? g.a_routed : g.a_shared) +
                        static_cast<size_t>(a_off) * g.K;
    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(A, static_cast<uint32_t>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        make_rsrc(Wb + static_cast<size_t>(s) * g.N * g.K, static_cast<uint32_t>(g.N) * row_bytes);
    const int n0 = nt * kBN;
    const uint32_t step64 = 64u * row_bytes;
    const uint32_t va = static_cast<uint32_t>(m0 + dr_row) * row_bytes + dr_ch * 16;
    const uint32_t vb = static_cast<uint32_t>(n0 + dr_row) * row_bytes + dr_ch * 16;

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto issue = [&](int stage, int kb) {
      u32x4* base = lds + stage * kStage + (8 * wave) * kCh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rsrc, (__attribute__((address_space(3))) void*)(base + 64 * i * kCh), 16, va, i * step64 + kb, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb_rsrc, (__attribute__((address_space(3))) void*)(base + (BM + 64 * i) * kCh), 16, vb,
            i * step64 + kb, 0, 0);
      }
    };
    // this wave's loads into the other stage have landed (published by the barrier)
    auto commit = [&](int) { __builtin_amdgcn_s_waitcnt(0); };

    issue(0, 0);
    commit(0);
    lds_barrier();

    // One K step: fragments of k-substep ks+1 and (when `load`) the next
    // stage's global loads are issued between the MFMAs of ks, one at a time,
    // so LDS and memory latency overlap the matrix pipe.
    auto kstep = [&](int kt, bool load) {
      const int cur = kt & 1;
      const u32x4* sa = lds + cur * kStage;
      const u32x4* sb = sa + BM * kCh;
      bf16x8 fa[2][4], fb[2][2];
      auto frag = [&](int ks, int buf) {
        const int ch = swz(rd_row, 2 * ks + (lane >> 5));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[buf][i] = __builtin_bit_cast(bf16x8, sa[(wm * 128 + i * 32 + rd_row) * kCh + ch]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[buf][j] = __builtin_bit_cast(bf16x8, sb[(wn * 64 + j * 32 + rd_row) * kCh + ch]);
      };
      frag(0, 0);
      if (load) issue(cur ^ 1, (kt + 1) * kBK * 2);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        if (ks + 1 < kBK / 16) frag(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
#if MOE_GEMM_SCHED
        if (ks == 0 && load) {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 global load
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        } else if (ks + 1 < kBK / 16) {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
#endif
      }
      if (load) commit(cur ^ 1);
      lds_barrier();
    };
    for (int kt = 0; kt + 1 < nk; ++kt) kstep(kt, true);
    kstep(nk - 1, false);

    // epilogue: accumulator v of block (i, j) holds row 8 (v / 4) + 4 (lane / 32) + v % 4,
    // column lane % 32 of that block
    const int col0 = n0 + wn * 64 + (lane & 31);
    float bj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) bj[j] = bf16_to_f32(Bias[static_cast<size_t>(s) * g.N + col0 + j * 32]);
    const bool full = m0 + BM <= rows;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (full || rl < rows) {
          uint16_t* crow = C + static_cast<size_t>(o_off + rl) * g.N + col0;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float val = acc[i][j][v] + bj[j];
            if (GELU) val = gelu_erf(val);
            crow[j * 32] = f32_to_bf16(val);
          }
        }
      }
    }
  }
}

// ------------------------------------------------- 128-row streaming path --
// For experts with few rows each (fine-grained experts, capacity-limited
// experts) the GEMM is bound by streaming the expert weights from HBM.
// 128 x 256 x 64 tiles, 4 waves (2 x 2, wave tile 64 x 128), direct
// global->LDS loads into a 3-stage LDS ring (48 KB per stage), issued two K
// steps ahead so ~96 KB per CU stay in flight.  The barrier before K step
// k+1 waits only for stage k+1 (vmcnt), never for stage k+2.
template <bool GELU>
__global__ __launch_bounds__(256) void gemm_bf16_stream_kernel(GemmArgs g) {
  constexpr int BM = 128;
  constexpr int NS = 3;
  constexpr int kStage = (BM + kBN) * kCh;     // u32x4 per stage (48 KB)
  constexpr int LA = BM / 32, LB = kBN / 32;   // direct loads per wave per stage (4 + 8)
  __shared__ u32x4 lds[NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const SegTable st = seg_table(const_cast<int32_t*>(g.seg), g.nseg, g.E);
  const int total_mt = uniform(st.tile_start[g.nseg]);
  const int ntn = g.N / kBN;
  const int total = total_mt * ntn;
  const int nk = g.K / kBK;
  const uint32_t row_bytes = static_cast<uint32_t>(g.K) * 2u;

  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  const uint16_t* Wb = static_cast<const uint16_t*>(g.W);
  const uint16_t* Bias = static_cast<const uint16_t*>(g.bias);
  uint16_t* C = static_cast<uint16_t*>(g.C);

  // direct loads: wave w's load i fills LDS rows 8 (4 i + w) + lane / 8 at
  // physical chunk lane % 8, fetching the logical chunk that lands there
  const int dr_row = 8 * wave + (lane >> 3);
  const int dr_ch = swz(dr_row, lane & 7);
  const int rd_row = lane & 31;

  for (int it = 0;; ++it) {
    const int L = it * gridDim.x + xcd * per_xcd + slot;
    if (L >= total) break;
    const int gsz = kGroupM * ntn;
    const int gq = L / gsz;
    const int first_m = gq * kGroupM;
    const int gm = min(kGroupM, total_mt - first_m);
    const int r = L - gq * gsz;
    const int mt = first_m + r % gm;
    const int nt = r / gm;

    const int s = uniform(find_segment(st.tile_start, g.nseg, mt));
    const int rows = uniform(st.rows[s]);
    const int m0 = (mt - uniform(st.tile_start[s])) * BM;
    const int a_off = uniform(g.a_by_o_off ? st.o_off[s] : st.a_off[s]);
    const int o_off = uniform(st.o_off[s]);
    const uint16_t* A = static_cast<const uint16_t*>(s < g.E ? g.a_routed : g.a_shared) +
                        static_cast<size_t>(a_off) * g.K;
    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(A, static_cast<uint32_t>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        make_rsrc(Wb + static_cast<size_t>(s) * g.N * g.K, static_cast<uint32_t>(g.N) * row_bytes);
    const int n0 = nt * kBN;
    const uint32_t step32 = 32u * row_bytes;
    const uint32_t va = static_cast<uint32_t>(m0 + dr_row) * row_bytes + dr_ch * 16;
    const uint32_t vb = static_cast<uint32_t>(n0 + dr_row) * row_bytes + dr_ch * 16;

    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto issue = [&](int k) {
      u32x4* base = lds + (k % NS) * kStage + (8 * wave) * kCh;
      const int kb = k * kBK * 2;
#pragma unroll
      for (int i = 0; i < LA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rsrc, (__attribute__((address_space(3))) void*)(base + 32 * i * kCh), 16, va, i * step32 + kb, 0, 0);
#pragma unroll
      for (int i = 0; i < LB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb_rsrc, (__attribute__((address_space(3))) void*)(base + (BM + 32 * i) * kCh), 16, vb,
            i * step32 + kb, 0, 0);
    };

    issue(0);
    if (nk > 1) {
      issue(1);
      __builtin_amdgcn_s_waitcnt(0x0F7C);   // vmcnt <= 12: stage 0 landed, stage 1 may be in flight
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    lds_barrier();

    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 2 < nk) issue(kt + 2);      // slot of stage kt-1, read before the last barrier
      const u32x4* sa = lds + (kt % NS) * kStage;
      const u32x4* sb = sa + BM * kCh;
      bf16x8 fa[2][2], fb[2][4];
      auto frag = [&](int ks, int buf) {
        const int ch = swz(rd_row, 2 * ks + (lane >> 5));
#pragma unroll
        for (int i = 0; i < 2; ++i)
          fa[buf][i] = __builtin_bit_cast(bf16x8, sa[(wm * 64 + i * 32 + rd_row) * kCh + ch]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fb[buf][j] = __builtin_bit_cast(bf16x8, sb[(wn * 128 + j * 32 + rd_row) * kCh + ch]);
      };
      frag(0, 0);
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        if (ks + 1 < kBK / 16) frag(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
      }
      // before K step kt+1: its stage has landed (stage kt+2's loads may stay in flight)
      if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F7C);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }

    // epilogue: accumulator v of block (i, j) holds row 8 (v / 4) + 4 (lane / 32) + v % 4,
    // column lane % 32 of that block
    const int col0 = n0 + wn * 128 + (lane & 31);
    float bj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bj[j] = bf16_to_f32(Bias[static_cast<size_t>(s) * g.N + col0 + j * 32]);
    const bool full = m0 + BM <= rows;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (full || rl < rows) {
          uint16_t* crow = C + static_cast<size_t>(o_off + rl) * g.N + col0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float val = acc[i][j][v] + bj[j];
            if (GELU) val = gelu_erf(val);
            crow[j * 32] = f32_to_bf16(val);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------ SIMT path --
constexpr int kSB = 64, kSK = 16;

__device__ __forceinline__ float ld_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st_out(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename TIn, bool GELU>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmArgs g, int max_mt) {
  __shared__ float sA[kSK][kSB + 1];
  __shared__ float sB[kSK][kSB + 1];
  const SegTable st = seg_table(const_cast<int32_t*>(g.seg), g.nseg, g.E);
  const int total_mt = st.tile_start[g.nseg];
  const int mt = blockIdx.x;
  if (mt >= total_mt) return;
  (void)max_mt;
  const int s = find_segment(st.tile_start, g.nseg, mt);
  const int rows = st.rows[s];
  const int m0 = (mt - st.tile_start[s]) * kSB;
  const int n0 = blockIdx.y * kSB;
  const int a_off = g.a_by_o_off ? st.o_off[s] : st.a_off[s];
  const TIn* A = static_cast<const TIn*>(s < g.E ? g.a_routed : g.a_shared) + static_cast<size_t>(a_off) * g.K;
  const TIn* B = static_cast<const TIn*>(g.W) + static_cast<size_t>(s) * g.N * g.K;
  const TIn* Bias = static_cast<const TIn*>(g.bias) + static_cast<size_t>(s) * g.N;
  TIn* C = static_cast<TIn*>(g.C);

  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += kSK) {
    for (int i = threadIdx.x; i < kSB * kSK; i += 256) {
      const int rr = i / kSK, kk = i % kSK;
      const int gm_ = m0 + rr, gk = k0 + kk, gn = n0 + rr;
      sA[kk][rr] = (gm_ < rows && gk < g.K) ? ld_f32(A, static_cast<size_t>(gm_) * g.K + gk) : 0.f;
      sB[kk][rr] = (gn < g.N && gk < g.K) ? ld_f32(B, static_cast<size_t>(gn) * g.K + gk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int o_off = st.o_off[s];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = m0 + ty * 4 + i;
    if (rl >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= g.N) continue;
      float v = acc[i][j] + ld_f32(Bias, col);
      if (GELU) v = gelu_erf(v);
      st_out(C, static_cast<size_t>(o_off + rl) * g.N + col, v);
    }
  }
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

}  // namespace

bool gemm_fast_path(const Problem& p) {
  if (p.dtype != MOE_BF16 || p.h % kBN != 0 || p.d % kBN != 0 || p.d % kBK != 0 || p.h % kBK != 0) return false;
  // buffer offsets are 32-bit: every operand region must stay below 2 GiB
  const long long rows = static_cast<long long>(p.T) * p.k + static_cast<long long>(p.S) * p.T + 256;
  const long long widest = p.d > p.h ? p.d : p.h;
  return rows * widest * 2 < (1LL << 31) && static_cast<long long>(p.h) * p.d * 2 < (1LL << 31);
}

// 256-row tiles (compute-bound, 8-wave kernel) for segments that average
// >= 512 rows; 128-row tiles (weight streaming kernel) otherwise.
int gemm_m_tile(const Problem& p) {
  if (!gemm_fast_path(p)) return kSB;
  long long avg = static_cast<long long>(p.T) * p.k / p.E;
  if (p.cap < avg) avg = p.cap;
  return avg >= 512 ? 256 : 128;
}

hipError_t launch_expert_ffn(const Problem& p, const void* x, const void* W1, const void* b1, const void* W2,
                             const void* b2, const Workspace& ws, int phase, hipStream_t st) {
  GemmArgs g;
  g.seg = ws.seg;
  g.nseg = p.E + p.S;
  g.E = p.E;
  if (phase == 1) {
    g.a_routed = ws.xperm;
    g.a_shared = x;
    g.a_by_o_off = 0;
    g.W = W1;
    g.bias = b1;
    g.C = ws.hbuf;
    g.N = p.h;
    g.K = p.d;
  } else {
    g.a_routed = ws.hbuf;
    g.a_shared = ws.hbuf;
    g.a_by_o_off = 1;
    g.W = W2;
    g.bias = b2;
    g.C = ws.ybuf;
    g.N = p.d;
    g.K = p.h;
  }
  if (gemm_fast_path(p)) {
    int grid = num_cus();
    grid = (grid + 7) / 8 * 8;
    if (p.gemm_bm == 256) {
      if (phase == 1)
        hipLaunchKernelGGL((gemm_bf16_w8_kernel<true>), dim3(grid), dim3(512), 0, st, g);
      else
        hipLaunchKernelGGL((gemm_bf16_w8_kernel<false>), dim3(grid), dim3(512), 0, st, g);
    } else {
      if (phase == 1)
        hipLaunchKernelGGL((gemm_bf16_stream_kernel<true>), dim3(grid), dim3(256), 0, st, g);
      else
        hipLaunchKernelGGL((gemm_bf16_stream_kernel<false>), dim3(grid), dim3(256), 0, st, g);
    }
  } else {
    // upper bound of M tiles: sum_e ceil(rows_e / 64) <= ceil(T k / 64) + E + S ceil(T / 64)
    const long long max_mt = (static_cast<long long>(p.T) * p.k + kSB - 1) / kSB + p.E +
                             static_cast<long long>(p.S) * ((p.T + kSB - 1) / kSB);
    dim3 grid(static_cast<unsigned>(max_mt), (g.N + kSB - 1) / kSB);
    if (p.dtype == MOE_BF16) {
      if (phase == 1)
        hipLaunchKernelGGL((gemm_simt_kernel<uint16_t, true>), grid, dim3(256), 0, st, g, (int)max_mt);
      else
        hipLaunchKernelGGL((gemm_simt_kernel<uint16_t, false>), grid, dim3(256), 0, st, g, (int)max_mt);
    } else {
      if (phase == 1)
        hipLaunchKernelGGL((gemm_simt_kernel<float, true>), grid, dim3(256), 0, st, g, (int)max_mt);
      else
        hipLaunchKernelGGL((gemm_simt_kernel<float, false>), grid, dim3(256), 0, st, g, (int)max_mt);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
