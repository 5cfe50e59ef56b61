// moe_grouped_gemm: the expert FFNs over the ragged expert segments.
//   phase 1: H[seg rows] = act(A[seg rows] W1_e^T + b1_e)    (A = expert-sorted tokens,
//                                                              or x for a shared expert)
//   phase 2: Y[seg rows] = H[seg rows] W2_e^T + b2_e
// act is GELU (erf form) or SiLU; a missing bias (NULL) is left out.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §3.1 (each expert is
// Linear(d, 4d) -> GELU -> Linear(4d, d), with bias, applied to the tokens
// routed to it), §6.1 (the Mixtral expert: bias-free Linear -> SiLU ->
// bias-free Linear) and §7.1 (shared experts see every token); "[BEE-30064]
// 混合專家架構與服務" (compute grows with the active parameters, memory with the
// total); "第7章 Mixture of Experts" §7.3 (one shared plus many fine-grained
// routed experts).
//
// Both operands are K-contiguous (A rows and nn.Linear weight rows), so
// C = A B^T is the "NT" product that MFMA prefers.  Tiles are BM x 256 with
// K steps of 64, BM in {128, 160, 256} chosen per problem; accumulation is
// float32 on the 16x16x32 bf16 MFMA, starting from the bias; the epilogue
// (phase 1) applies the activation in float32 and rounds once to bf16.  The tail of a
// persistent launch is split along K (stream-K style) with a deterministic
// fix-up.
//
// Shared pieces: operands are read with buffer loads whose range check returns
// zero past a segment's last row (ragged tails need no clamping); LDS rows use
// a 16-byte-chunk XOR swizzle that makes the MFMA operand reads conflict-free;
// the grid is persistent (one workgroup per CU); workgroup b runs on XCD b % 8
// and the logical tile order gives each XCD a contiguous run of tiles grouped
// 8 M-tiles x N, so concurrently running tiles share A and B panels in that
// XCD's L2.
//
// float32 layers run a float32 matrix-core kernel (BM x 128 tiles, K slabs
// of 32 through LDS).  Fallback (bf16 with d or h not a multiple of 256):
// 64 x 64 SIMT tiles, float32 accumulation.
#include "moe_internal.h"


namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// Row r of segment s reads A row
//   row_token[a_off_s + r]   phase 1, routed expert (gathered token rows of x)
//   a_off_s + r              phase 1, shared expert (x rows in token order)
//   o_off_s + r              phase 2 (hbuf rows of the segment)
struct GemmArgs {
  const void* A;         // phase 1: x [T, d]; phase 2: hbuf [R, h]
  int a_rows;            // rows of A (the range of its buffer descriptor)
  const int32_t* row_token;  // phase 1: token of each expert-sorted row; phase 2: nullptr
  int a_by_o_off;        // phase 2: the A row offset of a segment is its output row offset
  const void* W;         // [nseg][N][K]
  const void* bias;      // [nseg][N], or nullptr (no bias)
  void* C;               // [rows][N]
  const int32_t* seg;    // segment table
  int nseg, E, N, K;
  float* part;           // fp32 partial tiles of the split tail (part_cap tiles of BM x 256)
  int part_cap;
  int packed;            // W in the tile-packed layout (bf16 MFMA path only)
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

// activation of the first Linear: none (phase 2), GELU or SiLU
constexpr int kActNone = 0, kActGelu = 1, kActSilu = 2;

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

// SiLU(v) = v / (1 + e^-v), IEEE division (SIMT path).  e^-v overflows to
// +inf for v < -88 and the quotient is then -0, the limit.
__device__ __forceinline__ float silu_exact(float v) { return v / (1.0f + expf(-v)); }

template <int ACT>
__device__ __forceinline__ float act_fast(float v) {
  if constexpr (ACT == kActGelu) return gelu_fast(v);
  else if constexpr (ACT == kActSilu) return silu_fast(v);
  else return v;
}

template <int ACT>
__device__ __forceinline__ float act_exact(float v) {
  if constexpr (ACT == kActGelu) return gelu_erf(v);
  else if constexpr (ACT == kActSilu) return silu_exact(v);
  else return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
// two floats -> two bfloat16 (round to nearest even) packed low/high
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// segment s containing global M-tile mt: tile_start[s] <= mt < tile_start[s+1]
// -------------------------------------------------------------- MFMA path --
constexpr int kBN = 256, kBK = 64;
constexpr int kCh = kBK / 8;                   // 16-byte chunks per tile row

// LDS layout of a tile row of 64 bf16 (8 chunks of 16 bytes): logical chunk c
// of row r is stored at chunk c ^ (r & 7) ^ ((r >> 3) & 1).  Fragment reads
// (16x16x32: lane l holds row l % 16 of a block, 8 consecutive k) assign the
// K chunks to lane quarters as chunk 2 (l / 16) + slice: slice 0 takes chunks
// {0, 2, 4, 6}, slice 1 {1, 3, 5, 7}.  Measured with an LDS probe on gfx950,
// that ds_read_b128 pattern has no bank conflicts under this swizzle, while
// the natural order (quarter q reading chunk 4 slice + q) costs 4 conflict
// cycles per read under any XOR swizzle tried and 12 without one.  A and B
// use the same assignment, so each MFMA still contracts matching k of A and
// B; only which 32 k share an MFMA changes.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

// ------------------------------------------------------------ MFMA path --
// BM x 256 x 64 tiles, BM in {128, 160, 256}; 4 waves (one per SIMD) in
// a 2 x 2 grid, wave tile (BM / 2) x 128 built from the 16x16x32 bf16 MFMA:
// (BM / 32) x 8 blocks of 4 float accumulators per lane (up to 256, held in
// the accumulation registers).  The 16x16x32 form moves half the accumulator
// register traffic per FLOP of the 32x32x16 form; on this part, whose clock
// drops under full MFMA load, energy per FLOP sets the speed.
//
// Operands reach LDS by direct loads (buffer_load ... lds: 64 lanes x 16
// bytes at a wave-uniform LDS address) into an NS-slot ring of 64-deep
// stages ((BM + 256) rows x 128 bytes).  A K step works on two 32-deep
// slices of its stage, in a fixed issue order (every MFMA followed by at most
// one LDS fragment read and one direct load):
//   slice 0: MFMAs; read slice 1 of stage t
//   slice 1: wait for stage t+1 and the barrier that publishes it; stage t is
//            then in registers in every wave, so its slot is refilled with
//            stage t+NS; MFMAs; read slice 0 of stage t+1 (early in the
//            slice); direct loads of stage t+NS (spread over the slice)
// so fragment reads have a slice of MFMAs to land and (NS - 1) stages of
// loads stay in flight.  NS = 3 for BM <= 160 (weight streaming: ~100 KB per
// CU in flight).  At BM = 256 two 64 KB stages would leave one in flight;
// instead LDS holds five 32 KB operand units (A_t, B_t, A_t+1, ...: 160 KB),
// the barrier of step t frees stage t's two units for B_t+2 and A_t+3, and
// about one and a half stages stay in flight.  The LDS address of a direct
// load (M0) is scalar arithmetic on a per-wave offset taken once.
//
// The tile height is chosen per problem so that an expert's rows usually
// fill whole tiles: every M tile of an expert re-streams that expert's
// weight panel, so rows spread over fewer, fuller tiles mean fewer weight bytes.
//
// Epilogue: the MFMA takes the B fragment first, so each block is
// accumulated transposed: lane l holds output row 16 i + l % 16 of the wave
// tile and the four consecutive columns 16 j + 4 (l / 16) + 0..3; the bias is
// the accumulators' starting value, then (phase 1) the activation in float32,
// rounded once to bf16, one 8-byte store.
template <int ACT, int BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_mfma_kernel(GemmArgs g) {
  constexpr int NS = BM <= 160 ? 3 : 2;
  constexpr bool kExpertMajor = BM <= 160;     // weight streaming: expert-major tile order
  constexpr int MB = BM / 32;                  // 16-row blocks per wave
  constexpr int NR = MB + 8;                   // fragment reads per slice = direct loads per stage, per wave
  constexpr int MF = MB * 8;                   // MFMAs per slice
  constexpr int LS = MF / NR;                  // direct loads go one every LS MFMAs
  constexpr int kStage = (BM + kBN) * kCh;     // u32x4 per LDS stage
  static_assert(MF >= 2 * NR, "slice too short for its reads and loads");
  // BM = 256: a ring of five 256-row operand units instead of whole stages
  constexpr bool kUnits = BM == 256;
  constexpr int kUnit = 256 * kCh;             // u32x4 per operand unit
  __shared__ u32x4 lds[kUnits ? 5 * kUnit : NS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, so the LDS addresses of the direct loads (M0) are scalar arithmetic
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = uniform(st.tile_start[g.nseg]);
  const int ntn = g.N / kBN;
  const int total = total_mt * ntn;
  const int nk = g.K / kBK;                    // >= 4: K is a multiple of 256 on this path
  const uint32_t row_bytes = static_cast<uint32_t>(g.K) * 2u;

  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  const uint16_t* Wb = static_cast<const uint16_t*>(g.W);
  const uint16_t* Bias = static_cast<const uint16_t*>(g.bias);
  uint16_t* C = static_cast<uint16_t*>(g.C);

  // direct loads: wave w's load i fills LDS rows 32 i + 8 w + lane / 8 of its
  // operand at physical chunk lane % 8, fetching the logical chunk that lands there
  const int dr_row = 8 * wave + (lane >> 3);
  const int dr_ch = swz(dr_row, lane & 7);
  const int rd_row = lane & 15;
  const int wofs = uniform(8 * wave * kCh);    // this wave's first LDS row of a direct load

  const TailPlan tp = tail_plan(total, gridDim.x, nk, g.part_cap);
  const int items = tp.full + tp.tail * tp.S;

  for (int it = 0;; ++it) {
    const int w = it * gridDim.x + xcd * per_xcd + slot;
    if (w >= items) break;
    // work item w: a whole tile (w < full), or piece p of tail tile full + idx / S
    int L = w, k0 = 0, kn = nk, piece = -1;
    if (w >= tp.full) {
      piece = w - tp.full;
      const int p = piece % tp.S;
      L = tp.full + piece / tp.S;
      k0 = p * nk / tp.S;
      kn = (p + 1) * nk / tp.S - k0;           // >= 4
    }
    int mt, nt, s;
    if constexpr (kExpertMajor) {
      s = uniform(tile_of_expert(L, st.tile_start, g.nseg, ntn, mt, nt));
    } else {
      tile_of(L, total_mt, ntn, mt, nt);
      s = uniform(find_segment(st.tile_start, g.nseg, mt));
    }
    const int rows = uniform(st.rows[s]);
    const int m0 = (mt - uniform(st.tile_start[s])) * BM;
    const int a_off = uniform(g.a_by_o_off ? st.o_off[s] : st.a_off[s]);
    const int o_off = uniform(st.o_off[s]);
    const bool gather = g.row_token != nullptr && s < g.E;
    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(g.A, static_cast<uint32_t>(g.a_rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        make_rsrc(Wb + static_cast<size_t>(s) * g.N * g.K, static_cast<uint32_t>(g.N) * row_bytes);
    const int n0 = nt * kBN;
    const uint32_t step32 = 32u * row_bytes;
    // A: the lane's row of direct load q, looked up once per tile; rows past
    // the segment get an offset past the end of A (the range check covers
    // voffset + soffset: they read zero and touch no memory)
    // (a vector type: hipcc's host pass omits this kernel's launch stub when a
    // plain scalar array is captured by the load lambda below)
    u32x8 va = {};
#pragma unroll
    for (int q = 0; q < MB; ++q) {
      const int r = m0 + 32 * q + dr_row;
      const int arow = r < rows ? (gather ? g.row_token[a_off + r] : a_off + r) : -1;
      va[q] = arow >= 0 ? static_cast<uint32_t>(arow) * row_bytes + dr_ch * 16 : 0x80000000u;
    }
    // B: row-major W, the lane's row and chunk; or, packed, 256-row x 64-column
    // blocks of 32 KB each in LDS order, so a direct load is one linear 1 KB
    // (load q of a wave at (4 (q - MB) + wave) KB of its stage's block)
    const uint32_t vb = g.packed ? static_cast<uint32_t>(n0) * row_bytes + static_cast<uint32_t>(wave * 1024 + lane * 16)
                                 : static_cast<uint32_t>(n0 + dr_row) * row_bytes + dr_ch * 16;
    const uint32_t b_qs = g.packed ? 4096u : step32;               // bytes between a wave's B loads of a stage
    const uint32_t b_ks = g.packed ? 32768u : static_cast<uint32_t>(kBK * 2);   // bytes per K step

    // A whole tile's accumulators start at the bias of their column (the
    // epilogue then has no bias to add); the pieces of a split tile start at
    // zero and the fix-up adds the bias once.  The MFMA takes the B fragment
    // first, so lane l's four accumulators of block j hold columns
    // 16 j + 4 (l / 16) + 0..3 of the wave tile.
    const int cbase = n0 + wn * 128 + 4 * (lane >> 4);
    floatx4 bias0[8];
    {
      const uint16_t* brow = Bias + static_cast<size_t>(s) * g.N + cbase;
      const bool with_bias = Bias != nullptr && piece < 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint2 b = with_bias ? *reinterpret_cast<const uint2*>(brow + 16 * j) : make_uint2(0u, 0u);
        bias0[j] = floatx4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                           __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u)};
      }
    }
    floatx4 acc[MB][8];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = bias0[j];

    // fragment q of 32-deep slice sl of a stage whose A rows start at LDS
    // offset ao and B rows at bo: q < MB -> A block q, else B block q - MB;
    // slice sl of every stage lives in fragment buffer sl
    bf16x8 fa[2][MB], fb[2][8];
    auto frag1 = [&](int ao, int bo, int sl, int q) {
      const int ch = swz(rd_row, 2 * (lane >> 4) + sl);
      if (q < MB)
        fa[sl][q] = __builtin_bit_cast(bf16x8, lds[ao + (wm * (BM / 2) + q * 16 + rd_row) * kCh + ch]);
      else
        fb[sl][q - MB] = __builtin_bit_cast(bf16x8, lds[bo + (wn * 128 + (q - MB) * 16 + rd_row) * kCh + ch]);
    };
    // direct load q of stage k (K step k0 + k): q < MB -> A rows 32 q + .. at
    // offset ao, else B rows 32 (q - MB) + .. at offset bo
    auto issue1 = [&](int ao, int bo, int k, int q) {
      const uint32_t kbytes = static_cast<uint32_t>((k0 + k) * kBK * 2);
      const uint32_t bk = static_cast<uint32_t>(k0 + k) * b_ks;
      if (q < MB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rsrc, (__attribute__((address_space(3))) void*)(lds + ao + wofs + 32 * q * kCh), 16, va[q], kbytes, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb_rsrc, (__attribute__((address_space(3))) void*)(lds + bo + wofs + 32 * (q - MB) * kCh), 16, vb,
            static_cast<uint32_t>(q - MB) * b_qs + bk, 0, 0);
    };
    auto slot_a = [&](int rs) { return rs * kStage; };
    auto slot_b = [&](int rs) { return rs * kStage + BM * kCh; };

    // Stage ring (BM <= 160): cur = ring slot of stage t (t % NS); stage t+1
    // sits in the next slot and stage t+NS refills slot cur.  The last NS
    // steps are peeled so every flag is a compile-time constant in the
    // unrolled body.  pend: stage t+2's loads may be in flight at the wait
    // for stage t+1.
    auto kstep = [&](int t, int cur, bool refill, bool next, bool pend) {
      const int nxt = cur + 1 == NS ? 0 : cur + 1;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
        for (int q = 0; q < MF; ++q) {
          if (sl == 1 && q == 0 && next) {
            // stage t+1 landed (stage t+2's loads, if any, may stay in flight)
            if (pend) __builtin_amdgcn_s_waitcnt(vm_wait_imm(NR));
            else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            lds_barrier();
          }
          const int i = q >> 3, j = q & 7;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[sl][j], fa[sl][i], acc[i][j], 0, 0, 0);
          if (sl == 0 && (q & 1) == 0 && (q >> 1) < NR) frag1(slot_a(cur), slot_b(cur), 1, q >> 1);
          if (sl == 1 && (q & 1) == 0 && (q >> 1) < NR && next) frag1(slot_a(nxt), slot_b(nxt), 0, q >> 1);
          if (sl == 1 && (q % LS) == LS - 1 && (q / LS) < NR && refill)
            issue1(slot_a(cur), slot_b(cur), t + NS, q / LS);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // Unit ring (BM = 256): five 32 KB units hold operand panels in the order
    // A_0 B_0 A_1 B_1 ...; A_t sits in unit 2t mod 5 (ua) and B_t in unit
    // 2t+1 mod 5.  During step t, stage t is being read, stage t+1 has landed
    // or is landing, and the fifth unit (ua + 4: B_{t-1}'s, freed at the
    // previous barrier) takes A_{t+2} in slice 0; the barrier of step t frees
    // stage t's units and B_{t+2} goes into unit ua in slice 1.  So about one
    // and a half stages stay in flight where whole 64 KB stages would leave
    // one, and the direct loads are spread over both slices (8 a slice at
    // BM = 256) rather than 16 in one: the address FIFO in front of the
    // texture unit then rarely fills and holds up the wave's MFMA issue.
    // Loads are issued in panel order, so the wait for stage t+1 leaves only
    // A_{t+2}'s MB loads a wave outstanding.
    constexpr int LSU = 4;                     // MFMAs between direct loads in a slice
    static_assert(!kUnits || (8 * LSU <= MF && MB * LSU <= MF), "slice too short for its loads");
    auto kstep_u = [&](int t, int ua, bool refill, bool next) {
      const int ub = ua == 4 ? 0 : ua + 1;
      const int na = ua >= 3 ? ua - 3 : ua + 2, nb = ub >= 3 ? ub - 3 : ub + 2;
      const int uf = ua == 0 ? 4 : ua - 1;     // the free unit
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
        for (int q = 0; q < MF; ++q) {
          if (sl == 1 && q == 0 && next) {
            if (refill) __builtin_amdgcn_s_waitcnt(vm_wait_imm(MB));
            else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            lds_barrier();
          }
          const int i = q >> 3, j = q & 7;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[sl][j], fa[sl][i], acc[i][j], 0, 0, 0);
          if (sl == 0 && (q & 1) == 0 && (q >> 1) < NR) frag1(ua * kUnit, ub * kUnit, 1, q >> 1);
          if (sl == 1 && (q & 1) == 0 && (q >> 1) < NR && next) frag1(na * kUnit, nb * kUnit, 0, q >> 1);
          if (refill && (q % LSU) == LSU - 1) {
            if (sl == 0 && q / LSU < MB) issue1(uf * kUnit, 0, t + 2, q / LSU);
            if (sl == 1 && q / LSU < 8) issue1(0, ua * kUnit, t + 2, MB + q / LSU);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    if constexpr (kUnits) {
      // prologue: A_0 B_0 A_1 B_1 in units 0..3, stage 0 published, its slice 0 read
#pragma unroll
      for (int q = 0; q < NR; ++q) issue1(0, kUnit, 0, q);
#pragma unroll
      for (int q = 0; q < NR; ++q) issue1(2 * kUnit, 3 * kUnit, 1, q);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(NR));
      lds_barrier();
#pragma unroll
      for (int q = 0; q < NR; ++q) frag1(0, kUnit, 0, q);
    } else {
      // prologue: stages 0 .. NS-1 in flight, stage 0 published, its slice 0 read
#pragma unroll
      for (int k = 0; k < NS; ++k)
#pragma unroll
        for (int q = 0; q < NR; ++q) issue1(slot_a(k), slot_b(k), k, q);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm((NS - 1) * NR));
      lds_barrier();
#pragma unroll
      for (int q = 0; q < NR; ++q) frag1(slot_a(0), slot_b(0), 0, q);
    }
    // Shorter tiles leave accumulation registers free, and the register
    // allocator then shuttles accumulators between register files inside the
    // loop.  Occupying the rest of that file with values pinned there across
    // the loop keeps the accumulators in place.
    constexpr int kPad = (256 - MB * 32) / 4;
    floatx4 pin[kPad > 0 ? kPad : 1];
    if constexpr (kPad > 0) {
#pragma unroll
      for (int k = 0; k < kPad; ++k) {
        pin[k] = floatx4{0.f, 0.f, 0.f, 0.f};
        __asm__ volatile("" : "+a"(pin[k]));
      }
    }
    if constexpr (kUnits) {
      // (the unit is derived from t in each step: carried through the loop
      // instead, it led the register allocator to rotate the accumulators
      // between registers on every step)
      int t = 0;
      for (; t + 2 < kn; ++t) kstep_u(t, (2 * t) % 5, true, true);
      kstep_u(t, (2 * t) % 5, false, true);
      kstep_u(t + 1, (2 * t + 2) % 5, false, false);
    } else {
      int t = 0, cur = 0;
      for (; t + NS < kn; ++t) {
        kstep(t, cur, true, true, NS == 3);
        cur = cur + 1 == NS ? 0 : cur + 1;
      }
      if constexpr (NS == 3) {
        // stage t+2 = kn-1 was issued a step ago and may still be in flight
        kstep(t++, cur, false, true, true);
        cur = cur + 1 == NS ? 0 : cur + 1;
      }
      kstep(t, cur, false, true, false);
      kstep(t + 1, cur + 1 == NS ? 0 : cur + 1, false, false, false);
    }
    if constexpr (kPad > 0) {
#pragma unroll
      for (int k = 0; k < kPad; ++k) __asm__ volatile("" ::"a"(pin[k]));
    }
    // the next tile's first loads reuse the ring: every wave is done reading
    lds_barrier();

    // Epilogue.  A piece of a tail tile stores its float32 partial tile
    // (row-major BM x 256, buffer stores: one lane offset plus scalar and
    // immediate offsets); a whole tile (its bias already in the accumulators)
    // applies the activation (phase 1) and stores bf16.  The choice is made per
    // 16-row block so only that block's accumulators are live in vector
    // registers at a time.
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.part, static_cast<uint32_t>(g.part_cap) * BM * kBN * 4u);
    const uint32_t pv = (static_cast<uint32_t>(wm * (BM / 2) + (lane & 15)) * kBN + wn * 128 + 4 * (lane >> 4)) * 4u;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int rl = m0 + wm * (BM / 2) + i * 16 + (lane & 15);
      if (piece >= 0) {
        const uint32_t ps = (static_cast<uint32_t>(piece) * BM + i * 16) * kBN * 4u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), pr, pv + 64 * j, ps, 0);
      } else if (rl < rows) {
        uint16_t* crow = C + static_cast<size_t>(o_off + rl) * g.N + cbase;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v0 = act_fast<ACT>(acc[i][j][0]);
          const float v1 = act_fast<ACT>(acc[i][j][1]);
          const float v2 = act_fast<ACT>(acc[i][j][2]);
          const float v3 = act_fast<ACT>(acc[i][j][3]);
          *reinterpret_cast<uint2*>(crow + 16 * j) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
      }
    }
  }
}

// Fix-up of the split tail, in 16-row chunks of the tail tiles strided over
// the launch's workgroups (P is the GEMM's grid, which fixed the tail plan).
// Each thread owns four consecutive columns of four rows; the S partial tiles
// are summed in piece order, then bias, the activation (phase 1) and one bf16
// rounding, as in the GEMM epilogue.
template <int ACT, int BM>
__global__ __launch_bounds__(256) void gemm_tail_fixup_kernel(GemmArgs g, int P) {
  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = st.tile_start[g.nseg];
  const int ntn = g.N / kBN;
  const TailPlan tp = tail_plan(total_mt * ntn, P, g.K / kBK, g.part_cap);
  if (tp.tail == 0) return;
  constexpr int kChunks = BM / 16;
  const int c = 4 * (threadIdx.x & 63);
  uint16_t* C = static_cast<uint16_t*>(g.C);
  for (int w = blockIdx.x; w < tp.tail * kChunks; w += gridDim.x) {
    const int tt = w / kChunks, r0 = (w % kChunks) * 16;
    int mt, nt, s;
    if constexpr (BM <= 160) {   // the GEMM kernel's tile order
      s = tile_of_expert(tp.full + tt, st.tile_start, g.nseg, ntn, mt, nt);
    } else {
      tile_of(tp.full + tt, total_mt, ntn, mt, nt);
      s = find_segment(st.tile_start, g.nseg, mt);
    }
    const int rows = st.rows[s];
    const int m0 = (mt - st.tile_start[s]) * BM;
    const int o_off = st.o_off[s];
    const int n = nt * kBN + c;
    const uint2 b = g.bias ? *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.bias) +
                                                             static_cast<size_t>(s) * g.N + n)
                           : make_uint2(0u, 0u);
    const float b0 = __uint_as_float(b.x << 16), b1 = __uint_as_float(b.x & 0xffff0000u);
    const float b2 = __uint_as_float(b.y << 16), b3 = __uint_as_float(b.y & 0xffff0000u);
    const float* part = g.part + static_cast<size_t>(tt) * tp.S * BM * kBN;
    // every partial of the thread's four rows is loaded before any is added
    // (up to kFixS pieces at a time), then summed in piece order
    constexpr int kFixS = 8;
    floatx4 a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < tp.S; p0 += kFixS) {
      floatx4 v[4][kFixS];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // rows past the segment and pieces past S read a row or piece that is
        // not used: unconditional loads are all in flight together
        const int rr = min(r0 + (threadIdx.x >> 6) + 4 * k, rows - 1 - m0);
#pragma unroll
        for (int p = 0; p < kFixS; ++p)
          v[k][p] = *reinterpret_cast<const floatx4*>(part + (static_cast<size_t>(min(p0 + p, tp.S - 1)) * BM + rr) * kBN + c);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < kFixS; ++p)
          if (p0 + p < tp.S) a[k] = p0 + p == 0 ? v[k][p] : a[k] + v[k][p];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = r0 + (threadIdx.x >> 6) + 4 * k;
      if (m0 + rr >= rows) break;
      float v0 = a[k][0] + b0, v1 = a[k][1] + b1, v2 = a[k][2] + b2, v3 = a[k][3] + b3;
      v0 = act_fast<ACT>(v0);
      v1 = act_fast<ACT>(v1);
      v2 = act_fast<ACT>(v2);
      v3 = act_fast<ACT>(v3);
      *reinterpret_cast<uint2*>(C + static_cast<size_t>(o_off + m0 + rr) * g.N + n) =
          make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    }
  }
}

// ------------------------------------------------------ float32 MFMA path --
// float32 layers (any d, h: multiples of 8) on the float32 matrix cores
// (v_mfma_f32_16x16x4_f32: 2048 FLOP per instruction, 157.3 TFLOP/s for the
// part), float32 products and sums: the same arithmetic class as the float32
// SIMT loop it replaces.  BM x 128 tiles, BM in {32, 64} chosen per problem
// (the float32 workloads have short experts: ~64 rows at the switch-shaped
// layer), K slabs of 32 staged through LDS (rows of 32 k padded to 36 floats,
// 16-byte stores and fragment reads) with the next two slabs' loads held in
// registers while the current one is multiplied.  One workgroup per tile
// (grid = M tiles x N tiles; the M tiles past the segment table's count exit),
// several resident per CU.  4 waves in a (BM / 32) x (4 / (BM / 32)) grid,
// each 32 rows x (128 / wave columns) of 16x16 blocks.  The MFMA takes the B
// fragment first, so a lane ends with one output row and four consecutive
// columns: bias, activation (library erff / expf, as the SIMT path) and one
// 16-byte store.  Rows past a segment, columns past N and k past K read zero.
constexpr int kFBN = 128, kFBK = 32;

template <int ACT, int BM>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(GemmArgs g) {
  constexpr int WM = BM / 32, WN = 4 / WM;      // wave grid
  constexpr int WTN = kFBN / WN;                // wave tile columns
  constexpr int NBk = WTN / 16;                 // 16-column blocks per wave
  constexpr int LDP = kFBK + 4;                 // LDS row pitch (floats): rows of 32 k, 16-byte aligned
  constexpr int AV = BM * kFBK / 4 / 256;       // float4 loads per thread per slab: A
  constexpr int BV = kFBN * kFBK / 4 / 256;     //                                   B
  __shared__ float4 sA[2][BM][LDP / 4];
  __shared__ float4 sB[2][kFBN][LDP / 4];

  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = st.tile_start[g.nseg];
  const int mt = blockIdx.x;
  if (mt >= total_mt) return;
  const int s = find_segment(st.tile_start, g.nseg, mt);
  const int rows = st.rows[s];
  const int m0 = (mt - st.tile_start[s]) * BM;
  const int n0 = blockIdx.y * kFBN;
  const int a_off = g.a_by_o_off ? st.o_off[s] : st.a_off[s];
  const bool gather = g.row_token != nullptr && s < g.E;
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.W) + static_cast<size_t>(s) * g.N * g.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // global -> register loads: thread tid takes float4 (tid + 256 v) of the
  // slab: row (tid + 256 v) / 8, k quad (tid % 8) (8 float4 per 32-deep row)
  const float* arow[AV];
  bool aok[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int r = (tid + 256 * v) >> 3;
    const int gm = m0 + r;
    aok[v] = gm < rows;
    const int ar = aok[v] ? (gather ? g.row_token[a_off + gm] : a_off + gm) : 0;
    arow[v] = A + static_cast<size_t>(ar) * g.K;
  }
  const int kq = tid & 7;
  auto load = [&](int k0, float4 (&ra)[AV], float4 (&rb)[BV]) {
    const int kk = k0 + 4 * kq;
    const bool k_ok = kk < g.K;    // K is a multiple of 8, so a quad is whole or absent
#pragma unroll
    for (int v = 0; v < AV; ++v)
      ra[v] = aok[v] && k_ok ? *reinterpret_cast<const float4*>(arow[v] + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int n = n0 + ((tid + 256 * v) >> 3);
      rb[v] = n < g.N && k_ok ? *reinterpret_cast<const float4*>(B + static_cast<size_t>(n) * g.K + kk)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int buf, const float4 (&ra)[AV], const float4 (&rb)[BV]) {
#pragma unroll
    for (int v = 0; v < AV; ++v) sA[buf][(tid + 256 * v) >> 3][kq] = ra[v];
#pragma unroll
    for (int v = 0; v < BV; ++v) sB[buf][(tid + 256 * v) >> 3][kq] = rb[v];
  };

  floatx4 acc[2][NBk];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NBk; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Fragments: lane (r = lane % 16, q = lane / 16) reads k 16 h + 4 q .. + 3 of
  // its row as one float4, and MFMA c of the group contracts component c: the
  // four MFMAs cover k 16 h + {c, 4 + c, 8 + c, 12 + c}, all 16 k of the group,
  // with A and B paired on the same k.
  const int fr = lane & 15, fq = lane >> 4;
  const int nslab = (g.K + kFBK - 1) / kFBK;
  auto compute = [&](int cur) {
#pragma unroll
    for (int h = 0; h < kFBK / 16; ++h) {
      float4 af[2], bf[NBk];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = sA[cur][32 * wm + 16 * i + fr][4 * h + fq];
#pragma unroll
      for (int j = 0; j < NBk; ++j) bf[j] = sB[cur][WTN * wn + 16 * j + fr][4 * h + fq];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NBk; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j].x, af[i].x, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j].y, af[i].y, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j].z, af[i].z, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j].w, af[i].w, acc[i][j], 0, 0, 0);
        }
    }
  };
  // Two slabs of loads ahead: slab s sits in LDS buffer s % 2 when it is
  // multiplied, slab s + 1 in the register set of its parity, and slab s + 2
  // is issued into the register set slab s has left.  A buffer is refilled
  // only after the barrier that follows its last readers.
  float4 ra0[AV], rb0[BV], ra1[AV], rb1[BV];
  load(0, ra0, rb0);
  store(0, ra0, rb0);
  if (nslab > 1) load(kFBK, ra1, rb1);
  __syncthreads();
  for (int sl = 0; sl < nslab; sl += 2) {
    if (sl + 2 < nslab) load((sl + 2) * kFBK, ra0, rb0);
    compute(0);
    if (sl + 1 >= nslab) break;
    store(1, ra1, rb1);
    __syncthreads();
    if (sl + 3 < nslab) load((sl + 3) * kFBK, ra1, rb1);
    compute(1);
    if (sl + 2 >= nslab) break;
    store(0, ra0, rb0);
    __syncthreads();
  }

  // lane holds row 32 wm + 16 i + lane % 16 of the tile, columns WTN wn + 16 j + 4 (lane / 16) + 0..3
  const float* Bias = static_cast<const float*>(g.bias);
  float* C = static_cast<float*>(g.C);
  const int o_off = st.o_off[s];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rl = m0 + 32 * wm + 16 * i + fr;
    if (rl >= rows) continue;
    float* crow = C + static_cast<size_t>(o_off + rl) * g.N;
#pragma unroll
    for (int j = 0; j < NBk; ++j) {
      const int n = n0 + WTN * wn + 16 * j + 4 * fq;
      if (n >= g.N) continue;   // N is a multiple of 8: a quad is whole or absent
      float4 b = Bias ? *reinterpret_cast<const float4*>(Bias + static_cast<size_t>(s) * g.N + n)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 o;
      o.x = act_exact<ACT>(acc[i][j][0] + b.x);
      o.y = act_exact<ACT>(acc[i][j][1] + b.y);
      o.z = act_exact<ACT>(acc[i][j][2] + b.z);
      o.w = act_exact<ACT>(acc[i][j][3] + b.w);
      *reinterpret_cast<float4*>(crow + n) = o;
    }
  }
}

// ------------------------------------------------------------ SIMT path --
constexpr int kSB = 64, kSK = 16;

__device__ __forceinline__ float ld_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st_out(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename TIn, int ACT>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmArgs g, int max_mt) {
  __shared__ float sA[kSK][kSB + 1];
  __shared__ float sB[kSK][kSB + 1];
  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = st.tile_start[g.nseg];
  const int mt = blockIdx.x;
  if (mt >= total_mt) return;
  (void)max_mt;
  const int s = find_segment(st.tile_start, g.nseg, mt);
  const int rows = st.rows[s];
  const int m0 = (mt - st.tile_start[s]) * kSB;
  const int n0 = blockIdx.y * kSB;
  const int a_off = g.a_by_o_off ? st.o_off[s] : st.a_off[s];
  const bool gather = g.row_token != nullptr && s < g.E;
  const TIn* A = static_cast<const TIn*>(g.A);
  const TIn* B = static_cast<const TIn*>(g.W) + static_cast<size_t>(s) * g.N * g.K;
  const TIn* Bias = g.bias ? static_cast<const TIn*>(g.bias) + static_cast<size_t>(s) * g.N : nullptr;
  TIn* C = static_cast<TIn*>(g.C);

  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += kSK) {
    for (int i = threadIdx.x; i < kSB * kSK; i += 256) {
      const int rr = i / kSK, kk = i % kSK;
      const int gm_ = m0 + rr, gk = k0 + kk, gn = n0 + rr;
      const int arow = gm_ < rows ? (gather ? g.row_token[a_off + gm_] : a_off + gm_) : 0;
      sA[kk][rr] = (gm_ < rows && gk < g.K) ? ld_f32(A, static_cast<size_t>(arow) * g.K + gk) : 0.f;
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
      float v = acc[i][j] + (Bias ? ld_f32(Bias, col) : 0.f);
      v = act_exact<ACT>(v);
      st_out(C, static_cast<size_t>(o_off + rl) * g.N + col, v);
    }
  }
}

// Tile-packed weights (layout in include/moe.h): block b = (m, n / 256,
// kk / 64) is the LDS image of one 256-row x 64-column B stage, so the GEMM's
// direct loads of a stage read 32 KB of contiguous memory.  One workgroup per
// block; thread t moves 16-byte chunks t, t + 256, ... (row = chunk / 8,
// position = chunk % 8), reading the logical chunk that the GEMM's fragment
// reads expect at that position.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wp,
                                                           int N, int K) {
  const int nkb = K / 64, nnb = N / 256;
  const int b = blockIdx.x;
  const int kb = b % nkb, nb = (b / nkb) % nnb, m = b / (nkb * nnb);
  const uint16_t* src = W + (static_cast<size_t>(m) * N + static_cast<size_t>(nb) * 256) * K + kb * 64;
  uint16_t* dst = Wp + static_cast<size_t>(b) * 16384;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = threadIdx.x + 256 * i;
    const int r = ch >> 3, pos = ch & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r) * K + swz(r, pos) * 8);
    *reinterpret_cast<u32x4*>(dst + r * 64 + pos * 8) = v;
  }
}

}  // namespace

hipError_t launch_pack_weights(const void* W, int n_mat, int N, int K, void* Wp, hipStream_t st) {
  const long long blocks = static_cast<long long>(n_mat) * (N / 256) * (K / 64);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Wp), N, K);
  return hipGetLastError();
}

bool gemm_fast_path(const Problem& p) {
  if (p.dtype != MOE_BF16 || p.h % kBN != 0 || p.d % kBN != 0 || p.d % kBK != 0 || p.h % kBK != 0) return false;
  // buffer offsets are 32-bit: every operand region must stay below 2 GiB
  const long long rows = static_cast<long long>(p.A) + static_cast<long long>(p.S) * p.T + 256;
  const long long widest = p.d > p.h ? p.d : p.h;
  return rows * widest * 2 < (1LL << 31) && static_cast<long long>(p.h) * p.d * 2 < (1LL << 31);
}

// Tile height of the MFMA path.  Experts averaging >= 512 rows: 256 (the
// compute-bound case).  Otherwise the height in {128, 160, 256} that
// covers the expected rows of an expert with the fewest padded rows: the
// capacity when it binds (an expert then holds exactly that many rows when
// full; under expert choice every expert holds exactly C), else 1.25 x the
// mean rows per expert as headroom for uneven routing; ties go to the taller
// tile, which streams each weight panel for more rows.
int gemm_m_tile(const Problem& p) {
  if (p.dtype == MOE_F32) {
    // float32 matrix-core path: 32 or 64 rows, whichever pads the expected
    // rows of an expert least (ties to 64)
    const long long mean = (static_cast<long long>(p.A) + p.E - 1) / p.E;
    const long long want = p.cap <= mean ? p.cap : (mean * 5 + 3) / 4;
    return (want + 31) / 32 * 32 < (want + 63) / 64 * 64 ? 32 : 64;
  }
  if (!gemm_fast_path(p)) return kSB;
  const long long mean = (static_cast<long long>(p.A) + p.E - 1) / p.E;
  if (mean >= 512 && p.cap >= 512) return 256;
  const long long want = p.cap <= mean ? p.cap : (mean * 5 + 3) / 4;
  int best = 256;
  long long best_pad = (want + 255) / 256 * 256;
  for (int bm : {160, 128}) {
    const long long pad = (want + bm - 1) / bm * bm;
    if (pad < best_pad) {
      best = bm;
      best_pad = pad;
    }
  }
  return best;
}

hipError_t launch_expert_ffn(const Problem& p, const void* x, const void* W1, const void* b1, const void* W2,
                             const void* b2, const Workspace& ws, int phase, hipStream_t st) {
  GemmArgs g;
  g.seg = ws.seg;
  g.nseg = p.E + p.S;
  g.E = p.E;
  if (phase == 1) {
    g.A = x;
    g.a_rows = p.T;
    g.row_token = ws.row_token;
    g.a_by_o_off = 0;
    g.W = W1;
    g.bias = b1;
    g.C = ws.hbuf;
    g.N = p.h;
    g.K = p.d;
  } else {
    g.A = ws.hbuf;
    g.a_rows = p.A + p.S * p.T;
    g.row_token = nullptr;
    g.a_by_o_off = 1;
    g.W = W2;
    g.bias = b2;
    g.C = ws.ybuf;
    g.N = p.d;
    g.K = p.h;
  }
  g.part = ws.part;
  g.part_cap = ws.part_cap;
  g.packed = p.packed_w ? 1 : 0;
  // the activation follows the first Linear only
  const int act = phase == 2 ? kActNone : (p.act == MOE_ACT_SILU ? kActSilu : kActGelu);
  if (gemm_fast_path(p)) {
    int grid = device_cu_count();
    grid = (grid + 7) / 8 * 8;
    const dim3 gd(grid), bd(256);
    // the fix-up runs right after the GEMM on the same stream; it returns at
    // once when the tail was not split.  Four workgroups a CU, so that a tail
    // of up to 4 P 16-row chunks is one chunk a workgroup (Mixtral-shaped
    // phase 2: 768 chunks; 18 -> 15 us against one workgroup a CU).
#define MOE_GEMM_LAUNCH(ACT_, BM_)                                                          \
  do {                                                                                      \
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<ACT_, BM_>), gd, bd, 0, st, g);               \
    hipLaunchKernelGGL((gemm_tail_fixup_kernel<ACT_, BM_>), dim3(4 * grid), bd, 0, st, g, grid); \
  } while (0)
#define MOE_GEMM_LAUNCH_BM(BM_)                                                             \
  do {                                                                                      \
    if (act == kActGelu) MOE_GEMM_LAUNCH(kActGelu, BM_);                                    \
    else if (act == kActSilu) MOE_GEMM_LAUNCH(kActSilu, BM_);                               \
    else MOE_GEMM_LAUNCH(kActNone, BM_);                                                    \
  } while (0)
    switch (p.gemm_bm) {
      case 128: MOE_GEMM_LAUNCH_BM(128); break;
      case 160: MOE_GEMM_LAUNCH_BM(160); break;
      default: MOE_GEMM_LAUNCH_BM(256); break;
    }
#undef MOE_GEMM_LAUNCH_BM
#undef MOE_GEMM_LAUNCH
  } else if (p.dtype == MOE_F32) {
    const int bm = p.gemm_bm;
    const long long max_mt = (static_cast<long long>(p.A) + bm - 1) / bm + p.E +
                             static_cast<long long>(p.S) * ((p.T + bm - 1) / bm);
    const dim3 grid(static_cast<unsigned>(max_mt), (g.N + kFBN - 1) / kFBN), block(256);
#define MOE_F32_LAUNCH(BM_)                                                                         \
  do {                                                                                              \
    if (act == kActGelu) hipLaunchKernelGGL((gemm_f32_mfma_kernel<kActGelu, BM_>), grid, block, 0, st, g); \
    else if (act == kActSilu) hipLaunchKernelGGL((gemm_f32_mfma_kernel<kActSilu, BM_>), grid, block, 0, st, g); \
    else hipLaunchKernelGGL((gemm_f32_mfma_kernel<kActNone, BM_>), grid, block, 0, st, g);          \
  } while (0)
    if (bm == 32) MOE_F32_LAUNCH(32);
    else MOE_F32_LAUNCH(64);
#undef MOE_F32_LAUNCH
  } else {
    // upper bound of M tiles: sum_e ceil(rows_e / 64) <= ceil(T k / 64) + E + S ceil(T / 64)
    const long long max_mt = (static_cast<long long>(p.A) + kSB - 1) / kSB + p.E +
                             static_cast<long long>(p.S) * ((p.T + kSB - 1) / kSB);
    dim3 grid(static_cast<unsigned>(max_mt), (g.N + kSB - 1) / kSB);
#define MOE_SIMT_LAUNCH(TIN_)                                                                               \
  do {                                                                                                      \
    if (act == kActGelu)                                                                                    \
      hipLaunchKernelGGL((gemm_simt_kernel<TIN_, kActGelu>), grid, dim3(256), 0, st, g, (int)max_mt);      \
    else if (act == kActSilu)                                                                               \
      hipLaunchKernelGGL((gemm_simt_kernel<TIN_, kActSilu>), grid, dim3(256), 0, st, g, (int)max_mt);      \
    else                                                                                                    \
      hipLaunchKernelGGL((gemm_simt_kernel<TIN_, kActNone>), grid, dim3(256), 0, st, g, (int)max_mt);      \
  } while (0)
    if (p.dtype == MOE_BF16) MOE_SIMT_LAUNCH(uint16_t);
    else MOE_SIMT_LAUNCH(float);
#undef MOE_SIMT_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace moe
