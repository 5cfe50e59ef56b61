// moe_mxfp8: the expert FFNs with MXFP8 operands (OCP microscaling: E4M3
// elements, one E8M0 power-of-two scale per 32 elements along the
// contracted dimension) on the gfx950 scaled matrix instruction.
//
// Pages: "AI-Research-SKILLs MoE 训练实战…全指南" §9.2 (serving with FP8
// quantization: vLLM's quantization="fp8", about 20-30% more throughput than
// 16-bit); the pages fix no encoding, so the OCP MX form is used, which is the
// FP8 form this part's scaled MFMA consumes directly.
//
// Formats.  An MX matrix [R, K] (K a multiple of 128) is uint8 E4M3 codes
// [R, K] row-major plus uint8 E8M0 scales [R, K / 32] row-major (scale of
// row r, elements 32 b .. 32 b + 31 is 2^(byte - 127)).  Quantizing a block:
// s = floor(log2 max|v|) - 8 (-127 for an all-zero block), element =
// v * 2^-s rounded to the nearest E4M3 value, ties to even, clamped to +-448.
//
//   mx_quantize_kernel   bf16 rows -> MX (x at run time; weights through the ABI)
//   gemm_mx_kernel       phase 1: H = act(xq W1q^T + b1), H written as MX
//                        phase 2: Y = Hq W2q^T + b2, bf16
//
// The scaled 16x16x128 MFMA (measured with probes on gfx950): lane l carries
// row l % 16 of each operand and, in bytes 0-15, K elements 16 (l / 16) ..
// +15, in bytes 16-31, K elements 64 + 16 (l / 16) .. +15; the scale of
// (row r, 32-element block b) comes from lane r + 16 b; the result of
// mfma(P, Q) puts P's rows at 4 (l / 16) + v and Q's rows at l % 16.  So a
// lane that reads 16-byte chunks l / 16 and l / 16 + 4 of a 128-byte K stage
// holds K in memory order, every MX block sits in one hardware block, and the
// lane's scale is that of its row and block l / 16.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.f;

// floor(log2 amax) - 8, clamped to [-127, 127]; -127 for amax == 0
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int s = ilogbf(amax) - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// 2^-s as a float for s in [-127, 126] (exact power of two)
__device__ __forceinline__ float mx_inv_scale(int s) { return __int_as_float((127 - s) << 23); }

// two floats (already scaled) -> two E4M3 codes (round to nearest even) in
// the low (HI = false) or high half of `old`; the clamp to +-448 first, since
// the conversion turns magnitudes from 480 up into NaN
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  i16x2 o = __builtin_bit_cast(i16x2, old);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, o);
}

// ------------------------------------------------------------- quantize --
// One thread per 32-element block of a bf16 row: 64 bytes in, 32 codes and one
// scale byte out.
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ src, size_t nblocks,
                                                          int blocks_per_row, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  for (size_t b = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; b < nblocks;
       b += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const u32x4* in = reinterpret_cast<const u32x4*>(src + b * 32);
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = in[i];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] & 0xffff0000u)));
      }
    const int s = mx_exponent(amax);
    const float inv = mx_inv_scale(s);
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // elements 8 i .. 8 i + 7 -> two code words
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = v[i][2 * h], w1 = v[i][2 * h + 1];
        uint32_t c = cvt2<false>(__uint_as_float(w0 << 16) * inv, __uint_as_float(w0 & 0xffff0000u) * inv, 0u);
        c = cvt2<true>(__uint_as_float(w1 << 16) * inv, __uint_as_float(w1 & 0xffff0000u) * inv, c);
        out[i / 2][(i % 2) * 2 + h] = c;
      }
    }
    u32x4* o = reinterpret_cast<u32x4*>(codes + b * 32);
    o[0] = out[0];
    o[1] = out[1];
    scales[b] = static_cast<uint8_t>(s + 127);
    (void)blocks_per_row;
  }
}

// ---------------------------------------------------------------- GEMM --
struct MxArgs {
  const uint8_t* A;        // phase 1: x codes [T, d]; phase 2: H codes [R, h]
  const uint8_t* As;       // their scales [rows, K / 32]
  int a_rows;
  const int32_t* row_token;
  int a_by_o_off;
  const uint8_t* W;        // [nseg][N][K] codes
  const uint8_t* Ws;       // [nseg][N][K / 32] scales
  const uint16_t* bias;    // [nseg][N] bf16, or nullptr
  void* C;                 // phase 1: H codes [R, N]; phase 2: Y bf16 [R, N]
  uint8_t* Cs;             // phase 1: H scales [R, N / 32]
  const int32_t* seg;
  int nseg, E, N, K;
  float* part;             // [part_cap][BM][256] float32 partial tiles of the split tail
  int part_cap;            // partial tiles the buffer holds (0: no split)
};

constexpr int kMxBN = 256, kMxBK = 128;     // tile columns, K elements (= bytes) per stage
constexpr int kMxCh = kMxBK / 16;           // 16-byte chunks per stage row

__device__ __forceinline__ int mx_swz(int row, int c) { return c ^ (row & 7); }

__device__ __forceinline__ void mx_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt 0 only
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// activation of the first Linear: 1 GELU(erf), 2 SiLU, 0 none (second Linear)
template <int ACT>
__device__ __forceinline__ float mx_act(float v) {
  if constexpr (ACT == 1) return gelu_fast(v);
  else if constexpr (ACT == 2) return silu_fast(v);
  else return v;
}

__device__ __forceinline__ uint32_t mx_pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  const floatx2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// BM x 256 tiles (BM 128, 192 or 256), 128-deep K stages in LDS rings of NA
// slots for the A rows and NB for the B (weight) rows, 4 waves in a 2 x 2 grid
// (wave tile BM/2 x 128 = (BM/32) x 8 blocks of the 16x16x128 MFMA).  Short
// tiles stream each expert's weights from HBM about once, so the B ring gets
// a third slot (two stages in flight) wherever it fits: NA = NB = 3 at
// BM = 128, NA = 2 and NB = 3 at BM = 192 (the A rows are shared by all N
// tiles of a row panel and mostly come from L2), 2 and 2 at BM = 256.
// Codes reach LDS by direct loads (rows of 128 bytes, 16-byte chunks XOR-
// swizzled by row).  Scales come SG stages at a time (4 SG bytes of a row,
// one row per lane; SG = 4, a quarter of the line requests of one load a
// stage, when rows of scales are a multiple of 16 bytes, else SG = 1) into a
// ring of their own (2 groups, or NB stages at SG = 1); a lane's scale operand
// is read straight from LDS as the byte of its row, stage and block.
//
// A fragment is 32 bytes a lane, so one stage's fragments (A and B) fill 128
// vector registers and cannot be double-buffered whole.  K step t runs its
// MFMAs in two halves (A rows 0 .. MB/2-1, then the rest), every MFMA followed
// by at most one fragment read and one direct load, in a fixed order:
//   half 0: MFMAs; read A rows 2 .. MB-1 of stage t
//   wait for stage t+1 and the barrier that publishes it; stage t is then in
//   registers in every wave, so its slots take A stage t+NA and B stage t+NB
//   half 1: MFMAs, B block outermost; read A rows 0, 1 of stage t+1, and its
//           B block j as soon as block j of stage t is done; direct loads: a
//           scale group (if one starts), A stage t+NA, B stage t+NB
// so the next stage's B fragments reuse the registers of this stage's, and
// arrive, with its first two A rows, while this stage's last rows multiply.
// LDS of one tile height: NA A code slots, NB B code slots, the scale slots,
// then 64 kSRow bytes where the skipped scale loads land
template <int BM, int SG>
struct MxGeom {
  static constexpr int NA = BM == 128 ? 3 : 2;            // A ring slots
  static constexpr int NB = BM == 256 ? 2 : 3;            // B ring slots
  static constexpr int kSRow = 4 * SG;                    // scale bytes of a row in one group
  static constexpr int kScaleSlot = (BM + kMxBN) * kSRow; // bytes of a scale group: A rows, then B rows
  static constexpr int NSS = SG == 1 ? NB : 2;            // scale ring slots
  static constexpr int kScaleBase = NA * BM * kMxCh + NB * kMxBN * kMxCh;   // u32x4 index of the scale slots
  static constexpr int kJunkBase = kScaleBase + NSS * kScaleSlot / 16;
  static constexpr int kWords = kJunkBase + 64 * kSRow / 16;                // u32x4 in all
};

// One work item: M tile mt (of segment s) x N tile nt over K steps k0 ..
// k0 + kn - 1; piece >= 0 marks a piece of a split tail tile, which leaves a
// float32 partial tile at rows PBM piece .. of the partial buffer.
template <int ACT, int BM, int SG, int PBM>
__device__ __forceinline__ void mx_tile(const MxArgs& g, u32x4* lds, const SegTableRO& st, int s, int mt, int nt,
                                        int k0, int kn, int piece) {
  using Geo = MxGeom<BM, SG>;
  constexpr bool kMxOut = ACT != 0;           // phase 1 writes H as MX
  constexpr int MB = BM / 32;                 // 16-row A blocks per wave
  constexpr int HM = MB / 2 * 8;              // MFMAs per half step
  constexpr int NR = MB + 8;                  // code loads per stage per wave (8 rows x 128 B each)
  constexpr int NA = Geo::NA, NB = Geo::NB, NSS = Geo::NSS;
  constexpr int kSRow = Geo::kSRow, kScaleSlot = Geo::kScaleSlot;
  constexpr int NF1 = MB - 2;                       // fragment reads in half 0
  static_assert(SG == 1 || SG == 4, "scale groups of 1 or 4 stages (4- or 16-byte direct loads)");
  static_assert(BM == 128 || BM == 192 || BM == 256, "tile heights 128, 192, 256 (an even number of 16-row blocks a wave)");
  static_assert(BM <= PBM, "partial tiles hold PBM rows");
  // a step that starts group G loads group G + kLook into the slot whose last
  // stage was read before the step's barrier: that of group G - 1 (SG = 4) or
  // of stage G itself (SG = 1: group G + NB goes with the B codes of stage G + NB)
  constexpr int kLook = SG == 1 ? NB : 1;
  static_assert(HM >= 2 * NF1 && HM >= NR + 2, "half step too short for its reads and loads");
  static_assert(NA >= 2 && NB >= 2, "ring depths");
  // the barrier of step t waits for stage t+1.  A step issues 2 scale loads,
  // MB A loads, 8 B loads; stage t+1's A rows went out with step t+1-NA and
  // its B rows with step t+1-NB, and only what followed the later of the two
  // may still be in flight: the 8 B loads of that step if it is the A rows
  // (NA < NB), and the min(NA, NB) - 2 steps after it.
  constexpr int kVmWait = (NA < NB ? 8 : 0) + ((NA < NB ? NA : NB) - 2) * (NR + 2);
  constexpr int kScaleBase = Geo::kScaleBase, kJunkBase = Geo::kJunkBase;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: picks descriptors and LDS rows
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, rr = lane & 15;
  const uint32_t row_bytes = static_cast<uint32_t>(g.K);
  const uint32_t srow_bytes = static_cast<uint32_t>(g.K / 32);
  const int dr_row = 8 * wave + (lane >> 3);
  const int dr_ch = mx_swz(dr_row, lane & 7);
  const uint8_t* l8 = reinterpret_cast<const uint8_t*>(lds);
  // LDS rings: NA A slots (BM rows each), then NB B slots (256 rows each),
  // so every fragment read is one of four lane bases plus an offset under 64 KB
  // that the read instruction carries.  The bases are hidden from the optimizer
  // so that it keeps one register each rather than one per offset.
  constexpr int kASlot = BM * kMxCh, kBSlot = kMxBN * kMxCh;   // u32x4 per slot
  int a_lo = (wm * (BM / 2) + rr) * kMxCh + mx_swz(rr, q);
  int a_hi = (wm * (BM / 2) + rr) * kMxCh + mx_swz(rr, q + 4);
  int b_lo = NA * kASlot + (wn * 128 + rr) * kMxCh + mx_swz(rr, q);
  int b_hi = NA * kASlot + (wn * 128 + rr) * kMxCh + mx_swz(rr, q + 4);
  int sa_b = kScaleBase * 16 + (wm * (BM / 2) + rr) * kSRow + q;
  int sb_b = kScaleBase * 16 + (BM + wn * 128 + rr) * kSRow + q;
  __asm__ volatile("" : "+v"(a_lo), "+v"(a_hi), "+v"(b_lo), "+v"(b_hi), "+v"(sa_b), "+v"(sb_b));

  const int rows = __builtin_amdgcn_readfirstlane(st.rows[s]);
  const int m0 = (mt - __builtin_amdgcn_readfirstlane(st.tile_start[s])) * BM;
  const int a_off = __builtin_amdgcn_readfirstlane(g.a_by_o_off ? st.o_off[s] : st.a_off[s]);
  const int o_off = __builtin_amdgcn_readfirstlane(st.o_off[s]);
  const bool gather = g.row_token != nullptr && s < g.E;
  const int n0 = nt * kMxBN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, static_cast<uint32_t>(g.a_rows) * row_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(g.As, static_cast<uint32_t>(g.a_rows) * srow_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.W + static_cast<size_t>(s) * g.N * g.K,
                                            static_cast<uint32_t>(g.N) * row_bytes);
  const __amdgpu_buffer_rsrc_t rbs = make_rsrc(g.Ws + static_cast<size_t>(s) * g.N * (g.K / 32),
                                             static_cast<uint32_t>(g.N) * srow_bytes);
  // code loads: load n of wave w fills rows 32 n + 8 w + lane / 8 (A rows, then B rows);
  // rows past the segment get an offset past the end (the range check reads zero)
  u32x8 va = {};
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = m0 + 32 * i + dr_row;
    const int arow = r < rows ? (gather ? g.row_token[a_off + r] : a_off + r) : -1;
    va[i] = arow >= 0 ? static_cast<uint32_t>(arow) * row_bytes + dr_ch * 16 : 0x80000000u;
  }
  const uint32_t vb = static_cast<uint32_t>(n0 + dr_row) * row_bytes + dr_ch * 16;
  // scale loads: 4 SG bytes (SG stages of 4 blocks) per row, one row per lane;
  // wave w loads A rows 64 w .. 64 w + 63 (rows from BM on, and past the
  // segment, read zero) and B rows 64 w .. 64 w + 63, with no branch
  uint32_t vs_a, vs_b;
  {
    const int r = 64 * wave + lane;
    const int rg = m0 + r;
    const int arow = r < BM && rg < rows ? (gather ? g.row_token[a_off + rg] : a_off + rg) : -1;
    vs_a = arow >= 0 ? static_cast<uint32_t>(arow) * srow_bytes : 0x80000000u;
    vs_b = static_cast<uint32_t>(n0 + r) * srow_bytes;
  }

  // direct load n < MB: A rows 32 n + .. of stage t (K step k0 + t) into A slot sl;
  // n >= MB: B rows 32 (n - MB) + .. of stage t into B slot sl
  auto issue1 = [&](int sl, int t, int n) __attribute__((always_inline)) {
    const uint32_t kb = static_cast<uint32_t>(k0 + t) * kMxBK;
    {
      if (n < MB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(lds + sl * kASlot + (32 * n + 8 * wave) * kMxCh), 16,
            va[n], kb, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb,
            (__attribute__((address_space(3))) void*)(lds + NA * kASlot + sl * kBSlot +
                                                      (32 * (n - MB) + 8 * wave) * kMxCh),
            16, vb, static_cast<uint32_t>(32 * (n - MB)) * row_bytes + kb, 0, 0);
    }
  };
  // scale group G (K steps SG G .. SG G + SG - 1) of this wave's A (n = 0) or B
  // (n = 1) rows 64 w .. 64 w + 63 into scale slot G % NSS; with on false (or
  // A rows from BM on) the load reads nothing (an offset past the end) and
  // lands in the scratch area
  auto issue_scales = [&](int G, int n, bool on) __attribute__((always_inline)) {
    on = on && (n == 1 || 64 * wave < BM);
    const int dst = on ? kScaleBase + ((G % NSS) * kScaleSlot + (n * BM + 64 * wave) * kSRow) / 16 : kJunkBase;
    const uint32_t vo = on ? (n == 0 ? vs_a : vs_b) : 0x80000000u;
    const uint32_t so = on ? static_cast<uint32_t>(G) * kSRow : 0u;
    auto* lp = (__attribute__((address_space(3))) void*)(lds + dst);
    if constexpr (SG == 4)   // (the load width must be a literal)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(n == 0 ? ras : rbs, lp, 16, vo, so, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(n == 0 ? ras : rbs, lp, 4, vo, so, 0, 0);
  };
  // byte offset, within the scale slots, of stage t's scales (K step k0 + t)
  auto sofs = [&](int t) __attribute__((always_inline)) {
    const int a = k0 + t;
    return ((a / SG) % NSS) * kScaleSlot + (a % SG) * 4;
  };

  // fragments: B blocks 0..7 and A blocks 0..MB-1 with their scale bytes;
  // a block of the next stage is read into the registers of the same block
  // of this stage once that block's last MFMA has been issued
  // (scale bytes stay bytes until the MFMA that takes them, so any widening
  // is placed there, not at the top of the loop)
  i32x8 fb[8], fa[MB];
  uint8_t sb[8], sa[MB];
  auto frag = [&](int lo_i, int hi_i, int sc_i, i32x8& f, uint8_t& sc) __attribute__((always_inline)) {
    const u32x4 lo = lds[lo_i];
    const u32x4 hi = lds[hi_i];
    f = __builtin_bit_cast(i32x8, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    sc = l8[sc_i];
  };
  // fragments of stage t (ring slots t % NA, t % NB); the wave-uniform
  // offsets are added to the lane bases once per use site
  // Stage t's slot offsets (u32x4 of its A and B slots, bytes of its scales)
  // are computed once per step as scalars the optimizer cannot take apart:
  // otherwise it rewrites them per read (as base + 32 KB, then - 32 KB again)
  // and a read costs two vector adds instead of an immediate offset.
  struct StageOfs {
    int a, b, s;
  };
  auto stage_ofs = [&](int t) __attribute__((always_inline)) {
    StageOfs o{(t % NA) * kASlot, (t % NB) * kBSlot, sofs(t)};
    __asm__ volatile("" : "+s"(o.a), "+s"(o.b), "+s"(o.s));
    return o;
  };
  auto readA = [&](const StageOfs& so, int i) __attribute__((always_inline)) {
    const int o = so.a + 16 * i * kMxCh;
    frag(a_lo + o, a_hi + o, sa_b + so.s + 16 * kSRow * i, fa[i], sa[i]);
  };
  auto readB = [&](const StageOfs& so, int j) __attribute__((always_inline)) {
    const int o = so.b + 16 * j * kMxCh;
    frag(b_lo + o, b_hi + o, sb_b + so.s + 16 * kSRow * j, fb[j], sb[j]);
  };

  floatx4 acc[MB][8];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: A stages 0 .. NA-1 and B stages 0 .. NB-1 in flight, stage sp
  // after two scale loads as in the loop (the first two scale groups, or at
  // SG = 1 the stage's own while sp < NB), then its A rows (sp < NA), then
  // its B rows (sp < NB); stage 0 published, its B blocks and A rows 0, 1
  // read.  Stages past the end load the last stage again, into slots no step
  // reads.
  constexpr int NP = NA > NB ? NA : NB;
#pragma unroll
  for (int sp = 0; sp < NP; ++sp) {
#pragma unroll
    for (int n = 0; n < 2; ++n) issue_scales(SG == 1 ? k0 + sp : k0 / SG + sp, n, SG == 1 ? sp < NB : sp < 2);
#pragma unroll
    for (int n = sp < NA ? 0 : MB; n < (sp < NB ? NR : MB); ++n) issue1(sp, min(sp, kn - 1), n);
  }
  // stage 0 (and what came before it): all but the loads of stages 1 .. NP-1
  constexpr int kPrologueWait = (NP - 1) * 2 + (NA - 1) * MB + (NB - 1) * 8;
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPrologueWait));
  mx_barrier();
  {
    const StageOfs o0 = stage_ofs(0);
    readA(o0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) readB(o0, j);
    readA(o0, 1);
  }
  // Let the prologue's reads land here, once per tile: otherwise the waits
  // at the top of the loop are sized for them (they land in another order
  // than the loop's own reads) on every step.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt 0

  // step t in ring slots t % NA, t % NB.  A step that starts a scale group G
  // loads group G + kLook, just before the codes of A stage t+NA, so the wait
  // for any later stage covers it.
  auto kstep = [&](int t) __attribute__((always_inline)) {
    const int ca = t % NA, cb = t % NB;
    // past the end: the last stage again, into a slot no step reads
    const int ta = min(t + NA, kn - 1), tb = min(t + NB, kn - 1);
    const bool group_start = (k0 + t) % SG == 0;
    const int gnext = (k0 + t) / SG + kLook;
    const StageOfs o0 = stage_ofs(t), o1 = stage_ofs(t + 1);
#pragma unroll
    for (int m = 0; m < HM; ++m) {
      const int i = m >> 3, j = m & 7;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, sb[j], 0,
                                                                   sa[i]);
      if ((m & 1) == 0 && (m >> 1) < NF1) readA(o0, 2 + (m >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(kVmWait));   // stage t+1 landed in this wave
    mx_barrier();                          // ... in every wave, and every wave has stage t in registers
#pragma unroll
    for (int m = 0; m < HM; ++m) {
      // B block outermost: block j of stage t is done after its last row and
      // block j of stage t+1 takes its registers; A rows 0, 1 are done already
      const int j = m / (MB / 2), i = MB / 2 + m % (MB / 2);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, sb[j], 0,
                                                                   sa[i]);
      if (m < 2) readA(o1, m);
      if (i == MB - 1) readB(o1, j);
      // the step's NR + 2 direct loads, spread evenly over the half step: issued
      // back to back they overfill the texture unit's address FIFO, and the
      // wave's next MFMA waits behind the stalled load
      if ((m * (NR + 2)) % HM < NR + 2) {
        const int l = m * (NR + 2) / HM;
        if (l < 2) issue_scales(gnext, l, group_start);
        else if (l < MB + 2) issue1(ca, ta, l - 2);
        else issue1(cb, tb, l - 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
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
  // One branch-free loop body for every step keeps one register assignment
  // and one basic block, so the interleaving above is what runs.  The last
  // steps' barrier, next-stage reads and refills are harmless: the reads fill
  // dead registers and the refills (of the last stage again) land in slots no
  // later step reads, and are waited for before the tile ends.
  for (int t = 0; t < kn; ++t) kstep(t);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt 0
  if constexpr (kPad > 0) {
#pragma unroll
    for (int k = 0; k < kPad; ++k) __asm__ volatile("" ::"a"(pin[k]));
  }
  mx_barrier();   // the next tile's loads reuse the ring

  // Epilogue: lane (rr, q) holds, for block (i, j), row 16 i + rr of the wave
  // tile and columns 16 j + 4 q .. + 3.  A piece of a tail tile stores its
  // float32 partial tile (row-major, rows PBM piece ..); a whole tile adds the bias,
  // applies the activation (phase 1) and stores MX blocks or bf16.
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.part, static_cast<uint32_t>(g.part_cap) * PBM * kMxBN * 4u);
  const uint32_t pv = (static_cast<uint32_t>(wm * (BM / 2) + rr) * kMxBN + wn * 128 + 4 * q) * 4u;
  const int cbase = n0 + wn * 128 + 4 * q;
  uint2 bq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    bq[j] = g.bias ? *reinterpret_cast<const uint2*>(g.bias + static_cast<size_t>(s) * g.N + cbase + 16 * j)
                   : make_uint2(0u, 0u);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int rl = m0 + wm * (BM / 2) + 16 * i + rr;
    const bool ok = rl < rows;
    if (piece >= 0) {
      const uint32_t ps = (static_cast<uint32_t>(piece) * PBM + 16 * i) * kMxBN * 4u;
      // (through vector registers: stored from the accumulation registers,
      // the accumulators of the shorter tiles get shuttled between register
      // files inside the K loop)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        floatx4 t = acc[i][j];
        __asm__ volatile("" : "+v"(t));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), pr, pv + 64 * j, ps, 0);
      }
    } else if constexpr (kMxOut) {
      // MX blocks of 32 columns: j pair (2 c, 2 c + 1) x the 4 lanes q of the
      // row, computed a block at a time (8 values a lane)
      uint8_t* crow = static_cast<uint8_t*>(g.C) + static_cast<size_t>(o_off + (ok ? rl : 0)) * g.N;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * c + h;
          v[h][0] = mx_act<ACT>(acc[i][j][0] + __uint_as_float(bq[j].x << 16));
          v[h][1] = mx_act<ACT>(acc[i][j][1] + __uint_as_float(bq[j].x & 0xffff0000u));
          v[h][2] = mx_act<ACT>(acc[i][j][2] + __uint_as_float(bq[j].y << 16));
          v[h][3] = mx_act<ACT>(acc[i][j][3] + __uint_as_float(bq[j].y & 0xffff0000u));
        }
        float am = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(v[h][e]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        const int sx = mx_exponent(am);
        const float inv = mx_inv_scale(sx);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t w = cvt2<false>(v[h][0] * inv, v[h][1] * inv, 0u);
          w = cvt2<true>(v[h][2] * inv, v[h][3] * inv, w);
          if (ok) *reinterpret_cast<uint32_t*>(crow + cbase + 16 * (2 * c + h)) = w;
        }
        if (ok && q == 0)
          g.Cs[static_cast<size_t>(o_off + rl) * (g.N / 32) + (n0 + wn * 128) / 32 + c] = static_cast<uint8_t>(sx + 127);
      }
    } else {
      if (ok) {
        uint16_t* crow = static_cast<uint16_t*>(g.C) + static_cast<size_t>(o_off + rl) * g.N + cbase;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v0 = acc[i][j][0] + __uint_as_float(bq[j].x << 16);
          const float v1 = acc[i][j][1] + __uint_as_float(bq[j].x & 0xffff0000u);
          const float v2 = acc[i][j][2] + __uint_as_float(bq[j].y << 16);
          const float v3 = acc[i][j][3] + __uint_as_float(bq[j].y & 0xffff0000u);
          *reinterpret_cast<uint2*>(crow + 16 * j) =
              make_uint2(mx_pack_bf16x2(mx_act<ACT>(v0), mx_act<ACT>(v1)), mx_pack_bf16x2(mx_act<ACT>(v2), mx_act<ACT>(v3)));
        }
      }
    }
  }
}

// The grouped GEMM: a persistent grid over the work items (whole tiles, then
// the pieces of the split tail).  With BM1 = 0 every tile is BM0 rows high;
// else each segment's tiles are BM0 or BM1 rows high, as the segment table
// records, and a tile runs the body of its height.
template <int ACT, int BM0, int BM1, int SG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_kernel(MxArgs g) {
  constexpr int PBM = BM1 > BM0 ? BM1 : BM0;
  constexpr int kW0 = MxGeom<BM0, SG>::kWords;
  constexpr int kW1 = BM1 ? MxGeom<BM1 ? BM1 : BM0, SG>::kWords : 0;
  // one LDS object, so the waits the compiler places for direct loads are the
  // ones the tile body writes
  __shared__ u32x4 lds[kW0 > kW1 ? kW0 : kW1];
  static_assert(sizeof(lds) <= 160 * 1024, "LDS");

  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = __builtin_amdgcn_readfirstlane(st.tile_start[g.nseg]);
  const int ntn = g.N / kMxBN;
  const int total = total_mt * ntn;
  const int nk = g.K / kMxBK;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const TailPlan tp = tail_plan(total, gridDim.x, nk, g.part_cap);
  const int items = tp.full + tp.tail * tp.S;

  for (int it = 0;; ++it) {
    const int w = it * gridDim.x + xcd * per_xcd + slot;
    if (w >= items) break;
    // work item w: a whole tile (w < full), or piece p of tail tile full + idx / S,
    // K steps k0 .. k0 + kn - 1
    int L = w, k0 = 0, kn = nk, piece = -1;
    if (w >= tp.full) {
      piece = w - tp.full;
      const int pp = piece % tp.S;
      L = tp.full + piece / tp.S;
      k0 = pp * nk / tp.S;
      kn = (pp + 1) * nk / tp.S - k0;        // >= 4
    }
    int mt, nt;
    tile_of(L, total_mt, ntn, mt, nt);
    const int s = __builtin_amdgcn_readfirstlane(find_segment(st.tile_start, g.nseg, mt));
    if constexpr (BM1 == 0) {
      mx_tile<ACT, BM0, SG, PBM>(g, lds, st, s, mt, nt, k0, kn, piece);
    } else {
      if (__builtin_amdgcn_readfirstlane(st.tile_bm[s]) == BM1)
        mx_tile<ACT, BM1 ? BM1 : BM0, SG, PBM>(g, lds, st, s, mt, nt, k0, kn, piece);
      else
        mx_tile<ACT, BM0, SG, PBM>(g, lds, st, s, mt, nt, k0, kn, piece);
    }
  }
}

// Fix-up of the split tail, in 16-row chunks of the tail tiles strided over
// the launch's workgroups (four a CU; P is the GEMM's grid, which fixed the
// tail plan).  Each thread owns four consecutive columns of four rows;
// the S partial tiles are summed in piece order, then the bias, the
// activation (phase 1) and the store as in the GEMM epilogue: phase 1 MX
// blocks of 32 columns (8 lanes a block), phase 2 bf16.  Tile heights as in
// gemm_mx_kernel; partial tiles are PBM rows apart.
template <int ACT, int BM0, int BM1>
__global__ __launch_bounds__(256) void mx_tail_fixup_kernel(MxArgs g, int P) {
  constexpr bool kMxOut = ACT != 0;
  constexpr int PBM = BM1 > BM0 ? BM1 : BM0;
  const SegTableRO st = seg_table_ro(g.seg, g.nseg, g.E);
  const int total_mt = st.tile_start[g.nseg];
  const int ntn = g.N / kMxBN;
  const TailPlan tp = tail_plan(total_mt * ntn, P, g.K / kMxBK, g.part_cap);
  if (tp.tail == 0) return;
  constexpr int kChunks = PBM / 16;
  const int c = 4 * (threadIdx.x & 63);
  for (int w = blockIdx.x; w < tp.tail * kChunks; w += gridDim.x) {
    const int tt = w / kChunks, r0 = (w % kChunks) * 16;
    int mt, nt;
    tile_of(tp.full + tt, total_mt, ntn, mt, nt);
    const int s = find_segment(st.tile_start, g.nseg, mt);
    const int bm = BM1 == 0 ? BM0 : st.tile_bm[s];
    if (r0 >= bm) continue;   // rows of the next tile
    const int rows = st.rows[s];
    const int m0 = (mt - st.tile_start[s]) * bm;
    const int o_off = st.o_off[s];
    const int n = nt * kMxBN + c;
    const uint2 b = g.bias ? *reinterpret_cast<const uint2*>(g.bias + static_cast<size_t>(s) * g.N + n)
                           : make_uint2(0u, 0u);
    const float b0 = __uint_as_float(b.x << 16), b1 = __uint_as_float(b.x & 0xffff0000u);
    const float b2 = __uint_as_float(b.y << 16), b3 = __uint_as_float(b.y & 0xffff0000u);
    const float* part = g.part + static_cast<size_t>(tt) * tp.S * PBM * kMxBN;
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
          v[k][p] = *reinterpret_cast<const floatx4*>(part + (static_cast<size_t>(min(p0 + p, tp.S - 1)) * PBM + rr) *
                                                                 kMxBN + c);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < kFixS; ++p)
          if (p0 + p < tp.S) a[k] = p0 + p == 0 ? v[k][p] : a[k] + v[k][p];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = r0 + (threadIdx.x >> 6) + 4 * k;   // one row per wave: the lanes of a block agree
      if (m0 + rr >= rows) break;
      const float v0 = mx_act<ACT>(a[k][0] + b0), v1 = mx_act<ACT>(a[k][1] + b1);
      const float v2 = mx_act<ACT>(a[k][2] + b2), v3 = mx_act<ACT>(a[k][3] + b3);
      const size_t row = static_cast<size_t>(o_off + m0 + rr);
      if constexpr (kMxOut) {
        float am = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        am = fmaxf(am, __shfl_xor(am, 4));
        const int sx = mx_exponent(am);
        const float inv = mx_inv_scale(sx);
        uint32_t wq = cvt2<false>(v0 * inv, v1 * inv, 0u);
        wq = cvt2<true>(v2 * inv, v3 * inv, wq);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(g.C) + row * g.N + n) = wq;
        if ((threadIdx.x & 7) == 0) g.Cs[row * (g.N / 32) + n / 32] = static_cast<uint8_t>(sx + 127);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + row * g.N + n) =
            make_uint2(mx_pack_bf16x2(v0, v1), mx_pack_bf16x2(v2, v3));
      }
    }
  }
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t* src, int rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t st) {
  const size_t nblocks = static_cast<size_t>(rows) * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  size_t grid = (nblocks + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, src, nblocks, cols / 32,
                     codes, scales);
  return hipGetLastError();
}

// Phase 1: A = x as MX (xq codes / scales), output H as MX in the hidden
// buffer (codes [R, h], then scales [R, h / 32]); phase 2: A = H, output Y bf16.
hipError_t launch_expert_ffn_mx(const Problem& p, const MxWeights& w, const Workspace& ws, int phase,
                                hipStream_t st) {
  MxArgs g;
  g.seg = ws.seg;
  g.nseg = p.E + p.S;
  g.E = p.E;
  const size_t R = static_cast<size_t>(p.A) + static_cast<size_t>(p.S) * p.T;
  uint8_t* hcodes = static_cast<uint8_t*>(ws.hbuf);
  uint8_t* hscales = hcodes + R * p.h;
  if (phase == 1) {
    g.A = ws.xq;
    g.As = ws.xq_scales;
    g.a_rows = p.T;
    g.row_token = ws.row_token;
    g.a_by_o_off = 0;
    g.W = w.W1;
    g.Ws = w.W1s;
    g.bias = static_cast<const uint16_t*>(w.b1);
    g.C = hcodes;
    g.Cs = hscales;
    g.N = p.h;
    g.K = p.d;
  } else {
    g.A = hcodes;
    g.As = hscales;
    g.a_rows = static_cast<int>(R);
    g.row_token = nullptr;
    g.a_by_o_off = 1;
    g.W = w.W2;
    g.Ws = w.W2s;
    g.bias = static_cast<const uint16_t*>(w.b2);
    g.C = ws.ybuf;
    g.Cs = nullptr;
    g.N = p.d;
    g.K = p.h;
  }
  g.part = ws.part;
  g.part_cap = ws.part_cap;
  int grid = device_cu_count();
  grid = (grid + 7) / 8 * 8;
  const int act = phase == 2 ? 0 : (p.act == MOE_ACT_SILU ? 2 : 1);
  // the fix-up runs right after the GEMM on the same stream; it returns at
  // once when the tail was not split
  // scales in groups of 4 stages (16-byte loads) when rows of scales are a
  // multiple of 16 bytes (K a multiple of 512), else one stage at a time
  const bool sg4 = g.K % 512 == 0;
#define MOE_MX_LAUNCH(ACT_, BM0_, BM1_)                                                                  \
  do {                                                                                                   \
    if (sg4) hipLaunchKernelGGL((gemm_mx_kernel<ACT_, BM0_, BM1_, 4>), dim3(grid), dim3(256), 0, st, g); \
    else hipLaunchKernelGGL((gemm_mx_kernel<ACT_, BM0_, BM1_, 1>), dim3(grid), dim3(256), 0, st, g);     \
    hipLaunchKernelGGL((mx_tail_fixup_kernel<ACT_, BM0_, BM1_>), dim3(4 * grid), dim3(256), 0, st, g, grid); \
  } while (0)
  // 256-row tiles, or per segment 128 or 192 rows (the table says which)
  if (!p.gemm_mixed) {
    if (act == 1) MOE_MX_LAUNCH(1, 256, 0);
    else if (act == 2) MOE_MX_LAUNCH(2, 256, 0);
    else MOE_MX_LAUNCH(0, 256, 0);
  } else {
    if (act == 1) MOE_MX_LAUNCH(1, 128, 192);
    else if (act == 2) MOE_MX_LAUNCH(2, 128, 192);
    else MOE_MX_LAUNCH(0, 128, 192);
  }
#undef MOE_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
