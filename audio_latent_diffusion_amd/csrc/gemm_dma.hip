// Pipelined MFMA GEMM for the DiT linears: y[M, N] = epilogue(X[M, K] . W[N, K]^T)
// with both operands K-contiguous, fed by direct global -> LDS loads.
//
//  * W8A8: int8 x int8 -> int32 on v_mfma_i32_32x32x32_i8; epilogue
//    acc * x_scale[m] * w_scale[n] + bias (+GELU) (+residual) -> fp16, and an
//    optional raw int32 accumulator dump;
//  * F16: fp16 x fp16 -> fp32 on v_mfma_f32_32x32x16_f16;
//  * Q4: fp16 activations x 4-bit weights (groups of 32 along K with fp16
//    scales): packed nibbles and scales travel to LDS, and each lane turns its
//    weight fragment into fp16(q * s) in registers right before the fp16 MFMA.
//
// Both MFMAs take, per operand, a 32-row x 32-byte fragment: lane l holds row
// l % 32 and the 16 bytes at 16 (l / 32) of the 32-byte K slice.  Only the
// pairing of K positions between the two operands matters for a dot product,
// so any K order inside a slice is correct when both operands share it.
// (The 32x32 shapes run at the full matrix rate with a few independent
// accumulators; the 16x16 int8 shape needs many more to hide its latency.)
//
// A K stage is 128 bytes of every tile row (one cache line per row).  LDS
// holds a stage as blocks of 8 rows x 128 bytes (1 KB), written by
// global_load_lds_dwordx4: lane l of a wave fetches row l / 8 of the block and
// the hardware stores its 16 bytes at slot l.  The lane picks which 16-byte
// chunk of the row it fetches: slot p of row r holds chunk p ^ g(r) with
// g(r) = (r & 7) ^ ((r >> 3) & 1), so that the 16 rows read together by an
// MFMA operand load (same chunk, consecutive rows) fall on distinct banks.
// Each operand fragment is then one ds_read_b128 per lane.  A Q4 stage (64 K
// values) holds the 32 packed bytes of each weight row as blocks of 32 rows
// (the 16 bytes of group 0 of every row, then those of group 1) and the two
// fp16 scales of each row (4-byte copies, 64 rows per instruction).  No VGPR
// staging: a ring of STAGES buffers keeps STAGES - 1 stages in flight.
//
// Per K stage: wait until this wave's loads of stage kt have landed
// (s_waitcnt vmcnt with the count of loads issued after them), barrier (every
// wave's loads of stage kt visible, every wave done with stage kt - 1), issue
// the loads of stage kt + STAGES - 1 into the buffer of stage kt - 1, then
// run the four 32-byte K slices of the stage.  The next stage's copies are
// issued in four parts, one before each slice's MFMAs, and fragment reads
// are double buffered in registers (slice s + 1 is read during slice s).
//
// Measured limits on MI355X that shape this: LDS serves ~128 B/clk per CU,
// shared by the DMA writes and the fragment reads; a 256 x 256 tile at full
// matrix rate needs ~94 B/clk of it with 4 waves of 128 x 128 (reads 64,
// copies 32) and ~128 B/clk with 8 waves of 128 x 64, so LDS, not HBM,
// bounds the main loop; a single CU's DMA copies stream ~66 B/clk from L2.
// The 256 x 256 tile still runs 8 waves (two per SIMD): the second wave
// covers the first one's stalls and measured faster on every serving shape.
//
// A persistent variant (one workgroup per CU walking its tiles, the next
// tile's first stages in flight during the epilogue, stores straight from the
// accumulators) measured 10-25% slower: in the MFMA layout a store
// instruction covers 16 contiguous bytes of each of 32 rows, four times the
// memory requests of the 128-byte rows the LDS-staged epilogue writes, and at
// 256 x 256 the staging area and a prefetched stage do not fit in LDS
// together.
//
// Operand roles are swapped in the MFMA (W fragment first): accumulator
// register r of lane l then holds output row l % 32 and column
// 8 (r / 4) + 4 (l / 32) + r % 4 of its 32x32 block.  The epilogue stages the
// accumulators through LDS and writes 8 consecutive fp16 per lane (16-byte
// stores); the epilogue kind (plain, residual, GELU) is a template parameter
// so no kernel carries code it does not run.
//
// The int8 256 x 192 tile (the serving model's qkv, o, q, ox and down
// projections) adds 4 producer waves to its 8 MFMA waves: they issue every
// stage copy, so an MFMA wave never stalls on a copy instruction's issue (with
// the copies spread over the MFMA waves, issuing them cost 15-20 % of the main
// loop even when nothing waited for them; measured on MI355X).  12 waves fit
// 3 per SIMD.
//
// Workgroups are mapped XCD-aware: consecutive workgroup ids land on
// different XCDs (round-robin).  Large tiles over an X at least as large as W
// take row bands (band_tile): each XCD owns a band of tile rows across all
// columns, so the band's X panels stay in its L2 over all rounds (qkv at the
// serving shapes: 9 % faster).  Other launches remap tile ids to give each XCD
// one contiguous run of tiles that is a compact block of the output (grouped
// order), so the X and W panels it touches stay few and in its L2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ald {
namespace {

constexpr int BLK = 1024;  // LDS block: one 16-byte copy instruction (64 lanes)
constexpr int KB = 128;    // X bytes per stage and row (one cache line)

enum { M_I8 = 0, M_F16 = 1, M_Q4 = 2, M_Q8W = 3 };                  // operand modes
enum { EPI_PLAIN = 0, EPI_RES = 1, EPI_GELU = 2, EPI_GELU_RES = 3 };  // epilogue kinds

template <int BM_, int BN_, int STAGES_, int MODE_, int WGN_ = 2, int WGM_ = 2>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_, MODE = MODE_;
  static constexpr bool INT = MODE == M_I8, Q4 = MODE == M_Q4, Q8W = MODE == M_Q8W;
  static constexpr int WGM = WGM_, WGN = WGN_, WAVES = WGM * WGN, THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MI = WM / 32, NJ = WN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int KS = 4;                      // 32-byte X slices per stage
  static constexpr int BX = BM / 8;                 // X blocks per stage (8 rows x 128 B)
  static constexpr int BW = Q4 ? BN / 32 : (Q8W ? BN / 16 : BN / 8);  // W blocks per stage
  // W copies padded with repeats of the last W block's copy (the same bytes
  // to the same place) so that the copies split evenly over the waves
  static constexpr int WPAD = Q4 ? 0 : (WAVES - (BX + BW) % WAVES) % WAVES;
  static constexpr int BWC = BW + WPAD;  // W copy instructions per stage
  // Q4 scale copies (64 rows each), padded the same way
  static constexpr int SC0 = Q4 ? BN / 64 : 0;
  static constexpr int SCL = Q4 ? SC0 + (WAVES - (BX + BW + SC0) % WAVES) % WAVES : 0;
  static constexpr int LOADS = (BX + BWC + SCL) / WAVES;  // copy instructions per wave and stage
  static constexpr int W_OFF = BX * BLK;                 // offsets within a stage
  static constexpr int S_OFF = (BX + BW) * BLK;
  static constexpr int STAGE_BYTES = S_OFF + SCL * 256;
  static constexpr int LDS = STAGES * STAGE_BYTES;
  // epilogue staging: PW columns per pass, rows padded by 4 words
  static constexpr int PW = WN < 64 ? WN : (WAVES > 4 ? 32 : 64);
  static constexpr int RS = PW + 4;
  static constexpr int EPI_LDS = WAVES * WM * (RS + 1) * 4;
  // per-row and per-column epilogue scalars (x_scale[BM], w_scale[BN], bias[BN])
  // (padded to whole copy instructions of 64 scalars)
  static constexpr int SC_OFF = LDS > EPI_LDS ? LDS : EPI_LDS;
  static constexpr int SC_N = BM + 2 * BN, SC_PAD = (SC_N + 63) / 64 * 64;
  static constexpr int LDS_TOTAL = SC_OFF + SC_PAD * 4;
  static constexpr int SC_LOADS = SC_PAD / 64;  // 64 scalars per copy instruction
  static_assert((BX + BWC + SCL) % WAVES == 0, "copies must split evenly over the waves");
  static_assert(BX % WAVES == 0, "X copies take whole rounds over the waves");
  static_assert(MI >= 1 && NJ >= 1 && WM == 32 * MI && WN == 32 * NJ, "wave tile");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) < 64, "vmcnt range");
  static_assert(BM % 32 == 0 && BN % 32 == 0, "whole 32 x 32 MFMA blocks");
  static_assert(WN % PW == 0 && PW % 32 == 0, "epilogue passes cover the wave tile");
};

// s_waitcnt vmcnt(N): expcnt and lgkmcnt fields left at their maxima
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until the oldest outstanding stage has landed: at most `ahead` later
// stages (LOADS instructions each) may remain in flight (vector memory loads
// retire in issue order)
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      vm_wait<LOADS * MAXA>();
      return;
    }
    wait_stages<LOADS, MAXA - 1>(ahead);
  } else {
    vm_wait<0>();
  }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// bank swizzle: chunk c of tile row r sits at slot c ^ g(r) of its 128-byte
// row, so that the 16 (or 8) consecutive rows read together with one chunk
// index cover distinct banks
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 8-bit weight rows of the weight-only mode are 64 bytes (four 16-byte
// chunks), two rows per 128-byte bank period: chunk c of row r sits at slot
// c ^ ((r >> 1) & 3), so the 32 rows of one fragment read (same chunk) cover
// all eight 16-byte positions of the period, four rows each, the fewest any
// 64-byte row layout allows (with c ^ (r & 3) the slot repeats the row's
// half of the period and only four positions were used, eight rows each)
__device__ __forceinline__ int q8w_swz(int r) { return (r >> 1) & 3; }

// The copy layout of config C dealt to P dedicated producer waves (int8 and
// fp16 operands: X blocks then W blocks, no padding needed when P divides
// their count).
template <class C, int P>
struct ProducerCfg {
  static constexpr bool INT = C::INT, Q4 = C::Q4, Q8W = C::Q8W;
  static constexpr int WAVES = P, BX = C::BX, BW = C::BW, BWC = C::BW, SC0 = C::SC0, S_OFF = C::S_OFF;
  static constexpr int LOADS = (BX + BWC) / P;
  static_assert(!Q4 && !Q8W && (BX + BWC) % P == 0, "producer copies split evenly");
  static_assert(LOADS * (C::STAGES - 2) < 64, "vmcnt range");
};

// The copies of one stage, dealt round-robin to the waves: X blocks, then W
// blocks, then (Q4) scale copies.  Each lane keeps a 32-bit byte offset of
// its source at K stage 0 from the operand's base pointer (uniform, so the
// copy can address as scalar base + vector offset); sources advance by a
// fixed step per stage.
template <class C>
struct Loader {
  uint32_t off[C::LOADS];

  // kind of copy i of a wave: 0 = X, 1 = W, 2 = Q4 scales (uniform)
  __device__ __forceinline__ static int kind(int wave, int i) {
    const int b = wave + C::WAVES * i;
    return b < C::BX ? 0 : (b < C::BX + C::BWC ? 1 : 2);
  }
  __device__ __forceinline__ static int step(int k) {
    return k == 0 ? KB : (C::Q4 ? (k == 1 ? 32 : 4) : (C::Q8W ? 64 : KB));
  }
  __device__ __forceinline__ static int dst(int b) {
    if (b < C::BX + C::BW) return b * BLK;
    if (b < C::BX + C::BWC) return (C::BX + C::BW - 1) * BLK;  // padding: the last W block again
    return C::S_OFF + (b - C::BX - C::BWC) * 256;
  }

  __device__ __forceinline__ void init(const GemmArgs& g, int m0, int n0, int wave, int lane) {
    constexpr int EB = C::INT ? 1 : 2;  // bytes per X (and int8 / fp16 W) element
    const uint32_t ldx = (uint32_t)g.lda * EB;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int b = wave + C::WAVES * i;  // copy index within the stage
      if (b < C::BX) {  // X: lane l fetches row l / 8 of the block, swizzled chunk
        const int tr = b * 8 + (lane >> 3);
        const int r = min(m0 + tr, g.M - 1);  // rows past the edge re-read a valid row; results dropped
        off[i] = (uint32_t)r * ldx + ((lane & 7) ^ swz(tr)) * 16;
      } else if (b < C::BX + C::BWC) {
        const int bw = min(b - C::BX, C::BW - 1);  // padding repeats the last W block
        if constexpr (C::Q8W) {  // int8 W of fp16 X: 64 bytes per row and stage, 16 rows per block
          const int tr = bw * 16 + (lane >> 2);
          const int r = min(n0 + tr, g.N - 1);
          off[i] = (uint32_t)r * (uint32_t)g.K + ((lane & 3) ^ q8w_swz(tr)) * 16;
        } else if constexpr (!C::Q4) {  // int8 / fp16 W: same layout as X
          const int tr = bw * 8 + (lane >> 3);
          const int r = min(n0 + tr, g.N - 1);
          off[i] = (uint32_t)r * (uint32_t)(g.K * EB) + ((lane & 7) ^ swz(tr)) * 16;
        } else {  // packed W: lane l fetches group l / 32 of the stage of row l % 32
          const int tr = bw * 32 + (lane & 31);
          const int r = min(n0 + tr, g.N - 1);
          off[i] = (uint32_t)r * (uint32_t)(g.K / 2) + (lane >> 5) * 16;
        }
      } else {  // Q4 scales: both fp16 group scales of a row (4 bytes); padding repeats the last copy
        const int sidx = min(b - C::BX - C::BWC, C::SC0 - 1);
        const int r = min(n0 + sidx * 64 + lane, g.N - 1);
        off[i] = (uint32_t)r * (uint32_t)(g.K / 32) * 2;
      }
    }
  }
  // part P of PARTS of the stage's copies (spread over the K slices so the
  // wave keeps feeding MFMAs while the memory pipeline accepts its copies)
  template <int P, int PARTS>
  __device__ __forceinline__ void issue_part(const uint8_t* xb, const uint8_t* wb, const uint8_t* sb, int wave,
                                             uint8_t* stage, int kt) const {
    constexpr int lo = C::LOADS * P / PARTS, hi = C::LOADS * (P + 1) / PARTS;
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      const int k = (C::WAVES * i < C::BX) ? 0 : kind(wave, i);  // X copies are static
      const uint8_t* base = k == 0 ? xb : (k == 1 ? wb : sb);
      const void* s = static_cast<const void*>(base + (off[i] + (uint32_t)(kt * step(k))));
      lds_void* d = (lds_void*)(stage + dst(wave + C::WAVES * i));
      if (C::Q4 && k == 2)
        __builtin_amdgcn_global_load_lds(s, d, 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(s, d, 16, 0, 0);
    }
  }
  __device__ __forceinline__ void issue(const uint8_t* xb, const uint8_t* wb, const uint8_t* sb, int wave,
                                        uint8_t* stage, int kt) const {
    issue_part<0, 1>(xb, wb, sb, wave, stage, kt);
  }
};

__device__ __forceinline__ int xcd_tile(int bid, int nt) {
  const int q = nt >> 3, rem = nt & 7;
  const int x = bid & 7, loc = bid >> 3;
  return x * q + (x < rem ? x : rem) + loc;
}

// tile t -> (tm, tn): groups of gm tile rows, column-major inside a group, so
// that the run of tiles one XCD receives covers a compact block of about
// gm x (run / gm) tiles (few distinct X and W panels through its L2)
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int per_group = gm * tiles_n;
  const int grp = t / per_group;
  const int first = grp * gm;
  const int rows = min(gm, tiles_m - first);
  const int r = t - grp * per_group;
  tm = first + r % rows;
  tn = r / rows;
}

// Row bands: XCD x (consecutive workgroup ids go round-robin to the 8 XCDs)
// takes tile rows [x R, (x + 1) R), R = tiles_m / 8, across every tile
// column, walked column-major, so that each round of its CUs covers R rows x
// (CUs / R) columns and the band's X panels stay in its L2 for every round
// (used when tiles_m is a multiple of 8 and X is the larger operand).
__device__ __forceinline__ void band_tile(int bid, int tiles_m, int& tm, int& tn) {
  const int R = tiles_m >> 3, x = bid & 7, loc = bid >> 3;
  tm = x * R + loc % R;
  tn = loc / R;
}

// GELU with erf from Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error of erf| <= 1.5e-7): for z >= 0,
// 1 - erf(z) = t P(t) exp(-z^2), t = 1 / (1 + p z), P of degree 4.  With
// z = |x| / sqrt 2 and E = 0.5 |x| t P(t) exp(-x^2 / 2), x Phi(x) is x - E for
// x >= 0 and -E for x < 0, i.e. max(x, 0) - E in both cases (14 VALU
// instructions where x (1 + erf) / 2 took 16; the 1/2 rides in the exponent).
__device__ __forceinline__ float gelu_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(ax, 0.3275911f * 0.70710678118654752f, 1.0f));
  float P = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
  P = __builtin_fmaf(t, P, 1.421413741f);
  P = __builtin_fmaf(t, P, -0.284496736f);
  P = __builtin_fmaf(t, P, 0.254829592f);
  const float q = x * -0.72134752044448170f;                               // -log2(e) / 2
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(q, x, -1.0f));    // exp(-x^2 / 2) / 2
  return __builtin_fmaf(-((ax * t) * P), e, fmaxf(x, 0.0f));
}

__device__ __forceinline__ void unpack_h8(uint4 raw, float f[8]) {
  const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f[2 * r] = h2f((uint16_t)(w4[r] & 0xFFFFu));
    f[2 * r + 1] = h2f((uint16_t)(w4[r] >> 16));
  }
}

// 8 packed two's-complement nibbles (value e in bits 4e..4e+3) -> 8 x
// fp16(q * s).  With the sign bit flipped a nibble is q + 8; the fp16 with
// bit pattern 0x6400 | (q + 8) is 1024 + q + 8, so subtracting 1032 gives q
// exactly, and the product with s is rounded once.  (Placing small integers
// under a fixed fp16 exponent and subtracting the offset is the
// integer-to-half conversion without conversion instructions described by
// Kim et al., "Who Says Elephants Can't Run: Bringing Large Scale MoE Models
// into Cloud Scale Production", 2022.)  v_perm_b32 pairs value 2i (byte i of
// the even nibbles) with value 2i + 1 (byte i of the odd ones) as the two
// halves of register i.
__device__ __forceinline__ v4i dequant8(uint32_t packed, v2h s2) {
  const uint32_t w = packed ^ 0x88888888u;
  const uint32_t ev = w & 0x0F0F0F0Fu;
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
  const v2h off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  v4i out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // selector bytes: ev byte i, zero, od byte i, zero
    const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
    const uint32_t h = __builtin_amdgcn_perm(od, ev, sel) | 0x64006400u;
    const v2h q = __builtin_bit_cast(v2h, h) + off;
    out[i] = __builtin_bit_cast(int, q * s2);
  }
  return out;
}

// 8 int8 weights -> 8 fp16, exact: with the sign bit flipped a byte is
// q + 128; placed under the fp16 exponent byte 0x64 it reads 1024 + q + 128,
// and subtracting 1152 gives q.  v_perm_b32 interleaves two bytes of the
// data with two 0x64 bytes per register.
__device__ __forceinline__ v4i widen_i8x8(uint2 w) {
  const uint32_t a = w.x ^ 0x80808080u, b = w.y ^ 0x80808080u;
  const v2h off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint32_t e = 0x64646464u;
  const uint32_t h[4] = {__builtin_amdgcn_perm(e, a, 0x04010400u), __builtin_amdgcn_perm(e, a, 0x04030402u),
                         __builtin_amdgcn_perm(e, b, 0x04010400u), __builtin_amdgcn_perm(e, b, 0x04030402u)};
  v4i out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, h[i]) + off);
  return out;
}

template <class C>
using AccT = typename std::conditional<C::INT, v16i, v16f>::type;

template <class C>
__device__ __forceinline__ void mfma_slice(AccT<C> (&acc)[C::NJ][C::MI], const v4i (&xf)[C::MI],
                                           const v4i (&wf)[C::NJ]) {
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      if constexpr (C::INT) {
        acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j], xf[i], acc[j][i], 0, 0, 0);
      } else {
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, wf[j]),
                                                           __builtin_bit_cast(v8h, xf[i]), acc[j][i], 0, 0, 0);
      }
    }
}

// Operand fragments of K slice ks from a stage.  X (and int8 / fp16 W): 16
// swizzled bytes per lane.  Q4 W: slice ks covers values 16 ks .. 16 ks + 15
// of the stage, i.e. bytes 8 (ks % 2) .. 8 (ks % 2) + 7 of group ks / 2; lane
// l takes the 4 bytes at 4 (l / 32) of those and its row's scale.  Q8W W
// (64-byte rows, chunk c at slot c ^ q8w_swz(row)): slice ks is chunk ks; lane l
// takes its 8 bytes at 8 (l / 32) and widens them to fp16.
template <class C>
struct Frags {
  int off[C::KS];  // lane's byte offset of slice ks in a 32-row block (8-row blocks of 128 B)
  int qoff;        // Q4: lane's packed word in a 32-row block
  int soff;        // Q4: lane's scale pair in the stage's scale area

  __device__ __forceinline__ void init(int lane, int wn) {
    const int lr = lane & 31;
    const int lane_off = (lr >> 3) * BLK + (lr & 7) * KB;
    const int g_l = swz(lr);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) off[ks] = lane_off + (((2 * ks + (lane >> 5)) ^ g_l) << 4);
    qoff = lr * 16 + (lane >> 5) * 4;
    soff = (wn * C::WN + lr) * 4;
  }
  __device__ __forceinline__ void read(const uint8_t* stage, int wm, int wn, int ks, v4i (&xf)[C::MI],
                                       v4i (&wf)[C::NJ]) const {
    constexpr int B32 = 4 * BLK;  // 32 rows of 8-row blocks
    const uint8_t* sx = stage + wm * C::MI * B32;
#pragma unroll
    for (int i = 0; i < C::MI; ++i) xf[i] = *reinterpret_cast<const v4i*>(sx + i * B32 + off[ks]);
    if constexpr (C::Q8W) {
      const int lr = threadIdx.x & 31, h = (threadIdx.x >> 5) & 1;
      const uint8_t* sw = stage + C::W_OFF + (wn * C::WN + lr) * 64 + ((ks ^ q8w_swz(lr)) << 4) + 8 * h;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) wf[j] = widen_i8x8(*reinterpret_cast<const uint2*>(sw + j * 32 * 64));
    } else if constexpr (!C::Q4) {
      const uint8_t* sw = stage + C::W_OFF + wn * C::NJ * B32;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) wf[j] = *reinterpret_cast<const v4i*>(sw + j * B32 + off[ks]);
    } else {
      const uint8_t* sw = stage + C::W_OFF + wn * C::NJ * BLK + (ks >> 1) * 512 + (ks & 1) * 8 + qoff;
      const uint8_t* ss = stage + C::S_OFF + soff + (ks >> 1) * 2;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const uint32_t packed = *reinterpret_cast<const uint32_t*>(sw + j * BLK);
        const _Float16 s = *reinterpret_cast<const _Float16*>(ss + j * 32 * 4);
        wf[j] = dequant8(packed, v2h{s, s});
      }
    }
  }
};

// LDS of config C with KS stage rings: the rings, then (overlapping them)
// the epilogue staging, then the epilogue scalars
template <class C, int KS>
struct KsLds {
  static constexpr int RINGS = KS * C::LDS;
  static constexpr int SC_OFF = RINGS > C::EPI_LDS ? RINGS : C::EPI_LDS;
  static constexpr int TOTAL = SC_OFF + C::SC_PAD * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// P > 0: P more waves (after the C::WAVES MFMA waves) issue every stage copy,
// so the MFMA waves never stall on copy issue; the copies of a stage are
// still issued one stage ahead and made visible by the stage barrier.
// KS = 2 (int8, no producers): two sets of C::WAVES waves split K in halves,
// each with its own stage ring (both meet at every stage barrier); at the
// end the second set's int32 accumulators are added to the first set's
// (exact: the result does not depend on the split), which runs the
// epilogue.  Each wave's dependent chain through the stages is halved, for
// the short launches of small tiles where that chain sets the time.
// bands != 0: row-band tile order (gm ignored), see band_tile.
template <class C, int EPI, int P = 0, int KS = 1>
__global__ __launch_bounds__(C::THREADS * KS + 64 * P, 1) void gemm_dma_kernel(GemmArgs g, int tiles_n, int gm,
                                                                               int bands) {
  static_assert(KS == 1 || (KS == 2 && P == 0 && C::INT), "K halves: int8, no producer waves");
  using L = KsLds<C, KS>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = KS > 1 ? wave_all / C::WAVES : 0;  // K half of this wave
  const int wave = KS > 1 ? wave_all % C::WAVES : wave_all;
  uint8_t* const ring = smem + kh * C::LDS;  // this half's stage ring
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const uint8_t* const xb = static_cast<const uint8_t*>(g.A);  // operand bases
  const uint8_t* const wb = static_cast<const uint8_t*>(g.B);
  const uint8_t* const sb = reinterpret_cast<const uint8_t*>(g.b_scale);
  const int nt = gridDim.x;
  int tm, tn;
  if (bands) band_tile(blockIdx.x, nt / tiles_n, tm, tn);
  else tile_coords(xcd_tile(blockIdx.x, nt), nt / tiles_n, tiles_n, gm, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  constexpr bool INT = C::INT;
  const int nk = g.K * (INT ? 1 : 2) / KB / KS;  // stages of this wave's K range
  const int kb0 = kh * nk;                        // its first stage

  if constexpr (P > 0) {
    if (wave >= C::WAVES) {  // producer: stage copies one stage ahead, one barrier per stage
      using PC = ProducerCfg<C, P>;
      Loader<PC> pl;
      const int pw = wave - C::WAVES;
      pl.init(g, m0, n0, pw, lane);
      for (int s = 0; s < C::STAGES - 1; ++s)
        if (s < nk) pl.issue(xb, wb, sb, pw, smem + s * C::STAGE_BYTES, s);
      for (int kt = 0; kt < nk; ++kt) {
        wait_stages<PC::LOADS, C::STAGES - 2>(min(C::STAGES - 2, nk - 1 - kt));
        __builtin_amdgcn_s_barrier();
        const int kn = kt + C::STAGES - 1;
        if (kn < nk) pl.issue(xb, wb, sb, pw, smem + (kn % C::STAGES) * C::STAGE_BYTES, kn);
      }
      vm_wait<0>();
      __syncthreads();  // the barrier that opens the MFMA waves' epilogue
      return;
    }
  }

  Loader<C> ld;
  if constexpr (P == 0) ld.init(g, m0, n0, wave, lane);

  AccT<C> acc[C::NJ][C::MI];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

  // Epilogue through LDS, one wave-private region per wave: the raw
  // accumulators of PW columns at a time go to LDS in [row][col] order (row
  // stride padded by 16 bytes so the 32 rows written together fall on
  // distinct banks); then each lane takes 8 consecutive columns of a row,
  // for coalesced 16-byte loads and stores.  A pass issues all of its
  // residual loads before any arithmetic, so their latency is paid once.
  const EpiArgs& e = g.epi;
  constexpr int PW = C::PW, RS = C::RS;
  constexpr int LPR = PW / 8;       // lanes per row
  constexpr int RPI = 64 / LPR;     // rows per iteration
  constexpr int NIT = C::WM / RPI;  // iterations per pass
  constexpr bool RES = EPI == EPI_RES || EPI == EPI_GELU_RES;
  constexpr bool GELU = EPI == EPI_GELU || EPI == EPI_GELU_RES;
  const bool vec = (g.N & 7) == 0 && (e.ldy & 7) == 0 && (!RES || (e.ldr & 7) == 0) && !e.acc;
  const int cl = (lane % LPR) * 8;
  const int rl0 = lane / LPR;
  const int rbase = m0 + wm * C::WM;
  const int lr = lane & 31;
  // residual of a pass, double buffered: pass p + 1's loads are issued before
  // pass p is processed, so their latency hides behind it
  constexpr int NPASS = C::WN / PW;
  constexpr int RBUF = RES ? (NPASS > 1 ? 2 : 1) : 1;
  uint4 resv[RBUF][RES ? NIT : 1];
  auto load_res = [&](int p) {
    if constexpr (RES) {
      const int col = n0 + wn * C::WN + p * PW + cl;
      const int left = g.N - col;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int row = min(rbase + it * RPI + rl0, g.M - 1);
        const uint16_t* rp = e.residual + (int64_t)row * e.ldr + min(col, g.N - 1);
        if (vec && left >= 8) {
          resv[p % RBUF][it] = *reinterpret_cast<const uint4*>(rp);
        } else {
          uint16_t h[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) h[r] = r < left ? rp[r] : (uint16_t)0;
          resv[p % RBUF][it] =
              make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        }
      }
    }
  };
  // Residual of the first epilogue pass, loaded before any copy when the
  // registers allow (small tiles): its latency then hides behind the main
  // loop instead of opening the epilogue.  Issued ahead of every stage copy,
  // these loads are older than all of them, so the stage waits stay exact.
  constexpr bool EARLY_RES = RES && NIT <= 4;
  if constexpr (EARLY_RES) {
    if (kh == 0) load_res(0);
  }

  // the epilogue's per-row / per-column scalars travel to LDS first; they
  // are older than every stage copy, so the stage waits cover them too
  if (kh == 0) {
    float* sc = reinterpret_cast<float*>(smem + L::SC_OFF);
#pragma unroll
    for (int i = wave; i < C::SC_LOADS; i += C::WAVES) {
      const int q = i * 64 + lane;  // x_scale rows, then w_scale columns, then bias columns, then padding
      const float* src;
      if (q < C::BM) src = e.x_scale ? e.x_scale + min(m0 + q, g.M - 1) : nullptr;
      else if (q < C::BM + C::BN) src = e.w_scale ? e.w_scale + min(n0 + q - C::BM, g.N - 1) : nullptr;
      else if (q < C::SC_N) src = e.bias ? e.bias + min(n0 + q - C::BM - C::BN, g.N - 1) : nullptr;
      else src = nullptr;
      if (src) {  // lane l of copy i lands at sc[64 i + l]; lanes without a source write the default
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(sc + i * 64), 4, 0, 0);
      } else {
        sc[q] = (q >= C::BM + C::BN) ? 0.0f : 1.0f;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (P == 0 && s < nk) ld.issue(xb, wb, sb, wave, ring + s * C::STAGE_BYTES, kb0 + s);

  Frags<C> fr;
  fr.init(lane, wn);

  // Per stage: wait for its copies, barrier, then four 32-byte K slices.  A
  // quarter of the next stage's copies is issued before each slice's MFMAs
  // (a long burst of copy issues stalls the wave while the matrix pipe
  // idles), and the fragments of slice s + 1 are read during slice s.
  for (int kt = 0; kt < nk; ++kt) {
    if constexpr (P == 0) wait_stages<C::LOADS, C::STAGES - 2>(min(C::STAGES - 2, nk - 1 - kt));
    __builtin_amdgcn_s_barrier();
    const int kn = kt + C::STAGES - 1;
    const bool more = kn < nk;
    uint8_t* const snext = ring + (kn % C::STAGES) * C::STAGE_BYTES;
    const uint8_t* const stage = ring + (kt % C::STAGES) * C::STAGE_BYTES;
    v4i xf[2][C::MI], wf[2][C::NJ];
    fr.read(stage, wm, wn, 0, xf[0], wf[0]);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (P == 0 && more) {
        if (ks == 0) ld.template issue_part<0, C::KS>(xb, wb, sb, wave, snext, kb0 + kn);
        if (ks == 1) ld.template issue_part<1, C::KS>(xb, wb, sb, wave, snext, kb0 + kn);
        if (ks == 2) ld.template issue_part<2, C::KS>(xb, wb, sb, wave, snext, kb0 + kn);
        if (ks == 3) ld.template issue_part<3, C::KS>(xb, wb, sb, wave, snext, kb0 + kn);
      }
      if (ks + 1 < C::KS) fr.read(stage, wm, wn, ks + 1, xf[(ks + 1) & 1], wf[(ks + 1) & 1]);
      mfma_slice<C>(acc, xf[ks & 1], wf[ks & 1]);
    }
  }

  // with producers, this wave's own loads are only the epilogue scalars
  if constexpr (P > 0) vm_wait<0>();
  if constexpr (KS > 1) {
    // the second half's accumulators through LDS (the rings are free once
    // every wave is past its last stage): value r of MFMA block (j, i) of
    // lane l of wave w at int (((w * NJ + j) * MI + i) * 16 + r) * 64 + l
    __syncthreads();
    int* xch = reinterpret_cast<int*>(smem);
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) xch[(((wave * C::NJ + j) * C::MI + i) * 16 + r) * 64 + lane] = acc[j][i][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][i][r] += xch[(((wave * C::NJ + j) * C::MI + i) * 16 + r) * 64 + lane];
    }
  }
  // Epilogue (the residual of pass 0 was loaded up front for the small tiles)
  if constexpr (!EARLY_RES) {
    if (kh == 0) load_res(0);
  }
  __syncthreads();  // every wave is done with the operand stages; the scalars have landed
  if (KS > 1 && kh != 0) return;
  uint32_t* reg = reinterpret_cast<uint32_t*>(smem) + wave * (C::WM * (RS + 1));
  const float* sc = reinterpret_cast<const float*>(smem + L::SC_OFF);
#pragma unroll
  for (int p = 0; p < C::WN / PW; ++p) {
    if (p + 1 < NPASS) load_res(p + 1);
#pragma unroll
    for (int jj = 0; jj < PW / 32; ++jj) {
      const int j = p * (PW / 32) + jj;
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        // bit-cast the whole vector (a cast of one element lvalue reads element 0)
        const v16i av = __builtin_bit_cast(v16i, acc[j][i]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<v4i*>(reg + (i * 32 + lr) * RS + jj * 32 + q * 8 + (lane >> 5) * 4) =
              v4i{av[q * 4], av[q * 4 + 1], av[q * 4 + 2], av[q * 4 + 3]};
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int ct = wn * C::WN + p * PW + cl;  // column within the tile
    const int col = n0 + ct;
    const int left = g.N - col;
    if (left > 0) {
      float ws[8], bs[8];
      {
        const float4 w0 = *reinterpret_cast<const float4*>(sc + C::BM + ct);
        const float4 w1 = *reinterpret_cast<const float4*>(sc + C::BM + ct + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(sc + C::BM + C::BN + ct);
        const float4 b1 = *reinterpret_cast<const float4*>(sc + C::BM + C::BN + ct + 4);
        ws[0] = w0.x; ws[1] = w0.y; ws[2] = w0.z; ws[3] = w0.w; ws[4] = w1.x; ws[5] = w1.y; ws[6] = w1.z; ws[7] = w1.w;
        bs[0] = b0.x; bs[1] = b0.y; bs[2] = b0.z; bs[3] = b0.w; bs[4] = b1.x; bs[5] = b1.y; bs[6] = b1.z; bs[7] = b1.w;
      }
      const bool full = vec && left >= 8;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int rl = it * RPI + rl0;
        const int row = rbase + rl;
        if (row >= g.M) continue;
        const uint4 a0 = *reinterpret_cast<const uint4*>(reg + rl * RS + cl);
        const uint4 a1 = *reinterpret_cast<const uint4*>(reg + rl * RS + cl + 4);
        const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        if constexpr (INT) {
          if (e.acc) {
            int32_t* ap = e.acc + (int64_t)row * g.N + col;
            for (int r = 0; r < 8 && r < left; ++r) ap[r] = (int32_t)a[r];
          }
        }
        if (!e.y) continue;
        const float xs = sc[wm * C::WM + rl];
        float res[8];
        if constexpr (RES) unpack_h8(resv[p % RBUF][it], res);
        uint32_t o[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float x;
          if constexpr (INT) x = __builtin_fmaf((float)(int32_t)a[r] * xs, ws[r], bs[r]);
          else if constexpr (C::Q8W) x = __builtin_fmaf(__builtin_bit_cast(float, a[r]), ws[r], bs[r]);
          else x = __builtin_bit_cast(float, a[r]) + bs[r];
          if constexpr (GELU) x = gelu_as(x);
          if constexpr (RES) x += res[r];
          o[r] = f2h(x);
        }
        uint16_t* yp = e.y + (int64_t)row * e.ldy + col;
        if (full) {
          *reinterpret_cast<uint4*>(yp) = make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                                                     o[6] | (o[7] << 16));
        } else {
          for (int r = 0; r < 8 && r < left; ++r) yp[r] = (uint16_t)o[r];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <class C, int EPI, int P, int KS = 1>
void launch_cfg(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + C::BM - 1) / C::BM, tn = (g.N + C::BN - 1) / C::BN;
  // large tiles over an X larger than W: row bands per XCD (band_tile);
  // otherwise each XCD gets about tiles / 8 consecutive tiles, a block of
  // about sqrt(run) x sqrt(run) tiles, as tall as needed to fit tn columns
  const int bands = (C::BM == 256 && tm % 8 == 0 && g.N <= g.M) ? 1 : 0;
  const int run = (tm * tn + 7) / 8;
  int gm = (int)(sqrtf((float)run) + 0.5f);
  gm = std::max(gm, (run + tn - 1) / tn);
  gm = std::max(1, std::min(gm, tm));
  hipLaunchKernelGGL((gemm_dma_kernel<C, EPI, P, KS>), dim3((unsigned)(tm * tn)), dim3(C::THREADS * KS + 64 * P),
                     (KsLds<C, KS>::TOTAL), st, g, tn, gm, bands);
}

// P producer waves for the epilogues without a residual, PR with one; KS
// K halves
template <class C, int P = 0, int PR = P, int KS = 1>
void launch_epi(const GemmArgs& g, hipStream_t st) {
  const bool res = g.epi.residual != nullptr, gelu = g.epi.act == 1;
  if (gelu && res) launch_cfg<C, EPI_GELU_RES, PR, KS>(g, st);
  else if (gelu) launch_cfg<C, EPI_GELU, P, KS>(g, st);
  else if (res) launch_cfg<C, EPI_RES, PR, KS>(g, st);
  else launch_cfg<C, EPI_PLAIN, P, KS>(g, st);
}

template <class C, int P = 0, int PR = P, int KS = 1>
void prep_cfg() {
  const void* k[4] = {reinterpret_cast<const void*>(&gemm_dma_kernel<C, EPI_PLAIN, P, KS>),
                      reinterpret_cast<const void*>(&gemm_dma_kernel<C, EPI_RES, PR, KS>),
                      reinterpret_cast<const void*>(&gemm_dma_kernel<C, EPI_GELU, P, KS>),
                      reinterpret_cast<const void*>(&gemm_dma_kernel<C, EPI_GELU_RES, PR, KS>)};
  for (const void* f : k)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, KsLds<C, KS>::TOTAL);
}

// tile configurations per mode (BM, BN, stages, waves along N, waves along
// M): the 256 x 256 tile runs 8 waves, two per SIMD, 128 x 64 each (one wave
// per SIMD with 128 x 128 each reads less from LDS but measured 4-13% slower
// on every serving shape: the second wave covers the first one's LDS and
// copy-issue stalls, the prologue and the epilogue, and overlaps the 4-bit
// dequantization with the MFMAs); a Q4 stage is smaller, so its 256 x 256
// tile keeps three stages in flight.  The 256 x 192 tile (8 waves of
// 64 x 96; int8, fp16 and 8-bit weight-only operands) exists for wave
// quantization: widths that are multiples of 192 can leave a partial last
// round of 256 x 256 tiles (N = 1536 at M = 8192 fills 192 of 256 CUs,
// N = 4608 runs 2.25 rounds) that 256 x 192 tiles fill exactly.  The
// smaller tiles serve short launches (M of a few hundred rows), where the
// launch is latency-bound: four stages measured 3-13 % faster than five
// (128 x 64) and eight (64 x 64) stages on those shapes in every operand
// mode, K = 4096 included; three or fewer stages, and more, were slower
template <int MODE>
struct Tiles {
  using T256 = Cfg<256, 256, (MODE == M_Q4 || MODE == M_Q8W) ? 3 : 2, MODE, 4>;
  using T256x192 = Cfg<256, 192, MODE == M_Q8W ? 3 : 2, MODE, 2, 4>;
  using T128 = Cfg<128, 128, 4, MODE>;
  using T128x64 = Cfg<128, 64, 4, MODE>;
  using T64 = Cfg<64, 64, 4, MODE>;
  using T32x64 = Cfg<32, 64, 4, MODE, 2, 1>;  // two waves of 32 x 32
  // producer waves of the int8 large tiles (12 waves, 3 per SIMD); the
  // 256 x 256 tile takes them only without a residual epilogue (with one its
  // MFMA waves would not fit 3 per SIMD without spilling)
  static constexpr int P192 = MODE == M_I8 ? 4 : 0;
  static constexpr int P256 = MODE == M_I8 ? 4 : 0;
};

int64_t tiles(int M, int N, int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

// compute units of the current device (one query per process; one device
// kind per process is assumed)
int64_t device_cus() {
  static int cus = 0;
  if (cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      return 256;
  }
  return cus;
}

template <int MODE>
void dispatch(const GemmArgs& g, hipStream_t st) {
  // largest tile that still fills most of the CUs with one workgroup each
  // (one round of 192 large tiles beats three rounds of smaller ones)
  constexpr int64_t FILL = 180;
  using T = Tiles<MODE>;
  if (tiles(g.M, g.N, 256, 256) >= FILL) {
    // among the large tiles, the one with the least tile area over whole
    // rounds of one workgroup per CU, 256 x 192 weighted by 9/8 for its
    // costlier operations (more LDS reads per MFMA, ragged column tiles when
    // N is not a multiple of 192): it wins where a partial last round of
    // 256 x 256 tiles idles many CUs (serving shapes at M = 8192: N = 1536
    // and 4608), not on long launches of many rounds (M = 37k, N = 4096
    // measured 3 % slower with it)
    if constexpr (MODE != M_Q4) {
      const int64_t cus = device_cus();
      const int64_t r256 = (tiles(g.M, g.N, 256, 256) + cus - 1) / cus;
      const int64_t r192 = (tiles(g.M, g.N, 256, 192) + cus - 1) / cus;
      if (r192 * 192 * 9 < r256 * 256 * 8) {
        launch_epi<typename T::T256x192, T::P192>(g, st);
        return;
      }
    }
    launch_epi<typename T::T256, T::P256, 0>(g, st);
  } else if (tiles(g.M, g.N, 128, 128) >= FILL) {
    launch_epi<typename T::T128>(g, st);
  } else if (tiles(g.M, g.N, 128, 64) >= FILL) {
    launch_epi<typename T::T128x64>(g, st);
  } else {
    // int8 launches of fewer 64 x 64 tiles than CUs (the 512-row step's
    // hidden-width projections) take 32 x 64 tiles: twice the workgroups
    if constexpr (MODE == M_I8) {
      if (tiles(g.M, g.N, 64, 64) < device_cus()) {
        // with K in two halves of whole stages: the 512-row step's o, q, ox
        // (5.35 -> 4.7 us) and down (K = 4096, 10.7 -> 8.1 us), mid-size loop
        // 851 -> 907 steps/s (MI355X).  The 128 x 64 tiles of its qkv and up
        // with split K (three-stage rings) ran faster alone but slowed the
        // loop, so they keep one ring.
        if ((g.K / KB) % 2 == 0 && g.K / KB >= 4) launch_epi<typename T::T32x64, 0, 0, 2>(g, st);
        else launch_epi<typename T::T32x64>(g, st);
        return;
      }
    }
    launch_epi<typename T::T64>(g, st);
  }
}

template <int MODE>
void prep_mode() {
  using T = Tiles<MODE>;
  prep_cfg<typename T::T256, T::P256, 0>();
  if constexpr (MODE != M_Q4) prep_cfg<typename T::T256x192, T::P192>();
  prep_cfg<typename T::T128>();
  prep_cfg<typename T::T128x64>();
  prep_cfg<typename T::T64>();
  if constexpr (MODE == M_I8) {
    prep_cfg<typename T::T32x64>();
    prep_cfg<typename T::T32x64, 0, 0, 2>();
  }
}

}  // namespace

void gemm_dma_prepare() {
  prep_mode<M_I8>();
  prep_mode<M_F16>();
  prep_mode<M_Q4>();
  prep_mode<M_Q8W>();
}

bool gemm_dma_applicable(int akind, int bkind, const GemmArgs& g) {
  const bool i8 = akind == A_I8 && bkind == B_I8;
  const bool f16 = akind == A_F16 && bkind == B_F16;
  const bool q4 = akind == A_F16 && bkind == B_Q4;
  const bool q8w = akind == A_F16 && bkind == B_I8;
  if (!(i8 || f16 || q4 || q8w)) return false;
  const int64_t kb = (int64_t)g.K * (i8 ? 1 : 2);
  if (kb % KB != 0) return false;  // whole 128-byte X stages (Q4: whole pairs of groups)
  const int64_t ldb = (int64_t)g.lda * (i8 ? 1 : 2);
  if (ldb % 16 != 0) return false;
  if ((reinterpret_cast<uintptr_t>(g.A) & 15) || (reinterpret_cast<uintptr_t>(g.B) & 15)) return false;
  if (q4 && (reinterpret_cast<uintptr_t>(g.b_scale) & 3)) return false;
  // copy sources are 32-bit byte offsets from the operand base pointers
  const int64_t wbytes = (int64_t)g.N * (q4 ? g.K / 2 : (q8w ? g.K : kb));
  if ((int64_t)g.M * ldb >= ((int64_t)1 << 32) || wbytes >= ((int64_t)1 << 32)) return false;
  return g.M > 0 && g.N > 0;
}

void launch_gemm_dma(int akind, int bkind, const GemmArgs& g, hipStream_t st) {
  if (akind == A_I8) dispatch<M_I8>(g, st);
  else if (bkind == B_Q4) dispatch<M_Q4>(g, st);
  else if (bkind == B_I8) dispatch<M_Q8W>(g, st);
  else dispatch<M_F16>(g, st);
}

}  // namespace ald
