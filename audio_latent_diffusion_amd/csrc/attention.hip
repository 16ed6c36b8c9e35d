// Flash-style non-causal attention, head_dim 64, fp16 in/out, fp32 online
// softmax, on v_mfma_f32_16x16x32_f16.  Dense and packed varlen sequences.
//
// Workgroup = NW waves; wave w owns 16 * QW queries of one (sequence, head).
// Keys and values stream through LDS in tiles of 64 rows, copied straight
// from global memory by global_load_lds_dwordx4 (each instruction fills 8 rows
// x 128 bytes; a lane picks which 16-byte chunk of its row it fetches, which
// gives the swizzles below), in a ring of three stages: tiles t + 1 and t + 2
// are in flight while tile t is consumed.
//
// Scores are computed transposed, S^T = K Q^T: the K fragment is the MFMA row
// operand (lane l: key l % 16, 8 dims at 8 (l / 16)), Q stays in registers as
// the column operand.  The accumulator of lane l then holds query l % 16 and
// keys 4 (l / 16) + r of each 16-key block, which is the column-operand
// layout the second product O^T = V^T P^T needs once the 8 K positions of a
// lane are taken as keys 32 c + 4 (l / 16) + {0..3} and 32 c + 16 + 4 (l / 16)
// + {0..3} (any pairing of K positions is exact as long as both operands use
// it), so P never leaves the registers.
//
// V stays row-major in LDS ([key][dim], as loaded) and each V^T fragment is
// two LDS transpose reads (ds_read_b64_tr_b16): within a 16-lane group, slot
// k of lane j receives element j % 4 of the 8 bytes addressed by lane
// 4 k + j / 4, so lanes 4 k + q point at key k, dims 4 q .. 4 q + 3 and lane j
// gets dim j of four consecutive keys.
//
// LDS swizzles (16-byte chunk c of row r stored at slot c ^ f(r)):
//   K: f(r) = (r & 7) ^ ((r >> 3) & 1): the 16 rows of one fragment read,
//      same chunk, fall on distinct banks per 8-lane phase and per 256-byte
//      (64-bank) period;
//   V: f(r) = 2 ((r & 3) ^ ((r >> 2) & 1)): the four keys of one transpose
//      read land in four different 32-byte bank groups, and the 8 keys two
//      adjacent 16-lane groups read (rows 4 g + tk, g = 0, 1) cover the 256
//      bytes of a 64-bank period once.
//
// Softmax in base 2: p = 2^(c s + r) with r = -c m per row, one FMA and one
// v_exp_f32.  The first tile sets m to the row maximum (reduced over the 4
// lanes that share a query with two lane-swap instructions); the reference
// moves only when an exponent c s + r would pass 8 (so p < 256, and the output
// rescale is rare), which later tiles detect with a lane-local maximum.  The
// row sum of the fp16 weights comes out of the MFMA against a block of ones.
#include "common.h"
#include "kernels.h"

namespace ald {

constexpr int KT = 64;                   // keys per tile
constexpr int HD = 64;                   // head dim
constexpr int TILE_BYTES = KT * HD * 2;  // one K or V tile (8 KB)
constexpr int ASTAGES = 3;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int kswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int vswz(int r) { return 2 * ((r & 3) ^ ((r >> 2) & 1)); }

// maximum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (one query's keys).
// v_permlane16_swap / v_permlane32_swap on two copies of v leave v of the
// partner lane (xor 16, resp. xor 32) in one register and the lane's own
// value in the other.  The swaps are inline assembly: through the compiler
// builtin the float maximum of the two results was compiled as the maximum
// of the first with itself (the generated code compared only one lane in
// four, so the row maximum covered a quarter of the row's keys).  The nop
// covers the VALU-write-to-permlane-read hazard.
__device__ __forceinline__ float max_over_query_lanes(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = fmaxf(a, b);
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// s_waitcnt vmcnt(N)
template <int N>
__device__ __forceinline__ void attn_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// EARLYQ: the tile copies are issued while this wave's Q loads are still in
// flight (vector memory loads complete in issue order, so the wait for tile
// 0 also covers Q); it pays off when there are only one or two key tiles
template <int QW, int NW, bool EARLYQ>
__global__ __launch_bounds__(64 * NW, 3) void attn_kernel(AttnArgs a) {
  constexpr int RPW = KT / NW;  // tile rows each wave copies
  constexpr int CI = RPW / 8;   // copy instructions per wave and operand
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];  // ASTAGES x (K tile, V tile)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs round-robin in dispatch order (x, then
  // y, then z).  On grids of at least 1024 workgroups the ids are remapped so
  // that each XCD runs one contiguous range of (sequence, head, query block)
  // tasks: the query blocks of one (sequence, head) then run together on one
  // XCD and share its L2 for their K and V (serving self-attention 46 -> 40
  // us, cross-attention 22 -> 19.4 us; on a single-round grid it cost 5 %).
  int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  {
    const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
    if (n >= 1024 && (n & 7) == 0) {
      const int bid = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
      const int task = (bid & 7) * (n >> 3) + (bid >> 3);
      qb = task % nx;
      const int r = task / nx;
      h = r % ny;
      b = r / ny;
    }
  }
  const int q_begin = a.cu_q ? a.cu_q[b] : b * a.Sq;
  const int q_len = a.cu_q ? a.cu_q[b + 1] - q_begin : a.Sq;
  const int k_begin = a.cu_k ? a.cu_k[b] : b * a.Sk;
  const int k_len = a.cu_k ? a.cu_k[b + 1] - k_begin : a.Sk;
  const int QT = 16 * QW * NW;
  const int tq0 = qb * QT;
  if (tq0 >= q_len) return;  // whole workgroup exits together

  const int ql = lane & 15, g = lane >> 4;
  const int wq0 = tq0 + wave * 16 * QW;

  if (k_len <= 0) {  // no keys: zeros
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      int qi = wq0 + qb * 16 + ql;
      if (qi < q_len) {
        uint16_t* o = a.out + (int64_t)(q_begin + qi) * a.o_stride + h * HD + g * 16;
        st16(o, v4i{0, 0, 0, 0});
        st16(o + 8, v4i{0, 0, 0, 0});
      }
    }
    return;
  }

  // Q fragments (column operand): query ql, dims 32 c + 8 g .. + 8
  v8h qf[QW][2];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    int qi = wq0 + qb * 16 + ql;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (qi < q_len)
        qf[qb][c] = __builtin_bit_cast(v8h, ld16(a.q + (int64_t)(q_begin + qi) * a.q_stride + h * HD + 32 * c + 8 * g));
      else
        qf[qb][c] = __builtin_bit_cast(v8h, v4i{0, 0, 0, 0});
    }
  }

  // oacc[qb][0..3]: O^T blocks of 16 dims; oacc[qb][4]: the row sums of P,
  // accumulated by the same MFMA against a block of ones (every element of
  // that block is the sum of the fp16 weights over the keys, for the lane's
  // query), so the sum needs no VALU adds and no cross-lane reduction
  v4f oacc[QW][5];
  // cm_run[qb]: -c times the exponent reference of the lane's query (set by
  // the first tile), so a weight is 2^(c s + cm_run)
  float cm_run[QW];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    cm_run[qb] = 0.0f;
#pragma unroll
    for (int d = 0; d < 5; ++d) oacc[qb][d] = v4f{0, 0, 0, 0};
  }
  v8h ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;

  const int n_tiles = (k_len + KT - 1) / KT;
  // Tile copies: wave w fills rows RPW w .. RPW (w + 1) - 1 of the K tile
  // and of the V tile (CI instructions each); lane l of instruction i covers
  // row RPW w + 8 i + l / 8, slot l % 8.
  // Each lane's rows (r0 + 8 i) and chunks are fixed; a tile adds
  // t * 64 rows.  Only the last tile clamps rows past the end (they repeat a
  // valid key; their scores are masked).
  const int slot = lane & 7;
  const int r0 = wave * RPW + (lane >> 3);
  const int64_t rstep = (int64_t)KT * a.kv_stride;
  const uint16_t* ksrc[CI];
  const uint16_t* vsrc[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int r = r0 + 8 * i;
    const int64_t ro = (int64_t)(k_begin + r) * a.kv_stride + h * HD;
    ksrc[i] = a.k + ro + 8 * (slot ^ kswz(r));
    vsrc[i] = a.v + ro + 8 * (slot ^ vswz(r));
  }
  auto issue_tile = [&](int t, int s) {
    uint8_t* base = smem + s * 2 * TILE_BYTES + (wave * RPW) * 128;
    const bool whole = (t + 1) * KT <= k_len;  // uniform
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      int64_t off = (int64_t)t * rstep;
      if (!whole) {
        const int r = r0 + 8 * i;
        off = (int64_t)(min(t * KT + r, k_len - 1) - r) * a.kv_stride;
      }
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(ksrc[i] + off), (lds_void_t*)(base + i * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(vsrc[i] + off),
                                       (lds_void_t*)(base + TILE_BYTES + i * 1024), 16, 0, 0);
    }
  };

  if constexpr (!EARLYQ) attn_vm_wait<0>();  // Q fragments in registers before any tile copy is in flight
  issue_tile(0, 0);
  if (n_tiles > 1) issue_tile(1, 1);

  // K fragment of lane (ql, g): row kb * 16 + ql, chunk 4 c + g (dims 32 c + 8 g)
  int koff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) koff[c] = ql * 128 + (((4 * c + g) ^ kswz(ql)) << 4);
  // V^T transpose reads: lane j = 4 tk + tq of group g points at key
  // 32 c + 16 h2 + 4 g + tk, dims 16 db + 4 tq .. + 3, i.e. chunk
  // 2 db + (tq >> 1) of that row.  The V swizzle depends on the row's low
  // three bits only (4 g + tk), so the byte offset is
  //   4096 c + 2048 h2 + (4 g + tk) 128 + 16 ((2 db + (tq >> 1)) ^ vswz(4 g + tk)) + 8 (tq & 1),
  // a per-lane part for each db plus an immediate for (c, h2).
  const int tk = ql >> 2, tq = ql & 3;
  int vlane[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vlane[db] = (4 * g + tk) * 128 + 16 * ((2 * db + (tq >> 1)) ^ vswz(4 * g + tk)) + 8 * (tq & 1);

  for (int t = 0; t < n_tiles; ++t) {
    // this wave's copies of tile t have landed (2 CI per tile; tile t + 1's are newer)
    if (t + 1 < n_tiles) attn_vm_wait<2 * CI>();
    else attn_vm_wait<0>();
    __builtin_amdgcn_s_barrier();  // every wave's copies visible; tile t - 1 fully consumed
    if (t + 2 < n_tiles) issue_tile(t + 2, (t + 2) % ASTAGES);
    const uint8_t* sK = smem + (t % ASTAGES) * 2 * TILE_BYTES;
    const uint8_t* sV = sK + TILE_BYTES;
    const int kbase = t * KT;

    v8h kf[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) kf[kb][c] = *reinterpret_cast<const v8h*>(sK + kb * 16 * 128 + koff[c]);
    // V^T fragments: 16 transpose reads.  They are issued as inline assembly
    // because the compiler, seeing an LDS read it cannot relate to the
    // direct-to-LDS copies, would wait for every copy in flight (the
    // prefetched tiles too); tile t's copies are already complete here.  One
    // lgkmcnt(0) tied to all results makes them available.
    const uint32_t vbase = (uint32_t)(uintptr_t)((lds_u8*)smem + (sV - smem));
    v2i vr[4][2][2];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint32_t va = vbase + vlane[db];
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vr[db][0][0]) : "v"(va) : "memory");
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(vr[db][0][1]) : "v"(va) : "memory");
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:4096" : "=v"(vr[db][1][0]) : "v"(va) : "memory");
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:6144" : "=v"(vr[db][1][1]) : "v"(va) : "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr[0][0][0]), "+v"(vr[0][0][1]), "+v"(vr[0][1][0]), "+v"(vr[0][1][1]), "+v"(vr[1][0][0]),
                   "+v"(vr[1][0][1]), "+v"(vr[1][1][0]), "+v"(vr[1][1][1]), "+v"(vr[2][0][0]), "+v"(vr[2][0][1]),
                   "+v"(vr[2][1][0]), "+v"(vr[2][1][1]), "+v"(vr[3][0][0]), "+v"(vr[3][0][1]), "+v"(vr[3][1][0]),
                   "+v"(vr[3][1][1])
                 :
                 : "memory");
    v8h vf[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        vf[db][c] = __builtin_bit_cast(v8h, v4i{vr[db][c][0][0], vr[db][c][0][1], vr[db][c][1][0], vr[db][c][1][1]});

    // scores of every query block first (independent MFMA chains the matrix
    // core works through while the softmax of the first block runs)
    v4f sc[QW][4];
#pragma unroll
    for (int qb = 0; qb < QW; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        v4f z = {0, 0, 0, 0};
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb][0], qf[qb][0], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb][1], qf[qb][1], z, 0, 0, 0);
        sc[qb][kb] = z;
      }
    // only the last tile can be partial: mask its keys past the end
    if (kbase + KT > k_len) {
#pragma unroll
      for (int qb = 0; qb < QW; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kbase + kb * 16 + g * 4 + r >= k_len) sc[qb][kb][r] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      // Online softmax in base 2 with a lazy reference: the weights are
      // p = 2^(c s + cm_run), and the reference moves only when a row's
      // exponent c s + cm_run would exceed 8 (p then stays below 256, exact
      // enough in fp16, and the output/sum rescale is rare after the first
      // tile).  The first tile sets the reference to the row maximum.  Later
      // tiles form the exponents against the current reference, and only when
      // one of the wave's exceeds 8 take each row's maximum exponent (over its
      // 4 lanes) and shift the rows that moved, so a tile without a move needs
      // only a lane-local maximum.
      const float c = a.scale_log2;
      float ex[4][4];
      if (t == 0) {
        float mx = sc[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[qb][kb][r]);
        cm_run[qb] = -c * max_over_query_lanes(mx);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) ex[kb][r] = fmaf(sc[qb][kb][r], c, cm_run[qb]);
      } else {
        float emax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ex[kb][r] = fmaf(sc[qb][kb][r], c, cm_run[qb]);
            emax = fmaxf(emax, ex[kb][r]);
          }
        if (__any(emax > 8.0f)) {
          const float me = max_over_query_lanes(emax);
          const float shift = me > 8.0f ? me : 0.0f;  // 0 where the row does not move
          const float corr = __builtin_amdgcn_exp2f(-shift);
#pragma unroll
          for (int db = 0; db < 5; ++db) oacc[qb][db] *= corr;
          cm_run[qb] -= shift;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) ex[kb][r] -= shift;
        }
      }
      v8h pf[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) pf[kb >> 1][(kb & 1) * 4 + r] = (_Float16)__builtin_amdgcn_exp2f(ex[kb][r]);
#pragma unroll
      for (int db = 0; db < 5; ++db) {
        const v8h* vv = db < 4 ? vf[db] : nullptr;
        v4f o = oacc[qb][db];
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(db < 4 ? vv[0] : ones, pf[0], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(db < 4 ? vv[1] : ones, pf[1], o, 0, 0, 0);
        oacc[qb][db] = o;
      }
    }
  }

  // normalise and store: lane holds query ql, dims 16 db + 4 g + r
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    const float inv = 1.0f / oacc[qb][4][0];
    const int qi = wq0 + qb * 16 + ql;
    if (qi >= q_len) continue;
    uint16_t* o = a.out + (int64_t)(q_begin + qi) * a.o_stride + h * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint16_t hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = f2h(oacc[qb][db][r] * inv);
      *reinterpret_cast<uint64_t*>(o + db * 16 + g * 4) = *reinterpret_cast<uint64_t*>(hv);
    }
  }
}

constexpr int ATTN_LDS = ASTAGES * 2 * TILE_BYTES;

template <bool EARLYQ>
void launch_attn_q(const AttnArgs& a, int batch, int max_sq, hipStream_t st) {
  // two query blocks per wave when there is enough parallelism, else one;
  // grids that would not cover the 256 CUs with 4-wave workgroups take
  // 2-wave ones (32 queries each: twice the workgroups, the same per-query
  // arithmetic, 4 % faster on the 512-token CFG pair of the mid-size step)
  const int64_t wgs2 = (int64_t)((max_sq + 127) / 128) * a.n_heads * batch;
  const int64_t wgs1 = (int64_t)((max_sq + 63) / 64) * a.n_heads * batch;
  if (wgs2 >= 512) {
    dim3 grid((unsigned)((max_sq + 127) / 128), (unsigned)a.n_heads, (unsigned)batch);
    hipLaunchKernelGGL((attn_kernel<2, 4, EARLYQ>), grid, dim3(256), ATTN_LDS, st, a);
  } else if (wgs1 >= 256) {
    dim3 grid((unsigned)((max_sq + 63) / 64), (unsigned)a.n_heads, (unsigned)batch);
    hipLaunchKernelGGL((attn_kernel<1, 4, EARLYQ>), grid, dim3(256), ATTN_LDS, st, a);
  } else {
    dim3 grid((unsigned)((max_sq + 31) / 32), (unsigned)a.n_heads, (unsigned)batch);
    hipLaunchKernelGGL((attn_kernel<1, 2, EARLYQ>), grid, dim3(128), ATTN_LDS, st, a);
  }
}

void launch_attn(const AttnArgs& a, int batch, int max_sq, hipStream_t st) {
  if (batch <= 0 || max_sq <= 0) return;
  // dense key sets of at most two tiles (cross-attention to the text) overlap
  // the Q loads with the first tile copies: 19.4 -> 18.5 us on the serving
  // cross-attention; with more tiles it measured 1-3 % slower
  if (!a.cu_k && a.Sk <= 2 * KT) launch_attn_q<true>(a, batch, max_sq, st);
  else launch_attn_q<false>(a, batch, max_sq, st);
}

}  // namespace ald
