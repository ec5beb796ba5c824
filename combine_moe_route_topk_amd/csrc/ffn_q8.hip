// Grouped INT8 SwiGLU experts on CDNA4 MFMA (v_mfma_i32_32x32x32_i8).
//
// [XDS DeepSeek INT8 量化, P085: QMM with token-wise activation scale and
//  channel-wise weight scale, y_ij ~ s_i s^w_j sum_k q(x_ik) q(w_jk);
//  P088: gate and up projections fused into one kernel, expert weights INT8.
//  SwiGLU (down(silu(gate) * up)) is the textbook form; the pages do not spell it.]
//
// Four launches, all stream ordered, no host synchronization:
//   prep     per-slot m-tile counts and their prefix (the tile work list).
//   gateup   grouped GEMM over (slot, m-tile, n-tile): A = the slot's message
//            rows gathered from the dispatch buffer (int8 codes, K = H),
//            B = [128 gate rows | 128 up rows] of the slot's logical expert.
//            Epilogue: dequantize both, h = silu(g) * u, write h (fp32) and
//            the per-(row, n-tile) max |h| (no atomics).
//   requant  per row: amax = max of the partial maxima (exact), token-wise
//            INT8 of h -> hq, hs.
//   down     grouped GEMM: A = hq rows (dense, K = I), B = 128 rows of W_down;
//            epilogue: y = bf16((f32(acc) * hs) * s_down) into the dense
//            return rows.
// Tiles: 128 x 256 outputs per 256-thread block (four wavefronts of 128 x 64,
// each 4 x 2 MFMA 32x32 blocks), K steps of 64 bytes.  The A rows move
// global -> LDS by DMA into a ring of four stages, two steps ahead,
// XOR-swizzled rows.  The weights come pre-packed (moe_pack_expert_weights) in
// MFMA fragment order: each wavefront loads its own 64 columns of a K step
// straight into a ring of four register buffers, 4 KB as four contiguous 1 KB
// runs of whole cache lines, also two steps ahead of the MFMAs.  The work
// list is ordered slot-major, then groups of m-tiles (kGroupM), then n-tiles,
// then m inside the group, and blocks are remapped so that each XCD walks one
// contiguous stretch of it: the m-tiles of a group share every weight tile in
// that XCD's L2.  Weight tiles that only one block reads, and the outputs,
// move as non-temporal accesses so that they do not evict the shared tiles.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 256, BK = 64;
static_assert(BM == kFfnTileRows, "the scratch's m-tile table assumes 128-row tiles");
#define MOE_LDS __attribute__((address_space(3)))
constexpr int LDS_STRIDE = BK;  // bytes per LDS row
// LDS layout: 16-byte chunk c of tile row r sits at r * BK + 16 * (c ^ ((r >> 2) & 3)).
// A 16-byte LDS access serves 16 lanes per cycle across 64 banks; the XOR
// makes both access patterns conflict-free: the staging stores (16 lanes =
// four rows x four chunks) and the MFMA operand reads (16 lanes = sixteen rows,
// one chunk: rows r, r+4, r+8, r+12 would share banks without it).
// m-tiles per group: gate/up 4 (its A rows, 7 KB each, are the bigger
// operand to keep in L2: 1.4% faster than 8 on the Zipf layer), down 8
template <int MODE> constexpr int kGroupM = MODE == 0 /* GATEUP */ ? 4 : 8;
// LDS arena of a block (72 KB): the four A stages of the main loop, then the
// epilogue's staging tile
constexpr int kArena = 3 * (BM + BN) * BK;
// epilogue staging: fp32 rows of 128 + 8 values (the row scans' 16 lanes, 8
// rows x 2 float4 columns, land on distinct bank groups; a stride of 128 + 4
// spreads the staging writes further but conflicts there, and measured slower)
// and bf16 rows of 256 values + 32 bytes
constexpr int kStageStride = 128 + 8;
constexpr int kStageStrideB = 2 * 256 + 32;
static_assert(128 * kStageStride * 4 <= kArena, "staging fits the LDS arena");
static_assert(128 * kStageStrideB <= kArena, "staging fits the LDS arena");
constexpr int kXcds = 8;

// GATEUP, DOWN: the two INT8 expert projections.
enum Mode { GATEUP = 0, DOWN = 1 };

// ------------------------------------------------------------------ prep ---
// tiles [P + 1]: exclusive prefix of the per-slot m-tile counts, then the
// total; slot_of [bound]: the slot of each m-tile, so that a GEMM block finds
// its slot with one load instead of a search over the prefix (slot counts
// from a dispatch of the same geometry never exceed the bound; m-tiles past it
// are neither listed nor run).
__global__ __launch_bounds__(1024) void ffn_prep_kernel(const int32_t *__restrict__ slot_count,
                                                        int P, int64_t bound,
                                                        int32_t *__restrict__ tiles,
                                                        int32_t *__restrict__ slot_of) {
  __shared__ int sh[16];
  __shared__ int start[MOE_MAX_P + 1];
  const int p = threadIdx.x, lane = p & 63, wave = p >> 6;
  const int v = p < P ? (slot_count[p] + BM - 1) / BM : 0;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += sh[w];
  if (p < P) {
    tiles[p] = incl - v;
    start[p] = incl - v;
  }
  if (p == P - 1) {
    tiles[P] = incl;
    start[P] = incl;
  }
  __syncthreads();
  // m-tile u belongs to the largest slot q with start[q] <= u (empty slots
  // share their start with the next one and are skipped that way)
  const int64_t total = start[P] < bound ? start[P] : bound;
  for (int64_t u = p; u < total; u += blockDim.x) {
    int lo = 0, hi = P - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= u) lo = mid;
      else hi = mid - 1;
    }
    slot_of[u] = lo;
  }
}

// ---------------------------------------------------------- tile decode ---
struct Tile {
  int p, m, n;
  int gsz;  // m-tiles in this tile's group: the blocks that read the same weight n-tile
};
// Returns false when this block has no work.  GM: m-tiles per group.  Three
// dependent loads: the total, the slot of the block's m-tile (slot p covers
// list positions [tiles[p] NT, tiles[p + 1] NT)), then that slot's fields.
template <int GM>
__device__ __forceinline__ bool decode_tile(const int32_t *tiles, const int32_t *slot_of,
                                            int64_t bound, const int32_t *slot_count, int P,
                                            int NT, Tile &tl) {
  const int64_t total = (int64_t)tiles[P] * NT;
  const int64_t per = (total + kXcds - 1) / kXcds;
  const int64_t w = blockIdx.x;
  const int64_t i = w / kXcds;
  if (i >= per) return false;
  const int64_t L = (w % kXcds) * per + i;
  if (L >= total || L / NT >= bound) return false;
  const int p = slot_of[L / NT];
  const int64_t first = (int64_t)tiles[p] * NT;
  const int mt = (slot_count[p] + BM - 1) / BM;
  const int64_t local = L - first;
  const int g = (int)(local / ((int64_t)GM * NT));
  const int rem = (int)(local % ((int64_t)GM * NT));
  const int gsz = min(GM, mt - g * GM);
  tl.p = p;
  tl.gsz = gsz;
  tl.n = rem / gsz;
  tl.m = g * GM + rem % gsz;
  return true;
}

// LDS byte address of a __shared__ object, and a 16-byte LDS read that the
// compiler does not track (the caller waits with lgkmcnt before using it).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const MOE_LDS void *)p;
}
__device__ __forceinline__ v4i ds_read16(uint32_t addr) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// ------------------------------------------------------------ the GEMM ---
// MODE GATEUP: A rows gathered from the dispatch buffer, K = H; the 256-wide N
//              tile is 128 gate columns followed by the 128 matching up columns;
//              epilogue: SwiGLU -> h (fp32) and per-(row, n-tile) max |h|.
// MODE DOWN:   A rows = hq (dense), K = I; N tile = 256 output channels;
//              epilogue: bf16 return rows.
// Block tile 128 x 256, four wavefronts side by side along N, each owning all
// 128 rows x 64 columns (4 x 2 MFMA 32x32 blocks, 128 accumulators): the four
// waves share every A fragment read from LDS.  The loads of step kt + 2 are in
// flight while step kt feeds the MFMAs; one barrier
// per K step; two blocks per CU overlap each other's waits.
// Q8OUT (DOWN only): the return rows are INT8 with one fp32 scale per 256
// columns (the n-tile) instead of bf16 -- see the epilogue.
template <int MODE, bool DBG, bool Q8OUT = false>
__global__ __launch_bounds__(256, 2) void ffn_gemm_kernel(
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ slot_count, const int32_t *__restrict__ slot_offset, const int32_t *__restrict__ slot_logical,
    const int32_t *__restrict__ slot_rows, const uint8_t *__restrict__ disp_buf, int64_t msg,
    const int8_t *__restrict__ hq, const float *__restrict__ hs, const int8_t *__restrict__ w,
    const float *__restrict__ wscale, int P, int E, int H, int I, int64_t nrows, int64_t mt_bound,
    float *__restrict__ h_out, float *__restrict__ pmax, uint16_t *__restrict__ ret,
    int64_t ret_row_bytes, int32_t *__restrict__ acc_dbg) {
  constexpr int MB = BM / 32, NB = 2;       // MFMA blocks per wave
  // one LDS arena: the ring of A stages during the main loop, then the
  // output staging of the epilogue
  __shared__ __attribute__((aligned(16))) uint8_t lds[kArena];
  __shared__ float row_scale[BM];
  // the tile's column scales (GATEUP: 128 gate, then the 128 matching up;
  // DOWN: 256 output channels), fetched by one DMA before the main loop
  __shared__ __attribute__((aligned(16))) float col_scale[BN];

  const int K = MODE == GATEUP ? H : I;
  const int NT = MODE == GATEUP ? (I + BN / 2 - 1) / (BN / 2) : (H + BN - 1) / BN;
  Tile tl;
  if (!decode_tile<kGroupM<MODE>>(tiles, slot_of, mt_bound, slot_count, P, NT, tl)) return;
  const int e = slot_logical[tl.p];
  if (e < 0 || e >= E) return;
  const int cnt = slot_count[tl.p];
  const int64_t row0 = (int64_t)slot_offset[tl.p] + (int64_t)tl.m * BM;  // first dense row
  const int rows_here = min(BM, cnt - tl.m * BM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // per-row scale of this tile (activation scale s_x, or hs): loaded now,
  // stored to LDS only after the main loop, so that waiting for it does not
  // hold back the loop's first loads
  float sc = 0.0f;
  if (tid < BM) {
    const int64_t rr = row0 + tid;
    if (tid < rows_here && rr < nrows) {
      if (MODE == GATEUP) {
        const int32_t dr = slot_rows[rr];
        if (dr >= 0) sc = *(const float *)(disp_buf + (int64_t)dr * msg + H);
      } else {
        sc = hs[rr];
      }
    }
  }

  // Column scales: one wave instruction of 16 bytes per lane into col_scale
  // (lane l -> floats 4l .. 4l + 3), issued before every load of the main
  // loop, so the loop's first wait covers it.  Addresses past the row are
  // clamped to its last run; the epilogue zeroes those columns.
  if (wave == 0) {
    const float *src;
    if (MODE == GATEUP) {
      const int n = min(tl.n * (BN / 2) + 4 * (lane & 31), I - 4);
      src = wscale + (int64_t)e * 2 * I + (lane >> 5) * I + n;
    } else {
      src = wscale + (int64_t)e * H + min(tl.n * BN + 4 * lane, H - 4);
    }
    __builtin_amdgcn_global_load_lds(src, (MOE_LDS void *)col_scale, 16, 0, 0);
  }

  // Global -> LDS by DMA (global_load_lds_dwordx4): each wavefront instruction
  // fills one 1 KB LDS chunk = 16 tile rows x 64 bytes, lane i landing at
  // chunk + 16 i.  Wave w fills A chunks 2w and 2w + 1.
  // Lane i covers row 16 q + i / 4 of chunk q and picks the source chunk
  // (i & 3) ^ ((row >> 2) & 3), which produces the swizzled layout above.
  // Tile rows past the slot's last row read a valid stand-in row instead, as
  // do weight rows past I or H (the packed image holds clamped rows there):
  // they only feed accumulators of rows or columns that the epilogue never
  // stores.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = lane >> 2;
  auto a_row_ptr = [&](int r) -> const uint8_t * {
    const int c = ((lane & 3) ^ ((r >> 2) & 3)) * 16;
    r = min(r, rows_here - 1);
    const int64_t rr = min(row0 + r, nrows - 1);
    if (MODE == GATEUP) {
      const int32_t dr = slot_rows[rr];
      return disp_buf + (int64_t)(dr >= 0 ? dr : 0) * msg + c;
    }
    return (const uint8_t *)hq + rr * I + c;
  };
  const uint8_t *pa0 = a_row_ptr(16 * (2 * wv) + lrow), *pa1 = a_row_ptr(16 * (2 * wv + 1) + lrow);
  // A: the DMA of one K step (wave w: A chunks 2w, 2w + 1) into an LDS stage
  auto dma_a = [&](int kstep, uint8_t *stage) __attribute__((always_inline)) {
    const int64_t off = (int64_t)kstep * BK;
    uint8_t *la = stage + 2 * wv * 1024;
    __builtin_amdgcn_global_load_lds(pa0 + off, (MOE_LDS void *)(la), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(pa1 + off, (MOE_LDS void *)(la + 1024), 16, 0, 0);
  };

  v16i acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

  const int KT = K / BK;
  const int mb_live = (rows_here + 31) / 32;
  // this lane's swizzled 16-byte chunk of each 32-wide K sub-step (row blocks
  // start at multiples of 32, so the swizzle depends on the lane only)
  const int koff0 = ((0 ^ (((lane & 31) >> 2) & 3)) ^ (lane >> 5)) * 16;
  const int koff1 = ((2 ^ (((lane & 31) >> 2) & 3)) ^ (lane >> 5)) * 16;
  {
    // B straight from the packed image into registers, two K steps ahead, in a
    // ring of four register buffers: each wavefront reads only its own 64
    // columns, 4 KB per step as four 1 KB runs in MFMA fragment order (the image
    // holds them so); A keeps the LDS DMA, at the same distance, so one vmcnt per
    // step covers both (vector loads complete in order).  The weight loads are
    // inline assembly the compiler does not track: its wait-count pass cannot
    // follow a register ring across the loop edge and would drain every load in
    // flight at each group of steps.  Their safety is a property of the
    // generated code -- no instruction may touch a destination register between
    // its load and the MFMA that reads it, and no load may be in flight when the
    // loop ends -- which the library's build checks on the assembly.  The steps
    // are padded to a whole number of groups of four (zero weights in the
    // image), the loop issues its loads unconditionally, and the last two
    // steps issue none and wait statically (6, then 0 loads in flight).  Two
    // steps ahead measured faster than three (2-3%; one step ahead is slower):
    // more loads in flight only queue longer.
    constexpr int kDepth = 2, kAStages = 4;
    static_assert(kAStages * BM * LDS_STRIDE <= kArena, "A ring fits");
    const int KTp = (KT + 3) & ~3;
    const uint8_t *bsrc = (const uint8_t *)w + ((int64_t)e * NT + tl.n) * KTp * kPackedStepBytes +
                          wv * 4096 + lane * 16;
    v4i breg[4][2][2];
    auto load_b = [&](auto bi, auto ntw, int kstep) __attribute__((always_inline)) {
      constexpr int B = decltype(bi)::value;
      const uint8_t *p = bsrc + (int64_t)kstep * kPackedStepBytes;
      v4i t0, t1, t2, t3;
      if constexpr (decltype(ntw)::value)
        asm volatile("global_load_dwordx4 %0, %4, off nt\n\t"
                     "global_load_dwordx4 %1, %4, off offset:1024 nt\n\t"
                     "global_load_dwordx4 %2, %4, off offset:2048 nt\n\t"
                     "global_load_dwordx4 %3, %4, off offset:3072 nt"
                     : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
                     : "v"(p)
                     : "memory");
      else
        asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                     "global_load_dwordx4 %1, %4, off offset:1024\n\t"
                     "global_load_dwordx4 %2, %4, off offset:2048\n\t"
                     "global_load_dwordx4 %3, %4, off offset:3072"
                     : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
                     : "v"(p)
                     : "memory");
      breg[B][0][0] = t0;
      breg[B][0][1] = t1;
      breg[B][1][0] = t2;
      breg[B][1][1] = t3;
    };
    auto a_stage = [&](int kstep) { return lds + (kstep & (kAStages - 1)) * BM * LDS_STRIDE; };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using W6 = std::integral_constant<int, 6>;
    using W0 = std::integral_constant<int, 0>;
    using Yes = std::true_type;
    using No = std::false_type;
    // one K step: buffer B of the ring, W loads of later steps allowed in flight,
    // ISSUE: start the loads of step kt + 2
    auto step = [&](auto bi, auto wi, auto issue, auto ntw, int kt) __attribute__((always_inline)) {
      constexpr int B = decltype(bi)::value, W = decltype(wi)::value;
      if constexpr (W == 6)
        __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6): the loads of the next step
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __builtin_amdgcn_s_barrier();
      const uint32_t la = lds_addr(a_stage(kt)) + (lane & 31) * LDS_STRIDE;
      v4i af[2][MB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t koff = ks ? koff1 : koff0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[ks][mb] = ds_read16(la + mb * 32 * LDS_STRIDE + koff);
      }
      if constexpr (decltype(issue)::value) {
        load_b(std::integral_constant<int, (B + kDepth) % 4>{}, ntw, kt + kDepth);
        dma_a(min(kt + kDepth, KT - 1), a_stage(kt + kDepth));  // padded steps: any valid A
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the A fragments are in registers
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          // 32-row blocks past the slot's rows have nothing to compute; the first
          // always runs (a tile has rows), so every path consumes the buffer
          if (mb > 0 && mb >= mb_live) break;
          // weights as the first operand: the accumulators come out with
          // token rows across lanes and output columns across registers
          acc[mb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(breg[B][ks][0], af[ks][mb], acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(breg[B][ks][1], af[ks][mb], acc[mb][1], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto ntw) __attribute__((always_inline)) {
      load_b(I0{}, ntw, 0);
      dma_a(0, a_stage(0));
      load_b(I1{}, ntw, 1);
      dma_a(min(1, KT - 1), a_stage(1));
      for (int kt0 = 0; kt0 < KTp - 4; kt0 += 4) {
        step(I0{}, W6{}, Yes{}, ntw, kt0);
        step(I1{}, W6{}, Yes{}, ntw, kt0 + 1);
        step(I2{}, W6{}, Yes{}, ntw, kt0 + 2);
        step(I3{}, W6{}, Yes{}, ntw, kt0 + 3);
      }
      step(I0{}, W6{}, Yes{}, ntw, KTp - 4);
      step(I1{}, W6{}, Yes{}, ntw, KTp - 3);  // starts the loads of the last step
      step(I2{}, W6{}, No{}, ntw, KTp - 2);
      step(I3{}, W0{}, No{}, ntw, KTp - 1);  // vmcnt(0): nothing is in flight past this point
    };
    // A weight n-tile that no other block of the group reads (a slot's lone
    // m-tile, or the last group's single one) streams past L2 as non-temporal
    // loads, so it does not evict the n-tiles that groups of blocks share.
    // Every other tile loads normally: non-temporal loads of shared n-tiles
    // lose their L2 reuse (the kernel runs ~30% slower that way).
    if (tl.gsz == 1) run(Yes{});
    else run(No{});
  }
  if (tid < BM) row_scale[tid] = sc;
  __syncthreads();


  // ------------------------------------------------------------ epilogue ---
  // GATEUP, DOWN: acc[mb][nb][r] holds token row mb*32 + (lane % 32) and
  // column 8*(r/4) + 4*(lane/32) + r%4 of the wave's nb-th 32-column block
  // (the weights are the MFMA's first operand).  Results go through an LDS
  // staging tile (fp32 h [128][128], or bf16 [128][256]), each lane writing
  // its runs of four consecutive columns at once, and leave as 16-byte vector
  // stores of whole rows.
  const int col = lane & 31, half = lane >> 5;
  float *stg = (float *)lds;
  if (MODE == GATEUP) {
    // acc[mb][0][r] / acc[mb][1][r]: gate / up of token row mb*32 + col and of
    // pair wave*32 + 8*(r/4) + 4*half + r%4 of the tile -- four runs of four
    // consecutive pairs, each staged by one 16-byte LDS write
    const int nw = tl.n * (BN / 2) + wave * 32 + 4 * half;  // + 8 g + q: pair index
    float sgv[4][4], suv[4][4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int n = nw + 8 * g4;  // I % 64 == 0: a run is all below I or all past it
      const int ln = wave * 32 + 4 * half + 8 * g4;  // the run's pair index in the tile
      const float4 a = n < I ? *(const float4 *)(col_scale + ln) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 b = n < I ? *(const float4 *)(col_scale + BN / 2 + ln)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      sgv[g4][0] = a.x; sgv[g4][1] = a.y; sgv[g4][2] = a.z; sgv[g4][3] = a.w;
      suv[g4][0] = b.x; suv[g4][1] = b.y; suv[g4][2] = b.z; suv[g4][3] = b.w;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int lr = mb * 32 + col;
      const int64_t rr = row0 + lr;
      const float sx = row_scale[lr];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t ag = acc[mb][0][4 * g4 + q], au = acc[mb][1][4 * g4 + q];
          const float g = ((float)ag * sx) * sgv[g4][q];
          const float u = ((float)au * sx) * suv[g4][q];
          const float ex = (float)exp(-(double)g);
          hv[q] = (g / (1.0f + ex)) * u;
          const int n = nw + 8 * g4 + q;
          if (DBG && n < I && lr < rows_here && rr < nrows) {
            acc_dbg[rr * 2 * I + n] = ag;
            acc_dbg[rr * 2 * I + I + n] = au;
          }
        }
        // pairs past I stage 0 (g = u = 0), so the row scans below see only real h
        *(float4 *)(stg + lr * kStageStride + wave * 32 + 4 * half + 8 * g4) =
            make_float4(hv[0], hv[1], hv[2], hv[3]);
      }
    }
    __syncthreads();
    // max |h| of each row over this n-tile, stored n-tile major (the block's 128
    // rows as one run of floats: a [row][n-tile] layout left 16 four-byte
    // fragments of every 64-byte row segment to as many blocks, each a partly
    // written line for the memory side to complete).  Two threads per row scan the staged
    // row, alternate float4 columns each (a cross-lane reduction per value costs
    // far more); 16 lanes then read 8 rows x 2 columns, on 16 distinct bank groups
    {
      const int row = tid >> 1, part = tid & 1;
      const float4 *rowp = (const float4 *)(stg + row * kStageStride);
      float m = 0.0f;
#pragma unroll 8
      for (int c = part; c < BN / 2 / 4; c += 2) {
        const float4 v = rowp[c];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      const int64_t rr = row0 + row;
      if (part == 0 && row < rows_here && rr < nrows) pmax[(int64_t)tl.n * nrows + rr] = m;
    }
    // 128 rows x 128 fp32 = 4096 chunks of 4 values; h is read only by the
    // requantization after this kernel, so the stores are non-temporal
    const int n0 = tl.n * (BN / 2);
#pragma unroll 4
    for (int q = tid; q < BM * (BN / 2) / 4; q += 256) {
      const int lr = q >> 5, c4 = (q & 31) * 4;
      const int64_t rr = row0 + lr;
      if (lr < rows_here && rr < nrows && n0 + c4 < I)
        __builtin_nontemporal_store(*(const v4i *)(stg + lr * kStageStride + c4),
                                    (v4i *)(h_out + rr * I + n0 + c4));
    }
  } else {
    // bf16 staging [128 rows][256 columns] (row stride kStageStrideB bytes),
    // converted before staging, so the stored bits are the same.
    // acc[mb][nb][r]: token row mb*32 + col, tile column
    // wave*64 + nb*32 + 8*(r/4) + 4*half + r%4 -- four runs of four columns,
    // each staged by one 8-byte LDS write
    const int n0 = tl.n * BN;
    uint16_t *stb = (uint16_t *)lds;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int sb = wave * 64 + nb * 32 + 4 * half;  // + 8 g + q: tile column
      float sdv[4][4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = n0 + sb + 8 * g4;  // H % 128 == 0: a run is all below H or all past it
        const float4 v = c < H ? *(const float4 *)(col_scale + sb + 8 * g4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        sdv[g4][0] = v.x; sdv[g4][1] = v.y; sdv[g4][2] = v.z; sdv[g4][3] = v.w;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int lr = mb * 32 + col;
        const int64_t rr = row0 + lr;
        const float hsr = row_scale[lr];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int32_t a = acc[mb][nb][4 * g4 + q];
            y[q] = ((float)a * hsr) * sdv[g4][q];
            const int c = n0 + sb + 8 * g4 + q;
            if (DBG && lr < rows_here && rr < nrows && c < H) acc_dbg[rr * H + c] = a;
          }
          *(uint2 *)(stb + lr * (kStageStrideB / 2) + sb + 8 * g4) =
              make_uint2(bf16x2_bits(y[0], y[1]), bf16x2_bits(y[2], y[3]));
        }
      }
    }
    __syncthreads();
    if constexpr (Q8OUT) {
      // INT8 returns [XDS DeepSeek INT8 量化, P089: expert outputs quantized
      // before they travel back]: the staged bf16 tile is what the bf16 path
      // returns; each row's 256 columns (one block) get the token rule --
      // amax over the block, s = amax / 127, q = clamp(rne(y / s), +-127).
      // Columns past H staged 0, so they do not move the amax.  Row layout:
      // H codes, then ceil(H / 256) fp32 block scales, padded to whole 128-byte
      // lines (so each block of codes a tile stores is two whole lines).
      // The quotient y / s is taken without a division per element: with the
      // row's r = 1 / s (one IEEE division), q0 = y r, e = fma(-q0, s, y) and
      // q = fma(e, r, q0) (Markstein's correction step).  For s >= 2^-100 this
      // gives the same code as the IEEE quotient for every pair of bf16 values
      // y, amax with |y| <= amax -- all 1.07e9 of them checked exhaustively;
      // below that the residual can underflow, and the division is used.
      __shared__ float qscale[BM], qrcp[BM];
      uint8_t *retq = (uint8_t *)ret;
      {  // two threads per row, alternate 16-byte chunks (as the gate/up row scan)
        const int row = tid >> 1, part = tid & 1;
        const uint4 *rowp = (const uint4 *)((const uint8_t *)stb + row * kStageStrideB);
        float m = 0.0f;
#pragma unroll 8
        for (int c = part; c < BN / 8; c += 2) {
          const uint4 v = rowp[c];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(wd[q] & 0xffffu)), fabsf(bf16_bits_to_f32(wd[q] >> 16))));
        }
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        if (part == 0) {
          const float sq = m / 127.0f;
          qscale[row] = sq;
          qrcp[row] = sq >= 0x1p-100f ? 1.0f / sq : 0.0f;  // 0: divide
          const int64_t rr = row0 + row;
          if (row < rows_here && rr < nrows) *(float *)(retq + rr * ret_row_bytes + H + 4 * tl.n) = sq;
        }
      }
      __syncthreads();
      // 128 rows x 256 columns = 2048 chunks of 16 codes -> one 16-byte store each
#pragma unroll 2
      for (int q = tid; q < BM * (BN / 16); q += 256) {
        const int lr = q >> 4, c16 = (q & 15) * 16;
        const int64_t rr = row0 + lr;
        if (lr < rows_here && rr < nrows && n0 + c16 < H) {
          const float sq = qscale[lr], rq = qrcp[lr];
          const uint4 *src = (const uint4 *)((const uint8_t *)stb + lr * kStageStrideB + c16 * 2);
          const uint4 a = src[0], b = src[1];
          const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          // code + 128 = median(rint(q) + 128, 1, 255) (exact: small integers),
          // converted into its byte by v_cvt_pk_u8_f32; the final xor with
          // 0x80 per byte turns code + 128 back into the int8 code
          uint32_t pk[4] = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};  // code 0
          auto put = [&](int e, float q) __attribute__((always_inline)) {
            const float t = __builtin_amdgcn_fmed3f(rintf(q) + 128.0f, 1.0f, 255.0f);
            pk[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(t, e & 3, pk[e >> 2]);
          };
          auto y_of = [&](int e) __attribute__((always_inline)) {
            return bf16_bits_to_f32((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          };
          if (sq != 0.0f && rq != 0.0f) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float y = y_of(e), q0 = y * rq;
              put(e, fmaf(fmaf(-q0, sq, y), rq, q0));
            }
          } else if (sq != 0.0f) {
#pragma unroll
            for (int e = 0; e < 16; ++e) put(e, y_of(e) / sq);
          }
          const v4i codes = {(int)(pk[0] ^ 0x80808080u), (int)(pk[1] ^ 0x80808080u),
                             (int)(pk[2] ^ 0x80808080u), (int)(pk[3] ^ 0x80808080u)};
          __builtin_nontemporal_store(codes, (v4i *)(retq + rr * ret_row_bytes + n0 + c16));
        }
      }
      return;
    }
    // 128 rows x 256 columns = 4096 chunks of 8 bf16 -> one 16-byte
    // non-temporal store each (the combine reads the rows after this kernel)
#pragma unroll 4
    for (int q = tid; q < BM * (BN / 8); q += 256) {
      const int lr = q >> 5, c8 = (q & 31) * 8;
      const int64_t rr = row0 + lr;
      if (lr < rows_here && rr < nrows && n0 + c8 < H)
        __builtin_nontemporal_store(
            *(const v4i *)((const uint8_t *)stb + lr * kStageStrideB + c8 * 2),
            (v4i *)(ret + rr * H + n0 + c8));
    }
  }
}

// ---------------------------------------------------------------- requant ---
// One wavefront per row: amax = max of the gate-up partial maxima, then the
// token-wise INT8 rule (IEEE divide, round half to even, clamp +-127).  Lane l
// holds the float4 groups q * 64 + l of the row, so every load instruction
// reads 1 KB of consecutive bytes and every store writes 256; all of a row's
// loads are issued before the reduction that needs the maxima.
constexpr int kRequantMaxI = 2048;  // the register copy of a row; longer rows take a second pass
__global__ __launch_bounds__(256) void ffn_requant_kernel(const float *__restrict__ h,
                                                          const float *__restrict__ pmax,
                                                          const int32_t *__restrict__ slot_offset,
                                                          int P, int I, int64_t nrows,
                                                          int8_t *__restrict__ hq,
                                                          float *__restrict__ hs) {
  constexpr int G = kRequantMaxI / 256;  // float4 groups per lane
  const int lane = threadIdx.x & 63;
  const int64_t rr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rr >= nrows || rr >= slot_offset[P]) return;
  const int NT = (I + BN / 2 - 1) / (BN / 2);  // gate/up n-tiles of the row
  const int n4 = I / 4;                         // float4 groups of the row
  const float4 *src = (const float4 *)(h + rr * I);
  float4 v[G];
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int c = q * 64 + lane;
    if (c < n4) v[q] = src[c];
  }
  float m = 0.0f;
  for (int i = lane; i < NT; i += 64) m = fmaxf(m, pmax[(int64_t)i * nrows + rr]);
  m = wave_max_f32(m);
  const float s = m / 127.0f;
  if (lane == 0) hs[rr] = s;
  auto code4 = [&](float4 x) -> uint32_t {
    const float f[4] = {x.x, x.y, x.z, x.w};
    uint32_t word = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int code = 0;
      if (s != 0.0f) {
        float y = rintf(f[r] / s);
        y = fminf(fmaxf(y, -127.0f), 127.0f);
        code = (int)y;
      }
      word |= ((uint32_t)code & 0xffu) << (8 * r);
    }
    return word;
  };
  uint32_t *dst = (uint32_t *)(hq + rr * I);
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int c = q * 64 + lane;
    if (c < n4) dst[c] = code4(v[q]);
  }
  for (int c = kRequantMaxI / 4 + lane; c < n4; c += 64) dst[c] = code4(src[c]);
}

// ------------------------------------------------------- weight packing ---
// One thread per 16-byte slot of the image.  Block (e, n, s) holds, for each
// wavefront w of the GEMM and each MFMA fragment (ks, nb) of its K step, the
// 64 lanes' 16-byte operands in lane order: lane l takes tile row
// col(w, nb) + (l & 31), K bytes 64 s + 32 ks + 16 (l >> 5) .. +16.  Steps
// past K (the image pads K to whole groups of four steps) are zero.
__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t *__restrict__ w,
                                                           int gateup, int E, int H, int I,
                                                           int8_t *__restrict__ packed) {
  const int K = gateup ? H : I, KT = K / BK, KTp = packed_ksteps(K);
  const int NT = packed_ntiles(gateup ? MOE_PROJ_GATEUP : MOE_PROJ_DOWN, H, I);
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)E * NT * KTp * (kPackedStepBytes / 16)) return;
  const int l = (int)(q & 63), f = (int)((q >> 6) & 3), wv = (int)((q >> 8) & 3);
  const int ks = f >> 1, nb = f & 1;
  const int64_t blk = q >> 10;
  const int s = (int)(blk % KTp), n = (int)((blk / KTp) % NT);
  const int64_t e = blk / ((int64_t)KTp * NT);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (s < KT) {
    int64_t row;
    if (gateup) {  // tile rows: 128 gate pairs, then the 128 matching up rows
      const int r = nb * (BN / 2) + wv * 32 + (l & 31);
      const int pair = min(n * (BN / 2) + (r & (BN / 2 - 1)), I - 1);
      row = e * 2 * I + (r < BN / 2 ? pair : I + pair);
    } else {
      row = e * H + min(n * BN + wv * 64 + nb * 32 + (l & 31), H - 1);
    }
    v = *(const uint4 *)(w + row * K + (int64_t)s * BK + 32 * ks + 16 * (l >> 5));
  }
  *(uint4 *)(packed + q * 16) = v;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {
namespace {

struct FfnArgs {
  FfnScratch L;
  int32_t *tiles, *slot_of;
  float *pmax, *h, *hs;
  int8_t *hq;
  int64_t nrows, msg, mt_bound;
};

int ffn_common(const moe_geom_t *g, int32_t I, void *scratch, size_t scratch_bytes, FfnArgs *a) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (I <= 0 || I % 64 != 0 || I > 16384 || g->H % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!scratch || !aligned16(scratch)) return MOE_ERR_INVALID_ARG;
  const FfnScratch L = ffn_scratch_layout(*g, I);
  if ((int64_t)scratch_bytes < L.total) return MOE_ERR_CAPACITY;
  uint8_t *sc = (uint8_t *)scratch;
  *a = FfnArgs{L,
                  (int32_t *)(sc + L.tiles),
                  (int32_t *)(sc + L.slot_of),
                  (float *)(sc + L.pmax),
                  (float *)(sc + L.h),
                  (float *)(sc + L.hs),
                  (int8_t *)(sc + L.hq),
                  (int64_t)g->T * g->k,
                  msg_bytes_of(*g),
                  ffn_mtile_bound(*g)};
  return MOE_OK;
}

dim3 gemm_grid(int64_t mt_bound, int NT) {
  int64_t gsz = mt_bound * NT;  // upper bound of sum_p ceil(n_p / BM) * NT
  gsz = (gsz + kXcds - 1) / kXcds * kXcds;
  return dim3((unsigned)gsz);
}

}  // namespace
}  // namespace moe

extern "C" int moe_expert_gateup_q8(const void *disp_buf, const int32_t *slot_count,
                                    const int32_t *slot_offset, const int32_t *slot_rows,
                                    const int32_t *slot_logical, const int8_t *w_gateup,
                                    const float *s_gateup, int32_t I, const moe_geom_t *g,
                                    int32_t *acc_gateup_dbg, void *scratch, size_t scratch_bytes,
                                    void *stream) {
  FfnArgs args{};
  FfnArgs *a = &args;
  int st = ffn_common(g, I, scratch, scratch_bytes, a);
  if (st != MOE_OK) return st;
  if (a->nrows == 0) return MOE_OK;
  if (!disp_buf || !slot_count || !slot_offset || !slot_rows || !slot_logical || !w_gateup ||
      !s_gateup)
    return MOE_ERR_INVALID_ARG;
  // the epilogue reads the channel scales four at a time (16-byte loads)
  if (!aligned16(disp_buf) || !aligned16(w_gateup) || !aligned16(s_gateup))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(ffn_prep_kernel, dim3(1), dim3(1024), 0, s, slot_count, g->P, a->mt_bound,
                     a->tiles, a->slot_of);
  if ((st = launch_status()) != MOE_OK) return st;
  const dim3 grid = gemm_grid(a->mt_bound, (I + BN / 2 - 1) / (BN / 2));
#define MOE_GATEUP(DBG)                                                                         \
  hipLaunchKernelGGL((ffn_gemm_kernel<GATEUP, DBG>), grid, dim3(256), 0, s, a->tiles,         \
                     a->slot_of, slot_count, slot_offset, slot_logical, slot_rows,              \
                     (const uint8_t *)disp_buf, a->msg, (const int8_t *)nullptr,                \
                     (const float *)nullptr, w_gateup, s_gateup, g->P, g->E, g->H, I, a->nrows, \
                     a->mt_bound, a->h, a->pmax, (uint16_t *)nullptr, (int64_t)0, acc_gateup_dbg)
  if (acc_gateup_dbg)
    MOE_GATEUP(true);
  else
    MOE_GATEUP(false);
#undef MOE_GATEUP
  return launch_status();
}

namespace moe {
namespace {

// requant + down GEMM; ret is bf16 [T*k][H], or with q8out the INT8 return rows
int expert_down(const int32_t *slot_count, const int32_t *slot_offset,
                const int32_t *slot_logical, const int8_t *w_down, const float *s_down, int32_t I,
                const moe_geom_t *g, void *ret, bool q8out, int32_t *acc_down_dbg, void *scratch,
                size_t scratch_bytes, void *stream) {
  FfnArgs args{};
  FfnArgs *a = &args;
  int st = ffn_common(g, I, scratch, scratch_bytes, a);
  if (st != MOE_OK) return st;
  if (q8out && g->relays > 0) return MOE_ERR_UNSUPPORTED;  // the E2A hop moves bf16 rows
  if (a->nrows == 0) return MOE_OK;
  if (!slot_count || !slot_offset || !slot_logical || !w_down || !s_down || !ret)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_down) || !aligned16(s_down) || !aligned16(ret)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(ffn_requant_kernel, dim3((unsigned)((a->nrows + 3) / 4)), dim3(256), 0, s,
                     a->h, a->pmax, slot_offset, g->P, I, a->nrows, a->hq, a->hs);
  if ((st = launch_status()) != MOE_OK) return st;
  const dim3 grid = gemm_grid(a->mt_bound, (g->H + BN - 1) / BN);
  const int64_t rb = q8out ? ret_q8_row_bytes_of(*g) : (int64_t)g->H * 2;
#define MOE_DOWN(DBG, Q)                                                                        \
  hipLaunchKernelGGL((ffn_gemm_kernel<DOWN, DBG, Q>), grid, dim3(256), 0, s, a->tiles,         \
                     a->slot_of, slot_count, slot_offset, slot_logical, (const int32_t *)nullptr, \
                     (const uint8_t *)nullptr, a->msg, a->hq, a->hs, w_down, s_down, g->P, g->E,  \
                     g->H, I, a->nrows, a->mt_bound, (float *)nullptr, (float *)nullptr,          \
                     (uint16_t *)ret, rb, acc_down_dbg)
  if (q8out) {
    if (acc_down_dbg) MOE_DOWN(true, true);
    else MOE_DOWN(false, true);
  } else {
    if (acc_down_dbg) MOE_DOWN(true, false);
    else MOE_DOWN(false, false);
  }
#undef MOE_DOWN
  return launch_status();
}

}  // namespace
}  // namespace moe

extern "C" int moe_expert_down_q8(const int32_t *slot_count, const int32_t *slot_offset,
                                  const int32_t *slot_logical, const int8_t *w_down,
                                  const float *s_down, int32_t I, const moe_geom_t *g,
                                  uint16_t *ret, int32_t *acc_down_dbg, void *scratch,
                                  size_t scratch_bytes, void *stream) {
  return expert_down(slot_count, slot_offset, slot_logical, w_down, s_down, I, g, ret, false,
                     acc_down_dbg, scratch, scratch_bytes, stream);
}

extern "C" int moe_expert_down_q8_int8ret(const int32_t *slot_count, const int32_t *slot_offset,
                                          const int32_t *slot_logical, const int8_t *w_down,
                                          const float *s_down, int32_t I, const moe_geom_t *g,
                                          void *ret_q8, int32_t *acc_down_dbg, void *scratch,
                                          size_t scratch_bytes, void *stream) {
  return expert_down(slot_count, slot_offset, slot_logical, w_down, s_down, I, g, ret_q8, true,
                     acc_down_dbg, scratch, scratch_bytes, stream);
}

extern "C" int moe_expert_ffn_q8(const void *disp_buf, const int32_t *slot_count,
                                 const int32_t *slot_offset, const int32_t *slot_rows,
                                 const int32_t *slot_logical, const int8_t *w_gateup,
                                 const float *s_gateup, const int8_t *w_down, const float *s_down,
                                 int32_t I, const moe_geom_t *g, uint16_t *ret,
                                 int32_t *acc_gateup_dbg, int32_t *acc_down_dbg, void *scratch,
                                 size_t scratch_bytes, void *stream) {
  if (g && g->T > 0 && (!w_down || !s_down || !ret)) return MOE_ERR_INVALID_ARG;
  int st = moe_expert_gateup_q8(disp_buf, slot_count, slot_offset, slot_rows, slot_logical,
                                w_gateup, s_gateup, I, g, acc_gateup_dbg, scratch, scratch_bytes,
                                stream);
  if (st != MOE_OK) return st;
  return moe_expert_down_q8(slot_count, slot_offset, slot_logical, w_down, s_down, I, g, ret,
                            acc_down_dbg, scratch, scratch_bytes, stream);
}

extern "C" int moe_pack_expert_weights(const int8_t *w, moe_proj_t proj, int32_t E, int32_t H,
                                       int32_t I, int8_t *packed, size_t packed_bytes,
                                       void *stream) {
  if (!w || !packed || !aligned16(w) || !aligned16(packed) || E <= 0) return MOE_ERR_INVALID_ARG;
  if (proj != MOE_PROJ_GATEUP && proj != MOE_PROJ_DOWN) return MOE_ERR_INVALID_ARG;
  if (H <= 0 || H % 128 != 0 || H > MOE_MAX_H || I <= 0 || I % 64 != 0 || I > 16384)
    return MOE_ERR_UNSUPPORTED;
  const int64_t bytes = packed_weight_bytes(proj, E, H, I);
  if ((int64_t)packed_bytes < bytes) return MOE_ERR_CAPACITY;
  const int64_t w_bytes = (int64_t)E * (proj == MOE_PROJ_GATEUP ? 2 * I : H) * (proj == MOE_PROJ_GATEUP ? H : I);
  const uintptr_t w0 = (uintptr_t)w, p0 = (uintptr_t)packed;
  if (w0 < p0 + (uintptr_t)bytes && p0 < w0 + (uintptr_t)w_bytes) return MOE_ERR_INVALID_ARG;
  const int64_t slots = bytes / 16;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, w, proj == MOE_PROJ_GATEUP ? 1 : 0, E, H, I, packed);
  return launch_status();
}
