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
//            B = [64 gate rows | 64 up rows] of the slot's logical expert.
//            Epilogue: dequantize both, h = silu(g) * u, write h (fp32) and
//            the per-(row, n-tile) max |h| (no atomics).
//   requant  per row: amax = max of the partial maxima (exact), token-wise
//            INT8 of h -> hq, hs.
//   down     grouped GEMM: A = hq rows (dense, K = I), B = 128 rows of W_down;
//            epilogue: y = bf16((f32(acc) * hs) * s_down) into the dense
//            return rows.
// Tiles: 128 x 128 outputs per 256-thread block (2 x 2 wavefronts of 64 x 64,
// each 2 x 2 MFMA 32x32 blocks), K steps of 64 bytes double-buffered in LDS
// with a 16-byte row pad.  The work list is ordered slot-major, then groups of
// kGroupM m-tiles, then n-tiles, then m inside the group, and blocks are
// remapped so that each XCD walks one contiguous stretch of it: the m-tiles of
// a group share every weight tile in that XCD's L2.
#include "common.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 16;  // bytes per LDS row (pad breaks bank aliasing)
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

enum Mode { GATEUP = 0, DOWN = 1 };

// ------------------------------------------------------------------ prep ---
__global__ __launch_bounds__(1024) void ffn_prep_kernel(const int32_t *__restrict__ slot_count,
                                                        int P, int32_t *__restrict__ tiles) {
  __shared__ int sh[16];
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
  if (p < P) tiles[p] = incl - v;
  if (p == P - 1) tiles[P] = incl;
}

// ---------------------------------------------------------- tile decode ---
struct Tile {
  int p, m, n;
};
// Returns false when this block has no work.
__device__ __forceinline__ bool decode_tile(const int32_t *tiles, const int32_t *slot_count,
                                            int P, int NT, Tile &tl) {
  const int64_t total = (int64_t)tiles[P] * NT;
  const int64_t per = (total + kXcds - 1) / kXcds;
  const int64_t w = blockIdx.x;
  const int64_t i = w / kXcds;
  if (i >= per) return false;
  const int64_t L = (w % kXcds) * per + i;
  if (L >= total) return false;
  // slot: largest p with tiles[p] * NT <= L
  int lo = 0, hi = P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)tiles[mid] * NT <= L) lo = mid;
    else hi = mid - 1;
  }
  const int p = lo;
  const int mt = (slot_count[p] + BM - 1) / BM;
  const int64_t local = L - (int64_t)tiles[p] * NT;
  const int g = (int)(local / ((int64_t)kGroupM * NT));
  const int rem = (int)(local % ((int64_t)kGroupM * NT));
  const int gsz = min(kGroupM, mt - g * kGroupM);
  tl.p = p;
  tl.n = rem / gsz;
  tl.m = g * kGroupM + rem % gsz;
  return true;
}

// ------------------------------------------------------------ the GEMM ---
// MODE GATEUP: A rows gathered from the dispatch buffer, K = H, N tile = 64 gate
//              + 64 up columns, epilogue SwiGLU -> h, partial row maxima.
// MODE DOWN:   A rows = hq (dense), K = I, N tile = 128 output channels,
//              epilogue -> bf16 return rows.
template <int MODE>
__global__ __launch_bounds__(256, 2) void ffn_gemm_kernel(
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ slot_count,
    const int32_t *__restrict__ slot_offset, const int32_t *__restrict__ slot_logical,
    const int32_t *__restrict__ slot_rows, const uint8_t *__restrict__ disp_buf, int64_t msg,
    const int8_t *__restrict__ hq, const float *__restrict__ hs, const int8_t *__restrict__ w,
    const float *__restrict__ wscale, int P, int E, int H, int I, int64_t nrows,
    float *__restrict__ h_out, float *__restrict__ pmax, uint16_t *__restrict__ ret,
    int32_t *__restrict__ acc_dbg) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * LDS_STRIDE];
  __shared__ float row_scale[BM];
  __shared__ float row_max[2][BM];

  const int K = MODE == GATEUP ? H : I;
  const int NT = MODE == GATEUP ? I / 64 : (H + BN - 1) / BN;
  Tile tl;
  if (!decode_tile(tiles, slot_count, P, NT, tl)) return;
  const int e = slot_logical[tl.p];
  if (e < 0 || e >= E) return;
  const int cnt = slot_count[tl.p];
  const int64_t row0 = (int64_t)slot_offset[tl.p] + (int64_t)tl.m * BM;  // first dense row
  const int rows_here = min(BM, cnt - tl.m * BM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // per-row scale of this tile (activation scale s_x, or hs)
  if (tid < BM) {
    float sc = 0.0f;
    const int64_t rr = row0 + tid;
    if (tid < rows_here && rr < nrows) {
      if (MODE == GATEUP) {
        const int32_t dr = slot_rows[rr];
        if (dr >= 0) sc = *(const float *)(disp_buf + (int64_t)dr * msg + H);
      } else {
        sc = hs[rr];
      }
    }
    row_scale[tid] = sc;
  }

  // global -> LDS assignment: 2 x 16 B of A and 2 x 16 B of B per thread per K step
  const uint8_t *a_src[2];
  const uint8_t *b_src[2];
  int ld_row[2], ld_col[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * 256;
    ld_row[i] = idx >> 2;
    ld_col[i] = (idx & 3) * 16;
    const int r = ld_row[i];
    const int64_t rr = row0 + r;
    a_src[i] = nullptr;
    if (r < rows_here && rr < nrows) {
      if (MODE == GATEUP) {
        const int32_t dr = slot_rows[rr];
        if (dr >= 0) a_src[i] = disp_buf + (int64_t)dr * msg + ld_col[i];
      } else {
        a_src[i] = (const uint8_t *)hq + rr * I + ld_col[i];
      }
    }
    b_src[i] = nullptr;
    if (MODE == GATEUP) {
      const int wrow = r < 64 ? tl.n * 64 + r : I + tl.n * 64 + (r - 64);
      b_src[i] = (const uint8_t *)w + ((int64_t)e * 2 * I + wrow) * H + ld_col[i];
    } else {
      const int wrow = tl.n * BN + r;
      if (wrow < H) b_src[i] = (const uint8_t *)w + ((int64_t)e * H + wrow) * I + ld_col[i];
    }
  }
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  uint4 ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = a_src[i] ? *(const uint4 *)(a_src[i] + (int64_t)kt * BK) : zero4;
      rb[i] = b_src[i] ? *(const uint4 *)(b_src[i] + (int64_t)kt * BK) : zero4;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(uint4 *)(&lds_a[buf][ld_row[i] * LDS_STRIDE + ld_col[i]]) = ra[i];
      *(uint4 *)(&lds_b[buf][ld_row[i] * LDS_STRIDE + ld_col[i]]) = rb[i];
    }
  };

  // B-tile row offsets of this wave's two 32-column blocks
  const int nbo0 = MODE == GATEUP ? wn * 32 : wn * 64;
  const int nbo1 = MODE == GATEUP ? 64 + wn * 32 : wn * 64 + 32;

  v16i acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int koff = ks * 32 + (lane >> 5) * 16;
      v4i af[2], bf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const v4i *)(&lds_a[buf][(wm * 64 + mb * 32 + (lane & 31)) * LDS_STRIDE + koff]);
      bf[0] = *(const v4i *)(&lds_b[buf][(nbo0 + (lane & 31)) * LDS_STRIDE + koff]);
      bf[1] = *(const v4i *)(&lds_b[buf][(nbo1 + (lane & 31)) * LDS_STRIDE + koff]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue ---
  // acc[mb][nb][r] holds output row wm*64 + mb*32 + 8*(r/4) + 4*(lane/32) + r%4,
  // column (lane % 32) of the wave's nb-th 32-column block.
  const int col = lane & 31, half = lane >> 5;
  if (MODE == GATEUP) {
    const int n = tl.n * 64 + wn * 32 + col;  // gate / up pair index, < I
    const float sg = wscale[(int64_t)e * 2 * I + n];
    const float su = wscale[(int64_t)e * 2 * I + I + n];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int64_t rr = row0 + lr;
        const bool ok = lr < rows_here && rr < nrows;
        const int32_t ag = acc[mb][0][r], au = acc[mb][1][r];
        const float sx = row_scale[lr];
        const float g = ((float)ag * sx) * sg;
        const float u = ((float)au * sx) * su;
        const float ex = (float)exp(-(double)g);
        const float hv = (g / (1.0f + ex)) * u;
        if (ok) {
          h_out[rr * I + n] = hv;
          if (acc_dbg) {
            acc_dbg[rr * 2 * I + n] = ag;
            acc_dbg[rr * 2 * I + I + n] = au;
          }
        }
        float m = ok ? fabsf(hv) : 0.0f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (col == 0) row_max[wn][lr] = m;
      }
    }
    __syncthreads();
    if (tid < BM) {
      const int64_t rr = row0 + tid;
      if (tid < rows_here && rr < nrows)
        pmax[rr * (I / 64) + tl.n] = fmaxf(row_max[0][tid], row_max[1][tid]);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int c = tl.n * BN + wn * 64 + nb * 32 + col;
      const float sd = c < H ? wscale[(int64_t)e * H + c] : 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const int64_t rr = row0 + lr;
          if (lr < rows_here && rr < nrows && c < H) {
            const int32_t a = acc[mb][nb][r];
            const float y = ((float)a * row_scale[lr]) * sd;
            ret[rr * H + c] = (uint16_t)f32_to_bf16_bits(y);
            if (acc_dbg) acc_dbg[rr * H + c] = a;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- requant ---
// One wavefront per row: amax = max of the gate-up partial maxima, then the
// token-wise INT8 rule (IEEE divide, round half to even, clamp +-127).
__global__ __launch_bounds__(256) void ffn_requant_kernel(const float *__restrict__ h,
                                                          const float *__restrict__ pmax,
                                                          const int32_t *__restrict__ slot_offset,
                                                          int P, int I, int64_t nrows,
                                                          int8_t *__restrict__ hq,
                                                          float *__restrict__ hs) {
  const int lane = threadIdx.x & 63;
  const int64_t rr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rr >= nrows || rr >= slot_offset[P]) return;
  const int NT = I / 64;
  float m = 0.0f;
  for (int i = lane; i < NT; i += 64) m = fmaxf(m, pmax[rr * NT + i]);
  m = wave_max_f32(m);
  const float s = m / 127.0f;
  if (lane == 0) hs[rr] = s;
  for (int e0 = lane * 16; e0 < I; e0 += 64 * 16) {
    const float4 *src = (const float4 *)(h + rr * I + e0);
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = src[q];
      const float f[4] = {v.x, v.y, v.z, v.w};
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
      pk[q] = word;
    }
    *(uint4 *)(hq + rr * I + e0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {
namespace {

struct FfnArgs {
  FfnScratch L;
  int32_t *tiles;
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
                  (float *)(sc + L.pmax),
                  (float *)(sc + L.h),
                  (float *)(sc + L.hs),
                  (int8_t *)(sc + L.hq),
                  (int64_t)g->T * g->k,
                  msg_bytes_of(*g),
                  (int64_t)g->T * g->k / BM + g->P};
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
  if (!aligned16(disp_buf) || !aligned16(w_gateup)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(ffn_prep_kernel, dim3(1), dim3(1024), 0, s, slot_count, g->P, a->tiles);
  if ((st = launch_status()) != MOE_OK) return st;
  hipLaunchKernelGGL((ffn_gemm_kernel<GATEUP>), gemm_grid(a->mt_bound, I / 64), dim3(256), 0, s,
                     a->tiles, slot_count, slot_offset, slot_logical, slot_rows,
                     (const uint8_t *)disp_buf, a->msg, (const int8_t *)nullptr,
                     (const float *)nullptr, w_gateup, s_gateup, g->P, g->E, g->H, I, a->nrows,
                     a->h, a->pmax, (uint16_t *)nullptr, acc_gateup_dbg);
  return launch_status();
}

extern "C" int moe_expert_down_q8(const int32_t *slot_count, const int32_t *slot_offset,
                                  const int32_t *slot_logical, const int8_t *w_down,
                                  const float *s_down, int32_t I, const moe_geom_t *g,
                                  uint16_t *ret, int32_t *acc_down_dbg, void *scratch,
                                  size_t scratch_bytes, void *stream) {
  FfnArgs args{};
  FfnArgs *a = &args;
  int st = ffn_common(g, I, scratch, scratch_bytes, a);
  if (st != MOE_OK) return st;
  if (a->nrows == 0) return MOE_OK;
  if (!slot_count || !slot_offset || !slot_logical || !w_down || !s_down || !ret)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_down) || !aligned16(ret)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(ffn_requant_kernel, dim3((unsigned)((a->nrows + 3) / 4)), dim3(256), 0, s,
                     a->h, a->pmax, slot_offset, g->P, I, a->nrows, a->hq, a->hs);
  if ((st = launch_status()) != MOE_OK) return st;
  hipLaunchKernelGGL((ffn_gemm_kernel<DOWN>), gemm_grid(a->mt_bound, g->H / BN), dim3(256), 0, s,
                     a->tiles, slot_count, slot_offset, slot_logical, (const int32_t *)nullptr,
                     (const uint8_t *)nullptr, a->msg, a->hq, a->hs, w_down, s_down, g->P, g->E,
                     g->H, I, a->nrows, (float *)nullptr, (float *)nullptr, ret, acc_down_dbg);
  return launch_status();
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
