// Combine: gather each token's k value rows, dequantize, gate-weighted sum.
//
// [XDS 合设 A2A, COMBINE procedure (result[token] += value * gate weight);
//  CMI EP320 FusedCombine (all k contributions present, dequantize, weight by
//  the gate)]
//
// One wavefront per pair of 1 KB element groups of a token.  The k row
// gathers of the two groups are issued together (2k x 16 B per lane in
// flight), then summed in fp32 in ascending route order with separate
// multiply and add (no FMA contraction), so the result is the same bits as the
// plain loop on the CPU.  Every value row is read exactly once, so the gathers
// are non-temporal loads (measured on the 12288-token layer: 284 us instead of
// 323 us).
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Q8: INT8 value rows (codes at byte 0).  QB: their scales are per block of
// MOE_RET_Q8_BLOCK columns from byte H (INT8 expert returns) instead of one
// scale at byte H (dispatch messages).
template <bool Q8, bool OUT_BF16, int KMAX, bool QB = false>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t *__restrict__ src,
                                                      const int32_t *__restrict__ row,
                                                      const float *__restrict__ topk_w, int T,
                                                      int H, int k, int64_t row_bytes, int cs,
                                                      void *__restrict__ out) {
  // cs wavefronts per token: wavefront part of token t takes element groups
  // part, part + cs, ... (the host makes it one pair of groups); every output
  // element is computed exactly as with one
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = wv / cs;
  const int part = (int)(wv % cs);
  if (t >= T) return;
  int64_t my_row = -1;
  float my_w = 0.0f, my_s = 0.0f;
  if (lane < k) {
    my_row = row[t * k + lane];
    my_w = topk_w[t * k + lane];
    if (Q8 && !QB && my_row >= 0) my_s = *(const float *)(src + my_row * row_bytes + H);
  }
  const uint8_t *base[KMAX];
  float w[KMAX], sc[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int64_t r = __shfl(my_row, j, 64);
    w[j] = __shfl(my_w, j, 64);
    sc[j] = __shfl(my_s, j, 64);
    base[j] = (j < k && r >= 0) ? src + r * row_bytes : nullptr;
  }
  constexpr int EPL = Q8 ? 16 : 8;  // elements per lane per 16-byte load
  constexpr int U = 2;              // element groups whose gathers are in flight together
  const int iters = (H + 64 * EPL - 1) / (64 * EPL);
  for (int i0 = part * U; i0 < iters; i0 += U * cs) {
    uint4 v[U][KMAX];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = ((i0 + u) * 64 + lane) * EPL;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (base[j] && e0 < H) {
          const v4u lv = __builtin_nontemporal_load((const v4u *)(base[j] + (Q8 ? e0 : 2 * e0)));
          v[u][j] = make_uint4(lv.x, lv.y, lv.z, lv.w);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = ((i0 + u) * 64 + lane) * EPL;
      if (e0 >= H) break;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (!base[j]) continue;
        const uint32_t *wd = (const uint32_t *)&v[u][j];
        // a lane's 16 codes lie in one scale block (16 divides the block)
        const float sj = QB ? *(const float *)(base[j] + H + 4 * (e0 / MOE_RET_Q8_BLOCK)) : sc[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float x;
          if (Q8) {
            const int8_t q = (int8_t)((wd[e >> 2] >> (8 * (e & 3))) & 0xffu);
            x = (float)q * sj;
          } else {
            x = bf16_bits_to_f32((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          }
          const float prod = w[j] * x;
          acc[e] = acc[e] + prod;
        }
      }
      if (OUT_BF16) {
        uint32_t pk[EPL / 2];
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e)
          pk[e] = bf16x2_bits(acc[2 * e], acc[2 * e + 1]);
        uint4 *dst = (uint4 *)((uint16_t *)out + t * H + e0);
#pragma unroll
        for (int q = 0; q < EPL / 8; ++q)
          dst[q] = make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
      } else {
        float4 *dst = (float4 *)((float *)out + t * H + e0);
#pragma unroll
        for (int q = 0; q < EPL / 4; ++q)
          dst[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
      }
    }
  }
}

template <int KMAX>
void launch_combine(bool q8, bool qb, bool obf, dim3 grid, hipStream_t s, const uint8_t *src,
                    const int32_t *row, const float *w, const moe_geom_t &g, int64_t rb, int cs,
                    void *out) {
#define MOE_COMBINE(Q, O, B)                                                                     \
  hipLaunchKernelGGL((combine_kernel<Q, O, KMAX, B>), grid, dim3(256), 0, s, src, row, w, g.T,    \
                     g.H, g.k, rb, cs, out)
  if (qb && obf) MOE_COMBINE(true, true, true);
  else if (qb) MOE_COMBINE(true, false, true);
  else if (q8 && obf) MOE_COMBINE(true, true, false);
  else if (q8) MOE_COMBINE(true, false, false);
  else if (obf) MOE_COMBINE(false, true, false);
  else MOE_COMBINE(false, false, false);
#undef MOE_COMBINE
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine(moe_ret_mode_t mode, const void *src, const int32_t *row,
                           const float *topk_w, const moe_geom_t *g, moe_dtype_t out_dtype,
                           void *out, void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (g->T > 0 && (!src || !row || !topk_w || !out)) return MOE_ERR_INVALID_ARG;
  if (mode != MOE_RET_Q8_FROM_DISPATCH && mode != MOE_RET_BF16 && mode != MOE_RET_Q8_BLOCKS &&
      mode != MOE_RET_Q8_ROWS)
    return MOE_ERR_INVALID_ARG;
  if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (g->T == 0) return MOE_OK;
  // Q8_ROWS: token-wise INT8 returns, the message layout (codes, then the row's
  // scale at byte H) at the INT8 return row size
  const bool qb = mode == MOE_RET_Q8_BLOCKS;
  const bool q8 = mode == MOE_RET_Q8_FROM_DISPATCH || mode == MOE_RET_Q8_ROWS || qb;
  const int64_t rb = (qb || mode == MOE_RET_Q8_ROWS) ? ret_q8_row_bytes_of(*g)
                     : q8                           ? msg_bytes_of(*g)
                                                    : (int64_t)g->H * 2;
  // wavefronts per token: one per pair of 1 KB element groups (7 at H = 7168
  // with bf16 rows, 4 with INT8 rows), at every batch size: more, shorter
  // wavefronts keep more gathers in flight (12288-token layer: bf16 returns
  // 286 -> 267 us, token-wise INT8 returns 163 -> 153 us against one wavefront
  // per token).  Block-scaled INT8 returns measured the same either way and
  // keep one wavefront per token unless the batch is small.
  const int groups = (int)((g->H + 64 * (q8 ? 16 : 8) * 2 - 1) / (64 * (q8 ? 16 : 8) * 2));
  const int cs = qb ? (int)std::max<int64_t>(1, std::min<int64_t>(groups, (1024 + g->T - 1) / g->T))
                    : groups;
  const dim3 grid((unsigned)(((int64_t)g->T * cs + 3) / 4));
  hipStream_t s = (hipStream_t)stream;
  const bool obf = out_dtype == MOE_DTYPE_BF16;
  const uint8_t *sp = (const uint8_t *)src;
  if (g->k <= 2)
    launch_combine<2>(q8, qb, obf, grid, s, sp, row, topk_w, *g, rb, cs, out);
  else if (g->k <= 4)
    launch_combine<4>(q8, qb, obf, grid, s, sp, row, topk_w, *g, rb, cs, out);
  else if (g->k <= 8)
    launch_combine<8>(q8, qb, obf, grid, s, sp, row, topk_w, *g, rb, cs, out);
  else
    launch_combine<16>(q8, qb, obf, grid, s, sp, row, topk_w, *g, rb, cs, out);
  return launch_status();
}

// ------------------------------------------------ token-wise INT8 returns ---
namespace moe {
namespace {
// One wavefront per dense return row (the send side of the return path): the
// row's bf16 values are loaded once into registers (lane l holds the 16-byte
// chunks i * 64 + l, eight values each), amax by a wavefront max, s = amax / 127
// (IEEE divide), then every value's code; each lane stores the eight codes of a
// chunk as one 8-byte store (512 consecutive bytes per wave instruction) and
// lane 0 the scale at byte H.  The quotient y / s is taken with the row's
// reciprocal r = 1 / s and one Markstein correction, q0 = y r,
// q = fma(fma(-q0, s, y), r, q0), which gives the IEEE quotient's code for
// every pair of bf16 values |y| <= amax when s >= 2^-100 (checked for all such
// pairs on the host); below that the division itself is used.
template <int NIT>
__global__ __launch_bounds__(256) void quant_returns_kernel(const uint16_t *__restrict__ ret,
                                                            const int32_t *__restrict__ slot_offset,
                                                            int P, int H, int64_t nrows,
                                                            int64_t row_bytes,
                                                            uint8_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nrows || r >= slot_offset[P]) return;
  const int nch = H / 8;  // 16-byte chunks of the bf16 row
  const uint16_t *src = ret + r * H;
  uint4 v[NIT];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int c = i * 64 + lane;
    if (c < nch) {
      const v4u lv = __builtin_nontemporal_load((const v4u *)(src + 8 * c));
      v[i] = make_uint4(lv.x, lv.y, lv.z, lv.w);
      const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(wd[q] & 0xffffu)),
                                 fabsf(bf16_bits_to_f32(wd[q] >> 16))));
    }
  }
  amax = wave_max_f32(amax);
  const float s = amax / 127.0f;
  const float rs = s >= 0x1p-100f ? 1.0f / s : 0.0f;  // 0: divide
  uint8_t *dst = out + r * row_bytes;
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int c = i * 64 + lane;
    if (c >= nch) break;
    const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    // code + 128 = median(rint(q) + 128, 1, 255), converted into its byte of the
    // packed word; the xor with 0x80 per byte turns it back into the int8 code
    uint32_t pk[2] = {0x80808080u, 0x80808080u};  // code 0 (s = 0)
    auto put = [&](int e, float q) __attribute__((always_inline)) {
      const float t = __builtin_amdgcn_fmed3f(rintf(q) + 128.0f, 1.0f, 255.0f);
      pk[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(t, e & 3, pk[e >> 2]);
    };
    auto y_of = [&](int e) __attribute__((always_inline)) {
      return bf16_bits_to_f32((wd[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    };
    if (s != 0.0f && rs != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = y_of(e), q0 = y * rs;
        put(e, fmaf(fmaf(-q0, s, y), rs, q0));
      }
    } else if (s != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) put(e, y_of(e) / s);
    }
    *(uint2 *)(dst + 8 * c) = make_uint2(pk[0] ^ 0x80808080u, pk[1] ^ 0x80808080u);
  }
  // the scale's 128-byte line is written whole (the scale, then zeros over the
  // row's padding up to the line's end or the row's): a lone 4-byte store leaves
  // a partly written line for the memory side to complete
  const int64_t line_end = min(row_bytes, (int64_t)((H + 4 + 127) & ~127));
  if (lane < (int)((line_end - H + 15) / 16))
    *(uint4 *)(dst + H + 16 * lane) = make_uint4(lane == 0 ? __float_as_uint(s) : 0u, 0u, 0u, 0u);
}
}  // namespace
}  // namespace moe

extern "C" int moe_quant_returns_q8(const uint16_t *ret, const int32_t *slot_offset,
                                    const moe_geom_t *g, void *ret_q8, void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (g->relays > 0) return MOE_ERR_UNSUPPORTED;  // the E2A hop moves bf16 rows
  const int64_t n = (int64_t)g->T * g->k;
  if (n == 0) return MOE_OK;
  if (!ret || !slot_offset || !ret_q8) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ret) || !aligned16(ret_q8)) return MOE_ERR_INVALID_ARG;
  const int nit = (g->H / 8 + 63) / 64;
  const dim3 grid((unsigned)((n + 3) / 4));
  hipStream_t s = (hipStream_t)stream;
  const int64_t rb = ret_q8_row_bytes_of(*g);
  uint8_t *o = (uint8_t *)ret_q8;
#define MOE_QR(N)                                                                              \
  hipLaunchKernelGGL((quant_returns_kernel<N>), grid, dim3(256), 0, s, ret, slot_offset, g->P, \
                     g->H, n, rb, o)
  if (nit <= 2) MOE_QR(2);
  else if (nit <= 4) MOE_QR(4);
  else if (nit <= 8) MOE_QR(8);
  else if (nit <= 16) MOE_QR(16);
  else MOE_QR(32);
#undef MOE_QR
  return launch_status();
}

// ------------------------------------------------------- E2A second hop ---
namespace moe {
namespace {
// One wavefront per route: rows of slots on partitions >= relays are staged
// after the T*k return rows, and the combine is pointed at the staged copy.
__global__ __launch_bounds__(256) void relay_returns_kernel(
    uint16_t *__restrict__ ret, const int32_t *__restrict__ phys,
    const int32_t *__restrict__ slot_partition, const int32_t *__restrict__ ret_row,
    int64_t n_routes, int P, int H, int relays, int32_t *__restrict__ comb_row) {
  const int lane = threadIdx.x & 63;
  const int64_t gi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gi >= n_routes) return;
  const int32_t rr = ret_row[gi];
  const int p = phys[gi];
  const bool relayed = rr >= 0 && p >= 0 && p < P && slot_partition[p] >= relays;
  if (lane == 0) comb_row[gi] = relayed ? (int32_t)(n_routes + rr) : rr;
  if (!relayed) return;
  const uint4 *src = (const uint4 *)(ret + (int64_t)rr * H);
  uint4 *dst = (uint4 *)(ret + (n_routes + rr) * H);
  for (int i = lane; i < H / 8; i += 64) dst[i] = src[i];
}
}  // namespace
}  // namespace moe

extern "C" int moe_relay_returns(uint16_t *ret, const int32_t *phys_ids,
                                 const int32_t *slot_partition, const int32_t *ret_row,
                                 const moe_geom_t *g, int32_t *comb_row, void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (!ret || !phys_ids || !slot_partition || !ret_row || !comb_row) return MOE_ERR_INVALID_ARG;
  if (g->relays <= 0 || !aligned16(ret)) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)g->T * g->k;
  if (n == 0) return MOE_OK;
  hipLaunchKernelGGL(relay_returns_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0,
                     (hipStream_t)stream, ret, phys_ids, slot_partition, ret_row, n, g->P, g->H,
                     g->relays, comb_row);
  return launch_status();
}
