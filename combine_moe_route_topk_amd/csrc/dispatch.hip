// INT8 dispatch: slot allocation (count phase) + token-wise quantization fused
// into the scatter of k message copies into static per-partition regions.
//
// [XDS 合设 A2A, P039-P040 and Fig. 7: histogram routes per receiver, write
//  {count, offset} metadata, wait for every sender's metadata, prefix-sum the
//  received counts, move the data; CMI EP320 FusedDispatch: quantize BF16 to
//  INT8 + scale early and write message + source info into the target's
//  static buffer; XDS 解耦 A2A P045 / Fig. 8: two-hop trampoline.]
//
// One GPU plays every partition, so the pages' "broadcast counts, then wait
// for all ranks" barrier becomes the boundary between kernels:
//   1. count    one block per chunk of <= 256 routes (never straddling a source
//               partition): stable in-chunk ranks of each route among the
//               routes with the same destination partition d and the same slot
//               p, by wavefront ballot multisplit (match masks from one ballot
//               per key bit, rank = popcount below the lane) plus per-wave
//               counts in LDS; writes per-chunk histograms over d and over p.
//   2. scan     one block per d and per p: exclusive prefix of the chunk
//               histograms in (source, chunk) order.  For d this single prefix
//               is both the receive layout offset of source s (its value at
//               s's first chunk) and, relative to it, the chunk's base row in
//               region (d, s); the d blocks write meta, the p blocks
//               slot_count / slot_local; the status word is cleared.
//   3. scatter  every block first prefixes slot_count into the slots' first
//               rows (block 0 stores them as slot_offset); then one wavefront
//               per token: amax, scale, IEEE divide + RNE to int8, 16-byte
//               stores of the k message rows and trailers.
//   4. relay    (two-hop only) second hop: relay region rows -> final region.
// Decode-size batches (at most 1024 routes, no relay hop) take one launch
// instead (dispatch_small_kernel): the same layout, ranked in LDS by every
// block, and one wavefront per 1024-element slice of a token.
// No atomics decide any order: every row index is a deterministic function of
// the routes, so the layout is bit-identical run to run.
#include <algorithm>
#include <atomic>

#include "common.h"

namespace moe {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// lanes of the wavefront holding the same key (0 for invalid lanes)
__device__ __forceinline__ uint64_t match_any(int key, int nbits, bool valid) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

// Lanes that write a message's trailer line whole: the trailer (lane 0), then
// zeros over the row's padding up to the end of the 128-byte line that holds
// the trailer, or the row's end if that comes first.
__device__ __forceinline__ int trailer_line_lanes(int H, int64_t msg) {
  const int64_t end = min(msg, (int64_t)((H + 16 + 127) & ~127));
  return 1 + (int)((end - (H + 16)) / 16);
}

__device__ __forceinline__ int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// ---------------------------------------------------------------- count ---
__global__ __launch_bounds__(256) void dispatch_count_kernel(
    const int32_t *__restrict__ phys, const int32_t *__restrict__ slot_partition, int T, int k,
    int P, int D, int LB, int ct, int cps, int nc, int32_t *__restrict__ hist_d,
    int32_t *__restrict__ hist_p, int32_t *__restrict__ route_rank) {
  extern __shared__ int32_t lds[];
  int32_t *wd = lds;              // [4][D]
  int32_t *wp = lds + 4 * D;      // [4][P]
  const int c = blockIdx.x;
  const int s = c / cps, ci = c % cps;
  const int64_t t0 = (int64_t)s * LB + (int64_t)ci * ct;
  const int64_t t1 = min(t0 + ct, (int64_t)(s + 1) * LB);
  const int n = (int)(t1 - t0) * k;
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * (D + P); i += 256) lds[i] = 0;
  __syncthreads();

  const int64_t gi = t0 * k + tid;
  int p = -1, d = -1, bad = 0;
  if (tid < n) {
    p = phys[gi];
    if (p < 0 || p >= P) {
      bad = -1;
    } else {
      d = slot_partition[p];
      if (d < 0 || d >= D) bad = -2;
    }
  }
  const bool valid = tid < n && bad == 0;
  const uint64_t lt = lanemask_lt();
  const uint64_t md = match_any(d, bits_for(D), valid);
  const uint64_t mp = match_any(p, bits_for(P), valid);
  const int rd = __popcll(md & lt), rp = __popcll(mp & lt);
  if (valid && rd == 0) wd[wave * D + d] = __popcll(md);
  if (valid && rp == 0) wp[wave * P + p] = __popcll(mp);
  __syncthreads();
  if (tid < n) {
    if (valid) {
      int bd = rd, bp = rp;
      for (int w = 0; w < wave; ++w) {
        bd += wd[w * D + d];
        bp += wp[w * P + p];
      }
      route_rank[gi] = bd | (bp << 16);
    } else {
      route_rank[gi] = bad;
    }
  }
  for (int i = tid; i < D; i += 256)
    hist_d[(int64_t)i * (nc + 1) + c] = wd[i] + wd[D + i] + wd[2 * D + i] + wd[3 * D + i];
  for (int i = tid; i < P; i += 256)
    hist_p[(int64_t)i * (nc + 1) + c] = wp[i] + wp[P + i] + wp[2 * P + i] + wp[3 * P + i];
}

// ----------------------------------------------------------------- scan ---
// Block b < D scans hist_d row b, block D + p scans hist_p row p: in place,
// exclusive over the nc chunks, total in column nc.
__device__ __forceinline__ int block_incl_scan_256(int v, int *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += sh[w];
  __syncthreads();
  return v + add;
}

// Block b < D scans hist_d row b and writes meta[b][s] = {event, prefix at
// s's first chunk, count} for every source s; block D + p scans hist_p row p
// and writes slot_count[p] and slot_local[p].  Scans are exclusive over the nc
// chunks, the total goes to column nc.  Block 0 clears the status word.  The
// slot totals' prefix (slot_offset) is taken by every scatter block from
// slot_count, so no block here waits for the others.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(
    int32_t *__restrict__ hist_d, int32_t *__restrict__ hist_p,
    const int32_t *__restrict__ slot_partition, int D, int P, int S, int cps, int nc,
    uint32_t event_id, moe_meta_t *__restrict__ meta, int32_t *__restrict__ slot_count,
    int32_t *__restrict__ slot_local, int32_t *__restrict__ status) {
  __shared__ int sh[4];
  __shared__ int carry_sh;
  const bool is_d = blockIdx.x < (unsigned)D;
  const int row = is_d ? blockIdx.x : blockIdx.x - D;
  int32_t *h = (is_d ? hist_d : hist_p) + (int64_t)row * (nc + 1);
  int carry = 0;
  for (int base = 0; base < nc; base += 256) {
    const int c = base + threadIdx.x;
    const int v = c < nc ? h[c] : 0;
    const int incl = block_incl_scan_256(v, sh);
    if (c < nc) h[c] = carry + incl - v;
    if (threadIdx.x == 255) carry_sh = incl;
    __syncthreads();
    carry += carry_sh;
    __syncthreads();
  }
  if (threadIdx.x == 0) h[nc] = carry;
  if (is_d) {
    __syncthreads();  // the block's scanned row is visible to all its threads
    for (int src = threadIdx.x; src < S; src += 256) {
      const int a = h[src * cps], b = h[(src + 1) * cps];  // (src + 1) * cps <= nc
      moe_meta_t m;
      m.event_id = event_id;
      m.offset = a;
      m.count = b - a;
      m.reserved = 0;
      meta[(int64_t)row * S + src] = m;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
    return;
  }
  // slot_local[row]: index of the slot among the slots of its partition
  {
    const int d = slot_partition[row];
    int nloc = 0;
    for (int q = threadIdx.x; q < row; q += 256) nloc += slot_partition[q] == d;
    for (int o = 32; o > 0; o >>= 1) nloc += __shfl_xor(nloc, o, 64);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = nloc;
    __syncthreads();
    if (threadIdx.x == 0) slot_local[row] = sh[0] + sh[1] + sh[2] + sh[3];
  }
  if (threadIdx.x == 0) slot_count[row] = carry;
}

// -------------------------------------------------------------- scatter ---
// One wavefront per token.  Lane l, iteration i covers elements
// [(i*64 + l)*16, +16) of the row: 32 B (bf16) or 64 B (fp32) loads and one
// 16-byte int8 store per message copy.  The token rows are read once: bf16
// rows come in by non-temporal loads (non-temporal stores of the messages
// measured slower, ordinary stores are kept).  Each 16-value chunk goes to
// every route's row as soon as its codes exist, so no register copy of the
// whole quantized row is kept (107 instead of 149 registers per lane for
// bf16 rows of 7168 values).
// PER_ROUTE (small batches, to spread them over the GPU): one wavefront per
// route instead of per token; it quantizes its token exactly as the token's
// wavefront would and writes that route's copy only.
template <int NIT, bool BF16, bool PER_ROUTE>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const void *__restrict__ x, const int32_t *__restrict__ phys,
    const int32_t *__restrict__ slot_partition, const int32_t *__restrict__ slot_local,
    const int32_t *__restrict__ hist_d, const int32_t *__restrict__ hist_p,
    const int32_t *__restrict__ route_rank, const int32_t *__restrict__ slot_count,
    int32_t *__restrict__ slot_offset, int T, int H, int k, int S, int P, int LB, int ct,
    int cps, int nc, int64_t cap, int64_t msg, int relays, uint32_t event_id,
    uint8_t *__restrict__ disp_buf, uint8_t *__restrict__ relay_buf,
    int32_t *__restrict__ slot_rows, int32_t *__restrict__ disp_row,
    int32_t *__restrict__ ret_row, int32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = PER_ROUTE ? wv / k : wv;
  const int jsel = PER_ROUTE ? (int)(wv % k) : 0;  // the wavefront's route (PER_ROUTE)
  const bool live = t < T;
  const bool mine = live && (PER_ROUTE ? lane == jsel : lane < k);  // lanes with a route

  // ---- loads first: the token row and the routes' ranks and slots, whose
  // latency then overlaps the slot prefix below and the lookups after it ----
  uint4 raw[NIT][BF16 ? 2 : 4];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int e0 = (i * 64 + lane) * 16;
    if (live && e0 < H) {
      if (BF16) {
        const v4u *src = (const v4u *)((const uint16_t *)x + t * H + e0);
        const v4u a0 = __builtin_nontemporal_load(src), a1 = __builtin_nontemporal_load(src + 1);
        raw[i][0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
        raw[i][1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
      } else {
        const uint4 *src = (const uint4 *)((const float *)x + t * H + e0);
#pragma unroll
        for (int q = 0; q < (BF16 ? 2 : 4); ++q) raw[i][q] = src[q];
      }
    }
  }
  const int64_t gi = t * k + lane;
  int rr = 0, p = 0;
  if (mine) {
    rr = route_rank[gi];
    p = phys[gi];
  }

  // the slots' first dense rows: an exclusive prefix of slot_count (1 KB at
  // P = 256, from L2), taken by every block; block 0 also stores it as
  // slot_offset [P + 1]
  __shared__ int32_t soff[MOE_MAX_P + 1];
  __shared__ int sh[4];
  __shared__ int carry_sh;
  {
    int carry = 0;
    for (int base = 0; base < P; base += 256) {
      const int q = base + threadIdx.x;
      const int v = q < P ? slot_count[q] : 0;
      const int incl = block_incl_scan_256(v, sh);
      if (q < P) soff[q] = carry + incl - v;
      if (threadIdx.x == 255) carry_sh = incl;
      __syncthreads();
      carry += carry_sh;
      __syncthreads();
    }
    if (threadIdx.x == 0) soff[P] = carry;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int q = threadIdx.x; q <= P; q += 256) slot_offset[q] = soff[q];
  }
  if (!live) return;
  const int s = (int)(t / LB), b = (int)(t % LB);
  const int c = s * cps + b / ct;

  // ---- per-route row indices (lanes 0..k-1, or the wavefront's route) ----
  int64_t drow = -1;
  int dpart = 0;
  uint32_t tail_w = 0;
  if (mine) {
    int32_t out_d = -1, out_r = -1;
    if (rr < 0) {
      atomicOr(status, rr == -1 ? MOE_DEVICE_BAD_ROUTE : MOE_DEVICE_BAD_PARTITION);
    } else {
      const int d = slot_partition[p];
      const int32_t *hd = hist_d + (int64_t)d * (nc + 1);
      const int64_t r = (int64_t)(hd[c] - hd[s * cps]) + (rr & 0xffff);
      const int32_t rrow = soff[p] + hist_p[(int64_t)p * (nc + 1) + c] + (rr >> 16);
      out_r = rrow;
      if (r >= cap) {
        atomicOr(status, MOE_DEVICE_OVER_CAPACITY);
        slot_rows[rrow] = -1;
      } else {
        drow = ((int64_t)d * S + s) * cap + r;
        dpart = d;
        out_d = (int32_t)drow;
        slot_rows[rrow] = out_d;
        tail_w = (uint32_t)lane | ((uint32_t)(slot_local[p] & 0xff) << 8) |
                 ((event_id & 0xffffu) << 16);
      }
    }
    disp_row[gi] = out_d;
    ret_row[gi] = out_r;
  }

  // ---- quantize ----
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int e0 = (i * 64 + lane) * 16;
    if (e0 < H) {
      if (BF16) {
        const uint32_t *w = (const uint32_t *)&raw[i][0];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] & 0xffffu)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] >> 16)));
        }
      } else {
        const float *f = (const float *)&raw[i][0];
#pragma unroll
        for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(f[q]));
      }
    }
  }
  amax = wave_max_f32(amax);
  const float scale = amax / 127.0f;
  // bf16 rows: v / scale as the row's reciprocal and one Markstein step,
  // q0 = v r, q = fma(fma(-q0, scale, v), r, q0), whose code equals the IEEE
  // quotient's for every pair of bf16 values |v| <= amax when scale >= 2^-100
  // (checked for all such pairs on the host); an infinite or tiny scale keeps
  // the division (rs = 0)
  const float rs = BF16 && scale >= 0x1p-100f ? 1.0f / scale : 0.0f;
  // the wavefront's amax, hence rs, is the same in every lane: one branch
  // picks the quotient for the whole row
  const bool fast = BF16 && __builtin_amdgcn_readfirstlane(rs != 0.0f ? 1 : 0) != 0;

  // the codes of chunk i (16 values), with quotient quot
  auto chunk_codes = [&](int i, auto quot) __attribute__((always_inline)) {
    float v[16];
    if (BF16) {
      const uint32_t *w = (const uint32_t *)&raw[i][0];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
        v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
      }
    } else {
      const float *f = (const float *)&raw[i][0];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = f[q];
    }
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int code = 0;
        if (scale != 0.0f) {
          float y = rintf(quot(v[4 * q + r]));
          y = fminf(fmaxf(y, -127.0f), 127.0f);
          code = (int)y;
        }
        word |= ((uint32_t)code & 0xffu) << (8 * r);
      }
      pk[q] = word;
    }
    return make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };

  // ---- k message copies, chunk by chunk: each chunk's codes go to every
  // route's row as soon as they exist (no register copy of the whole row) ----
  const int64_t relay_base = (int64_t)relays * S * cap;
  const int jend = PER_ROUTE ? jsel + 1 : k;
  const int drow_lo = (int)(uint32_t)drow, drow_hi = (int)(drow >> 32);
  auto dst_of = [&](int j) __attribute__((always_inline)) -> uint8_t * {
    const int64_t row = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(drow_hi, j) << 32) |
                                  (uint32_t)__builtin_amdgcn_readlane(drow_lo, j));
    if (row < 0) return nullptr;
    const int d = __builtin_amdgcn_readlane(dpart, j);
    return (relays > 0 && d >= relays) ? relay_buf + (row - relay_base) * msg : disp_buf + row * msg;
  };
  auto emit = [&](auto quot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int e0 = (i * 64 + lane) * 16;
      const uint4 cv = chunk_codes(i, quot);
      for (int j = jsel; j < jend; ++j) {
        uint8_t *dst = dst_of(j);
        if (dst && e0 < H) *(uint4 *)(dst + e0) = cv;
      }
    }
  };
  if (fast)
    emit([&](float y) __attribute__((always_inline)) {
      const float q0 = y * rs;
      return fmaf(fmaf(-q0, scale, y), rs, q0);
    });
  else
    emit([&](float y) __attribute__((always_inline)) { return y / scale; });
  // The trailer's 128-byte line is written whole: lanes after the first fill
  // the row's padding behind the trailer with zeros up to the line's end (never
  // past the row).  A 16-byte store alone leaves a partly written line, which
  // the memory side completes with a read (233 -> 205 us per layer12288
  // dispatch, the message bytes unchanged).
  const int tail_lanes = trailer_line_lanes(H, msg);
  for (int j = jsel; j < jend; ++j) {
    uint8_t *dst = dst_of(j);
    const uint32_t tw = (uint32_t)__builtin_amdgcn_readlane((int)tail_w, j);
    if (dst && lane < tail_lanes)
      *(uint4 *)(dst + H + 16 * lane) =
          lane == 0 ? make_uint4(__float_as_uint(scale), (uint32_t)s, (uint32_t)b, tw)
                    : make_uint4(0u, 0u, 0u, 0u);
  }
}

// -------------------------------------------------------- small batches ---
// Decode-size batches (at most kSmallRoutes routes, D x S <= kSmallRegions,
// no relay hop): count, scan and scatter in one launch.  Every block ranks all
// T k routes in LDS: a route's row in region (d, s) is the number of valid
// routes before it (route order t k + j) with the same d and s, and its slot
// row the number before it with the same slot after the earlier slots'
// totals -- the layout the three-kernel path builds from its chunk prefixes.
// Wavefront w takes token w / ns and its 1024-element slice w % ns for all k
// copies (the token's amax from a first pass over the whole row), so no
// wavefront quantizes more than a slice.  Block 0 also writes meta, the slot
// counts and offsets, and the status word: every error bit of the batch,
// written whole (no other block touches it).
constexpr int kSmallRoutes = 1024, kSmallRegions = 4096;

template <bool BF16>
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const void *__restrict__ x, const int32_t *__restrict__ phys,
    const int32_t *__restrict__ slot_partition, int T, int H, int k, int S, int P, int D, int LB,
    int ns, int64_t cap, int64_t msg, uint32_t event_id, uint8_t *__restrict__ disp_buf,
    moe_meta_t *__restrict__ meta, int32_t *__restrict__ slot_count,
    int32_t *__restrict__ slot_offset, int32_t *__restrict__ slot_rows,
    int32_t *__restrict__ disp_row, int32_t *__restrict__ ret_row, int32_t *__restrict__ status) {
  __shared__ int32_t kd[kSmallRoutes];    // region d S + s of each route; -2 bad slot, -3 bad partition
  __shared__ int32_t kp[kSmallRoutes];    // slot of each valid route, else -1
  __shared__ int32_t spart[MOE_MAX_P];    // slot_partition
  __shared__ int32_t soff[MOE_MAX_P + 1]; // slot totals, then their exclusive prefix
  __shared__ int32_t region[kSmallRegions];
  __shared__ int sh[4];
  __shared__ int carry_sh, bits_sh;
  const int N = T * k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (tid >> 6);
  const int64_t t = wv / ns;
  const int slice = (int)(wv % ns);
  const bool live = t < T;

  // ---- the layout, in every block ----
  for (int q = tid; q < P; q += 256) {
    spart[q] = slot_partition[q];
    soff[q] = 0;
  }
  const bool b0 = blockIdx.x == 0;
  if (b0)
    for (int r = tid; r < D * S; r += 256) region[r] = 0;
  if (tid == 0) bits_sh = 0;
  __syncthreads();
  int bits = 0;
  for (int g = tid; g < N; g += 256) {
    const int p = phys[g];
    int keyd = -2, keyp = -1;
    if (p >= 0 && p < P) {
      const int d = spart[p];
      if (d >= 0 && d < D) {
        keyd = d * S + (g / k) / LB;
        keyp = p;
        atomicAdd(&soff[p], 1);
        if (b0) atomicAdd(&region[keyd], 1);
      } else {
        keyd = -3;
        bits |= MOE_DEVICE_BAD_PARTITION;
      }
    } else {
      bits |= MOE_DEVICE_BAD_ROUTE;
    }
    kd[g] = keyd;
    kp[g] = keyp;
  }
  if (b0 && bits) atomicOr(&bits_sh, bits);
  __syncthreads();
  {
    int carry = 0;
    for (int base = 0; base < P; base += 256) {
      const int q = base + tid;
      const int v = q < P ? soff[q] : 0;
      const int incl = block_incl_scan_256(v, sh);
      if (q < P) soff[q] = carry + incl - v;
      if (tid == 255) carry_sh = incl;
      __syncthreads();
      carry += carry_sh;
      __syncthreads();
    }
    if (tid == 0) soff[P] = carry;
    __syncthreads();
  }
  if (b0) {
    for (int q = tid; q <= P; q += 256) {
      slot_offset[q] = soff[q];
      if (q < P) slot_count[q] = soff[q + 1] - soff[q];
    }
    int over = 0;
    for (int d = tid; d < D; d += 256) {
      int off = 0;
      for (int src = 0; src < S; ++src) {
        const int c = region[d * S + src];
        moe_meta_t m;
        m.event_id = event_id;
        m.offset = off;
        m.count = c;
        m.reserved = 0;
        meta[(int64_t)d * S + src] = m;
        off += c;
        if (c > cap) over = MOE_DEVICE_OVER_CAPACITY;
      }
    }
    if (over) atomicOr(&bits_sh, over);
    __syncthreads();
    if (tid == 0) *status = bits_sh;
  }
  // ---- ranks of this block's routes (its waves cover tokens t0 .. t1) ----
  // nr routes, tpr threads each (a power of two, at least 4, within one
  // wavefront): thread (r, seg) counts the matches among routes seg, seg + tpr,
  // ... before route r, then the tpr partial counts are summed by shuffles
  __shared__ int32_t rk_d[64], rk_p[64], rk_loc[64];
  const int64_t t0 = (int64_t)blockIdx.x * 4 / ns;
  const int64_t t1 = min(((int64_t)blockIdx.x * 4 + 3) / ns, (int64_t)T - 1);
  const int nr = (int)(t1 - t0 + 1) * k;  // <= 4 k <= 64
  int tpr = 64;
  while (tpr > 4 && tpr * nr > 256) tpr >>= 1;
  {
    const int r = tid / tpr, seg = tid % tpr;
    int cd = 0, cp = 0, cl = 0;
    const int gr = (int)(t0 * k) + r;
    const bool act = r < nr && gr < N;
    const int kdr = act ? kd[gr] : -1, kpr = act ? kp[gr] : -1;
    if (kdr >= 0) {
      for (int g = seg; g < gr; g += tpr) {
        cd += kd[g] == kdr;
        cp += kp[g] == kpr;
      }
      const int dr = spart[kpr];
      for (int q = seg; q < kpr; q += tpr) cl += spart[q] == dr;
    }
    for (int o = tpr >> 1; o > 0; o >>= 1) {
      cd += __shfl_xor(cd, o, 64);
      cp += __shfl_xor(cp, o, 64);
      cl += __shfl_xor(cl, o, 64);
    }
    if (act && seg == 0) {
      rk_d[r] = cd;
      rk_p[r] = cp;
      rk_loc[r] = cl;
    }
    __syncthreads();
  }
  if (!live) return;

  // ---- the token's k routes (lane j: route j) ----
  const int src_s = (int)(t / LB), bpos = (int)(t % LB);
  int64_t drow = -1;
  int32_t rrow = -1;
  uint32_t tail_w = 0;
  if (lane < k) {
    const int gi = (int)(t * k + lane);
    const int kdj = kd[gi], kpj = kp[gi];
    if (kdj >= 0) {
      const int r = gi - (int)(t0 * k);
      const int cd = rk_d[r];
      drow = cd < cap ? (int64_t)kdj * cap + cd : -1;
      rrow = soff[kpj] + rk_p[r];
      tail_w = (uint32_t)lane | ((uint32_t)(rk_loc[r] & 0xff) << 8) | ((event_id & 0xffffu) << 16);
    }
  }
  if (slice == 0 && lane < k) {
    const int64_t gi = t * k + lane;
    if (rrow >= 0) slot_rows[rrow] = drow >= 0 ? (int32_t)drow : -1;
    disp_row[gi] = drow >= 0 ? (int32_t)drow : -1;
    ret_row[gi] = rrow;
  }

  // ---- amax over the row, then this wavefront's slice into every copy ----
  float amax = 0.0f;
  for (int i = 0; i * 1024 < H; ++i) {
    const int e0 = (i * 64 + lane) * 16;
    if (e0 < H) {
      if (BF16) {
        const v4u *sp = (const v4u *)((const uint16_t *)x + t * H + e0);
        const v4u a0 = sp[0], a1 = sp[1];
        const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] & 0xffffu)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] >> 16)));
        }
      } else {
        const float4 *fp = (const float4 *)((const float *)x + t * H + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = fp[q];
          amax = fmaxf(amax, fabsf(f.x));
          amax = fmaxf(amax, fabsf(f.y));
          amax = fmaxf(amax, fabsf(f.z));
          amax = fmaxf(amax, fabsf(f.w));
        }
      }
    }
  }
  amax = wave_max_f32(amax);
  const float scale = amax / 127.0f;
  const int e0 = (slice * 64 + lane) * 16;
  uint4 code = make_uint4(0u, 0u, 0u, 0u);
  if (e0 < H) {
    float v[16];
    if (BF16) {
      const v4u *sp = (const v4u *)((const uint16_t *)x + t * H + e0);
      const v4u a0 = sp[0], a1 = sp[1];
      const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
        v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
      }
    } else {
      const float *f = (const float *)x + t * H + e0;
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = f[q];
    }
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int c = 0;
        if (scale != 0.0f) {
          float y = rintf(v[4 * q + r] / scale);
          y = fminf(fmaxf(y, -127.0f), 127.0f);
          c = (int)y;
        }
        word |= ((uint32_t)c & 0xffu) << (8 * r);
      }
      pk[q] = word;
    }
    code = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  const int tail_lanes = trailer_line_lanes(H, msg);
  for (int j = 0; j < k; ++j) {
    const int64_t row = __shfl(drow, j, 64);  // with every lane active
    const uint32_t tw = __shfl(tail_w, j, 64);
    if (row < 0) continue;
    uint8_t *dst = disp_buf + row * msg;
    if (e0 < H) *(uint4 *)(dst + e0) = code;
    if (slice == 0 && lane < tail_lanes)  // the trailer's line whole, as in the scatter
      *(uint4 *)(dst + H + 16 * lane) =
          lane == 0 ? make_uint4(__float_as_uint(scale), (uint32_t)src_s, (uint32_t)bpos, tw)
                    : make_uint4(0u, 0u, 0u, 0u);
  }
}

// ---------------------------------------------------------------- relay ---
// Second hop: each route whose partition is >= relays moves its message row
// from the relay region to its final region (same region-relative row).
__global__ __launch_bounds__(256) void dispatch_relay_kernel(
    const int32_t *__restrict__ disp_row, int64_t n_routes, int64_t relay_base, int64_t msg,
    const uint8_t *__restrict__ relay_buf, uint8_t *__restrict__ disp_buf) {
  const int lane = threadIdx.x & 63;
  const int64_t gi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gi >= n_routes) return;
  const int64_t row = disp_row[gi];
  if (row < relay_base) return;  // direct route (or dropped: -1)
  const uint4 *src = (const uint4 *)(relay_buf + (row - relay_base) * msg);
  uint4 *dst = (uint4 *)(disp_buf + row * msg);
  for (int64_t i = lane; i < msg / 16; i += 64) dst[i] = src[i];
}

// Empty batch: meta = {event, 0, 0}, zero slot counts and offsets, clear status.
__global__ void dispatch_empty_kernel(int D, int S, int P, uint32_t event_id,
                                      moe_meta_t *__restrict__ meta,
                                      int32_t *__restrict__ slot_count,
                                      int32_t *__restrict__ slot_offset,
                                      int32_t *__restrict__ status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nm = (int64_t)D * S;
  if (i < nm) {
    moe_meta_t m;
    m.event_id = event_id;
    m.offset = 0;
    m.count = 0;
    m.reserved = 0;
    meta[i] = m;
  } else if (i < nm + P) {
    slot_count[i - nm] = 0;
    slot_offset[i - nm] = 0;
  } else if (i == nm + P) {
    slot_offset[P] = 0;
    *status = 0;
  }
}

template <int NIT, bool PR>
void launch_scatter2(bool bf16, dim3 grid, hipStream_t st, const void *x, const int32_t *phys,
                     const int32_t *sp, const int32_t *sl, const int32_t *hd, const int32_t *hp,
                     const int32_t *rr, const int32_t *scount, int32_t *so, const moe_geom_t &g,
                     int ct, int cps, int nc, int64_t cap, int64_t msg, uint32_t ev, uint8_t *db,
                     uint8_t *rb, int32_t *srows, int32_t *drow, int32_t *rrow, int32_t *status) {
  if (bf16)
    hipLaunchKernelGGL((dispatch_scatter_kernel<NIT, true, PR>), grid, dim3(256), 0, st, x, phys,
                       sp, sl, hd, hp, rr, scount, so, g.T, g.H, g.k, g.S, g.P, g.LB, ct, cps, nc,
                       cap, msg, g.relays, ev, db, rb, srows, drow, rrow, status);
  else
    hipLaunchKernelGGL((dispatch_scatter_kernel<NIT, false, PR>), grid, dim3(256), 0, st, x, phys,
                       sp, sl, hd, hp, rr, scount, so, g.T, g.H, g.k, g.S, g.P, g.LB, ct, cps, nc,
                       cap, msg, g.relays, ev, db, rb, srows, drow, rrow, status);
}

// One wavefront per token, or per route when the tokens alone would give
// fewer blocks than the GPU has CUs (decode batches).
template <int NIT>
void launch_scatter(bool bf16, hipStream_t st, const void *x, const int32_t *phys,
                    const int32_t *sp, const int32_t *sl, const int32_t *hd, const int32_t *hp,
                    const int32_t *rr, const int32_t *scount, int32_t *so, const moe_geom_t &g,
                    int ct, int cps, int nc, int64_t cap, int64_t msg, uint32_t ev, uint8_t *db,
                    uint8_t *rb, int32_t *srows, int32_t *drow, int32_t *rrow, int32_t *status) {
  const bool per_route = (g.T + 3) / 4 < 256;
  const int64_t waves = per_route ? (int64_t)g.T * g.k : g.T;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (per_route)
    launch_scatter2<NIT, true>(bf16, grid, st, x, phys, sp, sl, hd, hp, rr, scount, so, g, ct,
                               cps, nc, cap, msg, ev, db, rb, srows, drow, rrow, status);
  else
    launch_scatter2<NIT, false>(bf16, grid, st, x, phys, sp, sl, hd, hp, rr, scount, so, g, ct,
                                cps, nc, cap, msg, ev, db, rb, srows, drow, rrow, status);
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {
namespace {
int dispatch_impl(const void *x, moe_dtype_t x_dtype, const int32_t *phys_ids,
                  const int32_t *slot_partition, uint32_t event_id, const moe_geom_t *g,
                  void *disp_buf, moe_meta_t *meta, int32_t *slot_count, int32_t *slot_offset,
                  int32_t *slot_rows, int32_t *disp_row, int32_t *ret_row, void *relay_buf,
                  void *scratch, size_t scratch_bytes, void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (!slot_partition || !meta || !slot_count || !slot_offset || !scratch) return MOE_ERR_INVALID_ARG;
  if (g->T > 0 && (!x || !phys_ids || !disp_buf || !slot_rows || !disp_row || !ret_row))
    return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(disp_buf) || !aligned16(scratch)) return MOE_ERR_INVALID_ARG;
  if (g->T > 0 && g->relays > 0 && (!relay_buf || !aligned16(relay_buf))) return MOE_ERR_INVALID_ARG;
  const DispatchScratch L = dispatch_scratch_layout(*g);
  if ((int64_t)scratch_bytes < L.total) return MOE_ERR_CAPACITY;
  if (g->T == 0) {
    // empty batch: every count is zero, the layout is empty
    const unsigned blocks = (unsigned)(((int64_t)g->D * g->S + g->P + 1 + 255) / 256);
    hipLaunchKernelGGL(dispatch_empty_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       g->D, g->S, g->P, event_id, meta, slot_count, slot_offset,
                       (int32_t *)((uint8_t *)scratch + L.status));
    return launch_status();
  }

  hipStream_t s = (hipStream_t)stream;
  uint8_t *sc = (uint8_t *)scratch;
  int32_t *status = (int32_t *)(sc + L.status);
  const int64_t cap = cap_of(*g), msg = msg_bytes_of(*g);
  if (g->relays == 0 && (int64_t)g->T * g->k <= kSmallRoutes &&
      (int64_t)g->D * g->S <= kSmallRegions) {
    const int ns = (g->H + 1023) / 1024;
    const dim3 grid((unsigned)(((int64_t)g->T * ns + 3) / 4));
    if (x_dtype == MOE_DTYPE_BF16)
      hipLaunchKernelGGL(dispatch_small_kernel<true>, grid, dim3(256), 0, s, x, phys_ids,
                         slot_partition, g->T, g->H, g->k, g->S, g->P, g->D, g->LB, ns, cap, msg,
                         event_id, (uint8_t *)disp_buf, meta, slot_count, slot_offset, slot_rows,
                         disp_row, ret_row, status);
    else
      hipLaunchKernelGGL(dispatch_small_kernel<false>, grid, dim3(256), 0, s, x, phys_ids,
                         slot_partition, g->T, g->H, g->k, g->S, g->P, g->D, g->LB, ns, cap, msg,
                         event_id, (uint8_t *)disp_buf, meta, slot_count, slot_offset, slot_rows,
                         disp_row, ret_row, status);
    return launch_status();
  }
  int32_t *hist_d = (int32_t *)(sc + L.hist_d);
  int32_t *hist_p = (int32_t *)(sc + L.hist_p);
  int32_t *route_rank = (int32_t *)(sc + L.route_rank);
  int32_t *slot_local = (int32_t *)(sc + L.slot_local);
  const int ct = chunk_tokens(*g);
  const int cps = (int)chunks_per_source(*g);
  const int nc = g->S * cps;

  const size_t lds = sizeof(int32_t) * 4 * (g->D + g->P);
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nc), dim3(256), lds, s, phys_ids, slot_partition,
                     g->T, g->k, g->P, g->D, g->LB, ct, cps, nc, hist_d, hist_p, route_rank);
  if ((st = launch_status()) != MOE_OK) return st;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(g->D + g->P), dim3(256), 0, s, hist_d, hist_p,
                     slot_partition, g->D, g->P, g->S, cps, nc, event_id, meta, slot_count,
                     slot_local, status);
  if ((st = launch_status()) != MOE_OK) return st;

  const bool bf16 = x_dtype == MOE_DTYPE_BF16;
  uint8_t *db = (uint8_t *)disp_buf, *rb = (uint8_t *)relay_buf;
  const int nit = (g->H + 1023) / 1024;
#define MOE_SCATTER(N)                                                                         \
  launch_scatter<N>(bf16, s, x, phys_ids, slot_partition, slot_local, hist_d, hist_p,           \
                    route_rank, slot_count, slot_offset, *g, ct, cps, nc, cap, msg, event_id, db, \
                    rb, slot_rows, disp_row, ret_row, status)
  if (nit <= 1)
    MOE_SCATTER(1);
  else if (nit <= 2)
    MOE_SCATTER(2);
  else if (nit <= 4)
    MOE_SCATTER(4);
  else if (nit <= 8)
    MOE_SCATTER(8);
  else
    MOE_SCATTER(16);
#undef MOE_SCATTER
  if ((st = launch_status()) != MOE_OK) return st;

  if (g->relays > 0) {
    const int64_t n = (int64_t)g->T * g->k;
    hipLaunchKernelGGL(dispatch_relay_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s,
                       disp_row, n, (int64_t)g->relays * g->S * cap, msg, rb, db);
    if ((st = launch_status()) != MOE_OK) return st;
  }
  return MOE_OK;
}

__global__ void clear_status_kernel(int32_t *__restrict__ status) {
  if (threadIdx.x == 0) *status = 0;
}

// The receiver's event check: meta entries first, then the trailers of the
// routed rows (event_lo is the top half of the trailer's last word).
__global__ __launch_bounds__(256) void check_event_kernel(
    const moe_meta_t *__restrict__ meta, int64_t nmeta, const uint8_t *__restrict__ disp_buf,
    int64_t msg, int H, const int32_t *__restrict__ slot_rows,
    const int32_t *__restrict__ slot_offset, int P, uint32_t event_id,
    int32_t *__restrict__ status) {
  const int64_t n = slot_offset[P];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool stale = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nmeta + n; i += stride) {
    if (i < nmeta) {
      stale |= meta[i].event_id != event_id;
    } else {
      const int32_t dr = slot_rows[i - nmeta];
      if (dr >= 0) {
        const uint32_t tw = *(const uint32_t *)(disp_buf + (int64_t)dr * msg + H + 12);
        stale |= (tw >> 16) != (event_id & 0xffffu);
      }
    }
  }
  if (stale) atomicOr(status, MOE_DEVICE_STALE_EVENT);
}

// Copies the device status word of a dispatch into the caller's int32.
__global__ void copy_status_kernel(const int32_t *__restrict__ src, int32_t *__restrict__ dst) {
  if (threadIdx.x == 0) *dst = *src;
}

// The allocation-free variant's scratch: one copy per GPU, held until the
// process ends.  In host code this name stands for the host-side shadow, not a
// device address: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_static_scratch[kMaxDevices];

// Device address of the current device's static scratch (looked up on the first
// call on that device); nullptr on a HIP error.
void *static_scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_static_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void *q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_static_scratch[dev].store(q, std::memory_order_release);  // same address if two threads race
  return q;
}
}  // namespace
}  // namespace moe

extern "C" int moe_dispatch_q8(const void *x, moe_dtype_t x_dtype, const int32_t *phys_ids,
                               const int32_t *slot_partition, uint32_t event_id,
                               const moe_geom_t *g, void *disp_buf, moe_meta_t *meta,
                               int32_t *slot_count, int32_t *slot_offset, int32_t *slot_rows,
                               int32_t *disp_row, int32_t *ret_row, void *relay_buf, void *scratch,
                               size_t scratch_bytes, void *stream) {
  return dispatch_impl(x, x_dtype, phys_ids, slot_partition, event_id, g, disp_buf, meta,
                       slot_count, slot_offset, slot_rows, disp_row, ret_row, relay_buf, scratch,
                       scratch_bytes, stream);
}

extern "C" int moe_dispatch_q8_static(const void *x, moe_dtype_t x_dtype, const int32_t *phys_ids,
                                      const int32_t *slot_partition, uint32_t event_id,
                                      const moe_geom_t *g, void *disp_buf, moe_meta_t *meta,
                                      int32_t *slot_count, int32_t *slot_offset,
                                      int32_t *slot_rows, int32_t *disp_row, int32_t *ret_row,
                                      void *relay_buf, int32_t *status, void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (dispatch_scratch_layout(*g).total > (int64_t)MOE_STATIC_SCRATCH_BYTES)
    return MOE_ERR_CAPACITY;
  void *sp = static_scratch_ptr();
  if (!sp) return MOE_ERR_HIP;
  st = dispatch_impl(x, x_dtype, phys_ids, slot_partition, event_id, g, disp_buf, meta,
                     slot_count, slot_offset, slot_rows, disp_row, ret_row, relay_buf, sp,
                     MOE_STATIC_SCRATCH_BYTES, stream);
  if (st != MOE_OK || !status) return st;
  const DispatchScratch L = dispatch_scratch_layout(*g);
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const int32_t *)((const uint8_t *)sp + L.status), status);
  return launch_status();
}

extern "C" int moe_check_event(const moe_meta_t *meta, const void *disp_buf,
                               const int32_t *slot_rows, const int32_t *slot_offset,
                               const moe_geom_t *g, uint32_t event_id, int32_t *status,
                               void *stream) {
  int st = validate_geom(g);
  if (st != MOE_OK) return st;
  if (!meta || !slot_offset || !status) return MOE_ERR_INVALID_ARG;
  if (g->T > 0 && (!disp_buf || !slot_rows)) return MOE_ERR_INVALID_ARG;
  const int64_t nmeta = (int64_t)g->D * g->S;
  const int64_t work = nmeta + (int64_t)g->T * g->k;
  const unsigned blocks = (unsigned)std::min<int64_t>(1024, (work + 255) / 256);
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, status);
  if ((st = launch_status()) != MOE_OK) return st;
  hipLaunchKernelGGL(check_event_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, meta,
                     nmeta, (const uint8_t *)disp_buf, msg_bytes_of(*g), g->H, slot_rows,
                     slot_offset, g->P, event_id, status);
  return launch_status();
}
