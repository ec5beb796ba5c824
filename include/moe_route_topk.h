/*
 * moe_route_topk.h -- C ABI of the MI355X (gfx950) MoE hot path:
 *   gate top-k routing (+ EPLB replica map) -> token-wise INT8 quantization
 *   fused into a scatter into static per-partition buffers -> grouped INT8
 *   SwiGLU experts on MFMA -> combine (gather, dequantize, gate-weighted sum).
 *
 * Pages this interface follows (cited by title, section, paragraph/figure):
 *   [XDS] "xDeepServe on CloudMatrix384" (translation of arXiv:2508.02520):
 *         "合设 MoE-Attention 的 All-to-All" -- dispatch/combine, P038-P041,
 *         Fig. 7 and the DISPATCH / COMBINE procedures;
 *         "解耦 MoE-Attention 的 All-to-All" -- A2E/E2A trampoline, P044-P047, Fig. 8;
 *         "专家负载均衡" -- EPLB, P068-P079, Fig. 12;
 *         "DeepSeek INT8 量化" -- token-wise / channel-wise INT8, P085, P088, P089.
 *   [CMI] "CloudMatrix384 LLM Serving" (explainer of arXiv:2506.12708):
 *         "EP320：token 去找专家" -- FusedDispatch / FusedCombine, fused_moe listing;
 *         "缓冲区公式" -- static buffer sizing.
 *
 * Model.  The pages' expert-parallel ranks are virtual partitions inside one
 * GPU's HBM: S source partitions of LB tokens each (T = S * LB), and D
 * destination partitions that hold the P physical expert slots (at most Epp
 * per partition).  Partition d's receive area has one fixed region per
 * source, region (d, s), of cap = LB * min(k, Epp) message rows.
 *
 * Conventions for every entry point:
 *  - All tensors are caller-allocated device memory (hipMalloc or torch),
 *    except where a parameter says "host".  The library never allocates,
 *    frees, memsets or synchronizes, and keeps no mutable global state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    GPU entry points only enqueue work; results are ready when the stream
 *    reaches that point.
 *  - Arguments are validated on the host before any launch; an invalid call
 *    launches nothing and returns a negative status.  Inputs that only the
 *    device sees (ids, replica maps) are range-checked in the kernels: an
 *    out-of-range route is dropped (its row indices are written as -1) and a
 *    bit is set in the status word at the start of the dispatch scratch
 *    (see MOE_DEVICE_*), never written out of bounds.
 *  - Row-major layouts; int32 indices; bf16 is passed as its 16-bit pattern.
 *  - Buffers that kernels access with 16-byte vector loads/stores must be
 *    16-byte aligned (marked "16B").
 *  - Device buffers may be reused across calls; a call overwrites everything
 *    it documents as an output.  Calls on different streams that share a
 *    buffer race unless every one of them only reads it: inputs such as the
 *    packed expert weights, scales, slot maps and replica maps may be shared
 *    by calls in flight on several streams at once.
 */
#ifndef MOE_ROUTE_TOPK_H
#define MOE_ROUTE_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status -- */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, inconsistent geometry   */
  MOE_ERR_UNSUPPORTED = -2, /* outside the limits below                         */
  MOE_ERR_CAPACITY = -3,    /* scratch too small / replica plan does not fit    */
  MOE_ERR_STALE = -4,       /* metadata or messages of another dispatch event   */
  MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed              */
};

/* bits of the device status word (first int32 of the dispatch scratch) */
enum {
  MOE_DEVICE_BAD_ROUTE = 1,    /* physical slot id outside [0, P)                 */
  MOE_DEVICE_BAD_PARTITION = 2, /* slot_partition[p] outside [0, D)               */
  MOE_DEVICE_OVER_CAPACITY = 4, /* a (d, s) region would exceed cap rows          */
  MOE_DEVICE_STALE_EVENT = 8    /* moe_check_event: an event id that is not the   */
                                /* expected one (meta or a message trailer)       */
};

/* limits */
#define MOE_MAX_E 1024     /* logical experts                     */
#define MOE_MAX_P 1024     /* physical slots                      */
#define MOE_MAX_D 1024     /* destination partitions              */
#define MOE_MAX_K 16       /* routes per token                    */
#define MOE_MAX_H 16384    /* hidden size (multiple of 16)        */

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;
typedef enum { MOE_GATING_SOFTMAX = 0, MOE_GATING_SIGMOID = 1 } moe_gating_t;
typedef enum { MOE_PROJ_GATEUP = 0, MOE_PROJ_DOWN = 1 } moe_proj_t;
typedef enum {
  MOE_RET_Q8_FROM_DISPATCH = 0, /* value rows are dispatch messages (int8 + scale) */
  MOE_RET_BF16 = 1,             /* value rows are bf16 expert returns              */
  MOE_RET_Q8_BLOCKS = 2,        /* value rows are INT8 expert returns: H codes and */
                                /* one fp32 scale per MOE_RET_Q8_BLOCK columns     */
  MOE_RET_Q8_ROWS = 3           /* value rows are token-wise INT8 expert returns   */
                                /* (moe_quant_returns_q8): H codes, then one fp32  */
                                /* scale for the whole row at byte H               */
} moe_ret_mode_t;

/* Columns per scale of the INT8 expert returns (the down projection's n-tile). */
#define MOE_RET_Q8_BLOCK 256

/* Geometry of one MoE layer call. */
typedef struct moe_geom {
  int32_t T;         /* tokens; T = S * LB                                    */
  int32_t H;         /* hidden size, multiple of 16, <= MOE_MAX_H             */
  int32_t E;         /* logical experts, k <= E <= MOE_MAX_E                  */
  int32_t P;         /* physical expert slots, E <= P <= MOE_MAX_P            */
  int32_t k;         /* routes per token, 1 <= k <= MOE_MAX_K                 */
  int32_t D;         /* destination partitions, <= MOE_MAX_D                  */
  int32_t Epp;       /* max slots on one destination partition                */
  int32_t S;         /* source partitions                                     */
  int32_t LB;        /* local batch of each source partition                  */
  int32_t msg_bytes; /* dispatch message row size; 0 = H + 16 rounded to 128 */
  int32_t relays;    /* two-hop relay partitions (A2E/E2A trampoline); 0 = off */
  int32_t reserved;  /* must be 0                                             */
} moe_geom_t;

/* Per-(destination, source) metadata [XDS 合设 A2A, P039: per sender an event id,
 * the sender's offset in the receiver's area and the received token count]. */
typedef struct moe_meta {
  uint32_t event_id; /* the event_id of the dispatch call that wrote it          */
  int32_t offset;    /* sum of count[d][s'] over s' < s (receive layout prefix)  */
  int32_t count;     /* rows of region (d, s) written by this call               */
  int32_t reserved;
} moe_meta_t;

/* Byte sizes of everything the caller allocates. */
typedef struct moe_sizes {
  int64_t msg_bytes;                   /* one dispatch message row                        */
  int64_t cap_rows;                    /* rows per (d, s) region = LB * min(k, Epp)       */
  int64_t dispatch_bytes;              /* D * S * cap * msg: all receive regions (16B)    */
  int64_t dispatch_bytes_per_partition;/* S * cap * msg: the pages' per-rank buffer_size  */
  int64_t combine_bytes_per_partition; /* D * cap * H * 2: the pages' bf16 combine buffer */
  int64_t relay_bytes;                 /* (D - relays) * S * cap * msg; 0 when relays = 0 */
  int64_t return_bytes;                /* T * k * H * 2 dense bf16 return rows; doubled   */
                                       /* when relays > 0 (E2A staging follows the rows)  */
  int64_t dispatch_scratch_bytes;      /* scratch of moe_dispatch_q8                      */
  int64_t ffn_scratch_bytes;           /* scratch of moe_expert_ffn_q8 (I > 0)            */
  int64_t ret_q8_row_bytes;            /* one INT8 return row: H + 4 ceil(H / 256) bytes  */
                                       /* rounded up to whole 128-byte lines              */
  int64_t ret_q8_bytes;                /* T * k INT8 return rows                          */
  int64_t router_scratch_bytes;        /* scratch of moe_router_logits / moe_router_topk  */
  int64_t w_gateup_packed_bytes;       /* moe_pack_expert_weights image, MOE_PROJ_GATEUP  */
  int64_t w_down_packed_bytes;         /* moe_pack_expert_weights image, MOE_PROJ_DOWN    */
} moe_sizes_t;

/*
 * moe_plan_sizes -- host only, pure.  Static buffer sizing [CMI 缓冲区公式]:
 * max_tokens = LB * min(k, Epp) rows per sender region, buffer_size =
 * rank_num * max_tokens * msg_size per receiving partition (rank_num = S here).
 * I is the SwiGLU intermediate size (0 if no expert FFN is run).
 * Returns MOE_OK, or MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for bad geometry.
 */
int moe_plan_sizes(const moe_geom_t *g, int32_t I, moe_sizes_t *out);

/*
 * moe_eplb_build_map -- host only.  Redundant-expert selection and placement
 * [XDS 专家负载均衡, P069-P076 and the SELECT_AND_PLACE_REPLICAS procedure].
 *   token_count  host [slices][E]  tokens per logical expert per time slice
 *   budget       number of redundant slots to fill (P = E + budget)
 *   primary_partition host [E]     partition of each expert's primary copy
 *   free_slots   host [D]          redundant slots available on each partition
 * Rounds: the candidates are each slice's hottest expert; each trial adds one
 * copy (the expert's original count split evenly over all its copies) and the
 * candidate with the smallest sum over slices of the largest simulated load
 * wins (ties: lower id).  Placement: replicas by total load descending (ties:
 * selection order) go to the least-loaded partition with a free slot (ties:
 * lower id); every copy carries total / copies.
 * Outputs (host): replica_offsets [E+1], replica_slots [P] (R_e = slots of e,
 * ascending), slot_partition [P], slot_logical [P]; slot p = e is e's primary,
 * slot E + i the i-th placed replica.  selected [budget] (may be NULL): picks in
 * round order.  Returns MOE_ERR_CAPACITY if the free slots run out.
 */
int moe_eplb_build_map(const int64_t *token_count, int32_t slices, int32_t E, int32_t budget,
                       int32_t D, const int32_t *primary_partition, const int32_t *free_slots,
                       int32_t *replica_offsets, int32_t *replica_slots, int32_t *slot_partition,
                       int32_t *slot_logical, int32_t *selected);

/*
 * moe_route_topk -- gate top-k and the EPLB logical->physical map
 * [XDS 合设 A2A, P038 (indices I and weights W of shape B x k); CMI EP320
 * (gate.topk(hidden, k=8)); XDS 专家负载均衡 P078-P079, Fig. 12 (gather of the
 * gating result into physical replicas, round robin by token position)].
 *   logits          [T][E] fp32 or bf16 (logits_dtype)
 *   bias            [E] fp32 or NULL; score = fp32(logit) + bias (one fp32 add)
 *   gating          weights over the k chosen: SOFTMAX w_j = exp(s_j - s_0) / sum,
 *                   SIGMOID w_j = sig(s_j) / sum sig (fp32, expf)
 *   replica_offsets [E+1] or NULL (NULL: phys = e, requires P == E)
 *   replica_slots   [P]   R_e = replica_slots[replica_offsets[e] .. replica_offsets[e+1])
 * Outputs: topk_ids [T][k] (descending score, lower id first on ties),
 *   topk_w [T][k] fp32, phys_ids [T][k] = R_e[(t mod LB) mod |R_e|] (-1 if R_e
 *   is empty or out of range), expert_counts [E] (may be NULL): routes per
 *   logical expert (the EPLB collect step, P068).
 */
int moe_route_topk(const void *logits, moe_dtype_t logits_dtype, const float *bias,
                   moe_gating_t gating, const int32_t *replica_offsets,
                   const int32_t *replica_slots, const moe_geom_t *g, int32_t *topk_ids,
                   float *topk_w, int32_t *phys_ids, int32_t *expert_counts, void *stream);

/*
 * moe_router_logits -- the gate's logits from the hidden states [CMI EP320
 * fused_moe listing: gate.topk(hidden, k = 8) opens the MoE step; CMI
 * "INT8：少搬一些": gating stays in BF16/FP32 while the matmuls go INT8; XDS
 * P038: dispatch and combine follow the gating scores]:
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h]
 * bf16 operands, products and sums in fp32 (MFMA), fp32 logits.  Tiles of 192
 * tokens x 256 experts; when they are too few to fill the GPU, the sum over h
 * is split into router_splits parts (whole 64-element steps) whose partial
 * sums are added in split order, so the result is the same every run; its
 * error against the exact value is within the fp32 summation bound
 * (H * 2^-24 * sum |x w|).  Feed the logits to moe_route_topk (MOE_DTYPE_F32).
 *   x        [T][H] bf16, 16B;  w_router [E][H] bf16, 16B;  H % 64 == 0, E % 4 == 0
 *   logits   [T][E] fp32, 16B
 *   scratch  router_scratch_bytes (moe_plan_sizes), 16B: the partial sums when
 *            H is split (unused otherwise, but still required)
 * Errors: MOE_ERR_UNSUPPORTED (H % 64 or E % 4), MOE_ERR_CAPACITY (scratch),
 * MOE_ERR_INVALID_ARG (NULL or misaligned pointers).
 */
int moe_router_logits(const void *x, const void *w_router, const moe_geom_t *g, float *logits,
                      void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_router_topk -- the gate from the hidden states to the routes in one call
 * [CMI EP320 fused_moe listing: gate.topk(hidden, k = 8); XDS 专家负载均衡 P068
 * (the collect step) and P078-P079 (the replica gather)]: the logits of
 * moe_router_logits, then moe_route_topk on them (MOE_DTYPE_F32), without the
 * round trip of the summed logits when H is split: the top-k reads the gate's
 * partial sums and adds them in split order itself.  Logits, ids, weights,
 * physical ids and counts are the same bits as the two calls give.
 *   x, w_router, scratch  as moe_router_logits (router_scratch_bytes)
 *   logits   [T][E] fp32, 16B, or NULL when the caller does not keep them
 *   bias, gating, replica_offsets, replica_slots, topk_ids, topk_w, phys_ids,
 *   expert_counts  as moe_route_topk
 * Errors: those of the two calls.
 */
int moe_router_topk(const void *x, const void *w_router, const float *bias, moe_gating_t gating,
                    const int32_t *replica_offsets, const int32_t *replica_slots,
                    const moe_geom_t *g, float *logits, int32_t *topk_ids, float *topk_w,
                    int32_t *phys_ids, int32_t *expert_counts, void *scratch,
                    size_t scratch_bytes, void *stream);

/*
 * moe_dispatch_q8 -- token-wise INT8 quantization fused into the scatter into
 * static per-partition buffers, plus the count/offset metadata
 * [XDS 合设 A2A, P039-P040, Fig. 7, DISPATCH procedure (count exchange, then
 * data); CMI EP320 FusedDispatch (quantize early, attach source info, write
 * into the target's static buffer)].
 *   x              [T][H] bf16 or fp32 (x_dtype), 16B
 *   phys_ids       [T][k] physical slot of each route
 *   slot_partition [P] destination partition of each slot
 *   event_id       stamped into meta and the message trailers
 * Per token: a = max|x|, s = a / 127 (fp32), q = clamp(rne(x / s), +-127)
 * (s = 0 gives q = 0).  Route (t, j) of source s = t / LB, b = t mod LB, to
 * partition d gets row r of region (d, s), where r counts the earlier routes
 * of s in (b, j) order that go to d.
 * Outputs:
 *   disp_buf  [D][S][cap][msg] bytes, 16B: row = q (H bytes) then a 16-byte
 *             trailer {f32 scale, i32 s, i32 b, u8 j, u8 local slot of the target on
 *             its partition, u16 event_id & 0xffff}, then zeros up to the end of the
 *             trailer's 128-byte line or of the row (written so that the line is
 *             stored whole); other padding and rows >= meta.count undefined
 *   meta      [D][S] {event_id, offset = sum_{s' < s} count[d][s'], count, 0}
 *   slot_count [P], slot_offset [P+1] (exclusive prefix sum)
 *   slot_rows [T*k]: for slot p, rows slot_offset[p] .. +slot_count[p] list the
 *             dispatch rows of its routes in (t, j) order
 *   disp_row  [T][k] = (d * S + s) * cap + r;  ret_row [T][k] = slot_offset[p] + rank
 *             of (t, j) among slot p's routes (the dense return row)
 *   relay_buf with g->relays = R > 0: routes to partitions d >= R are written first
 *             to relay region (d - R, s) ([D-R][S][cap][msg], 16B) and then copied
 *             to disp_buf (two-hop trampoline, XDS P045, Fig. 8); NULL when R = 0.
 *   scratch   dispatch_scratch_bytes (16B); its first int32 is the device status
 *             word (MOE_DEVICE_* bits, cleared by this call).
 */
int moe_dispatch_q8(const void *x, moe_dtype_t x_dtype, const int32_t *phys_ids,
                    const int32_t *slot_partition, uint32_t event_id, const moe_geom_t *g,
                    void *disp_buf, moe_meta_t *meta, int32_t *slot_count, int32_t *slot_offset,
                    int32_t *slot_rows, int32_t *disp_row, int32_t *ret_row, void *relay_buf,
                    void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_check_event -- the receiver's event check of the dispatch protocol
 * [XDS 合设 MoE-Attention 的 All-to-All, P039-P040: each sender's metadata
 * carries an event id, so that a receiver consumes only data of the current
 * step].  Checks, on the device, that every meta[d][s].event_id equals
 * event_id and that every message row listed in slot_rows[0 .. slot_offset[P])
 * (the rows the expert FFN gathers and the INT8 combine reads) carries
 * event_id & 0xffff in its trailer.  *status receives MOE_DEVICE_STALE_EVENT if
 * anything mismatches, 0 otherwise.  The debug mode of the layer
 * (MOE_DEBUG_CHECKS) runs it before the experts and before the combine and
 * turns the bit into MOE_ERR_STALE.  Rows whose slot_rows entry is -1 (routes
 * dropped by the dispatch) are skipped.
 *   meta [D][S], disp_buf, slot_rows [T*k], slot_offset [P+1] as written by
 *   moe_dispatch_q8;  status: device int32, written by this call.
 * Errors: MOE_ERR_INVALID_ARG (NULL pointers), geometry errors.
 */
int moe_check_event(const moe_meta_t *meta, const void *disp_buf, const int32_t *slot_rows,
                    const int32_t *slot_offset, const moe_geom_t *g, uint32_t event_id,
                    int32_t *status, void *stream);

/*
 * moe_dispatch_q8_static -- moe_dispatch_q8 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same inputs, outputs, validation and errors as
 * moe_dispatch_q8, but the scratch lives in a device array inside the library:
 * MOE_STATIC_SCRATCH_BYTES on each GPU the library runs on, held until the
 * process ends.  The call allocates nothing.
 *   status   device int32 or NULL: receives the call's device status word
 *            (MOE_DEVICE_* bits) when its kernels have run.
 * Errors: those of moe_dispatch_q8; MOE_ERR_CAPACITY if the geometry needs more
 * than MOE_STATIC_SCRATCH_BYTES of scratch (dispatch_scratch_bytes of
 * moe_plan_sizes); MOE_ERR_HIP if the array's address cannot be obtained.
 * Every call on one GPU shares that GPU's array and leaves its contents behind
 * (nothing in it needs to start cleared): calls on one GPU that overlap in time
 * -- on different streams, or from different threads without ordering -- race.
 */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
int moe_dispatch_q8_static(const void *x, moe_dtype_t x_dtype, const int32_t *phys_ids,
                           const int32_t *slot_partition, uint32_t event_id, const moe_geom_t *g,
                           void *disp_buf, moe_meta_t *meta, int32_t *slot_count,
                           int32_t *slot_offset, int32_t *slot_rows, int32_t *disp_row,
                           int32_t *ret_row, void *relay_buf, int32_t *status, void *stream);

/*
 * moe_pack_expert_weights -- INT8 expert weights into the expert GEMMs' operand
 * image [XDS DeepSeek INT8 量化, P088: the routed experts' weights are stored
 * INT8; how they sit in memory is left open].  In the image, the weights that
 * each of a GEMM tile's four wavefronts multiplies in one 64-byte K step are 4
 * KB of consecutive bytes, already in MFMA operand order, so the GEMM loads
 * them straight into registers as whole 128-byte lines, several steps ahead.
 * Run once when the weights are loaded; the GEMMs take only the image.
 *   proj MOE_PROJ_GATEUP: w = [E][2I][H] (rows 0..I-1 gate, I..2I-1 up), K = H,
 *     NT = ceil(I / 128) n-tiles of 128 gate/up pairs; tile row r < 128 is gate
 *     row min(128 n + r, I - 1), row r >= 128 is up row I + min(128 n + r - 128, I - 1).
 *   proj MOE_PROJ_DOWN: w = [E][H][I], K = I, NT = ceil(H / 256); tile row r is
 *     row min(256 n + r, H - 1).
 *   Image: 16 KB blocks (e, n, s) for K steps s < KTp = K / 64 rounded up to a
 *     multiple of 4 (steps past K / 64 are zero).  Within a block, 16-byte slot
 *     1024 w + 256 ks + 64 nb + l (w, ks, nb < 2 or 4 as below, lane l < 64)
 *     holds K bytes 64 s + 32 ks + 16 (l >> 5) .. +16 of tile row
 *     GATEUP: 128 nb + 32 w + (l & 31),  DOWN: 64 w + 32 nb + (l & 31)
 *     (w < 4 wavefronts, ks < 2 MFMA K halves, nb < 2 column blocks).
 *     Size E * NT * KTp * 16384 bytes (w_gateup_packed_bytes / w_down_packed_bytes).
 *   Requirements: E > 0, H a multiple of 128, I a multiple of 64 and <= 16384,
 *     w and packed 16B-aligned and not overlapping, packed_bytes >= the size.
 * Errors: MOE_ERR_INVALID_ARG (NULL, misaligned, bad proj or E),
 *   MOE_ERR_UNSUPPORTED (H or I), MOE_ERR_CAPACITY (packed_bytes), MOE_ERR_HIP.
 */
int moe_pack_expert_weights(const int8_t *w, moe_proj_t proj, int32_t E, int32_t H, int32_t I,
                            int8_t *packed, size_t packed_bytes, void *stream);

/*
 * moe_expert_ffn_q8 -- grouped INT8 SwiGLU experts on MFMA
 * [XDS DeepSeek INT8 量化, P085 (QMM: y_ij ~ s_i s^w_j sum_k q(x_ik) q(w_jk), token-wise
 * activation and channel-wise weight scales), P088 (gate and up projections
 * fused in one kernel, all expert weights INT8)].  SwiGLU = down(silu(gate) * up).
 * For every physical slot p (logical expert e = slot_logical[p]) and each of its
 * rows (dispatch row slot_rows[slot_offset[p] + i], codes q and scale s_x from
 * the message):
 *   acc_g = q . Wgu[e][n], acc_u = q . Wgu[e][I + n]              (int32, n < I)
 *   g = (f32(acc_g) * s_x) * s_gateup[e][n];  u likewise with s_gateup[e][I + n]
 *   h = (g / (1 + f32(exp(-g)))) * u   (exp in double precision, rounded once)
 *   (hq, hs) = token-wise INT8 of h (same rule as dispatch)
 *   acc_d = hq . Wd[e][c]                                           (int32, c < H)
 *   ret[slot_offset[p] + i][c] = bf16_rne((f32(acc_d) * hs) * s_down[e][c])
 *   disp_buf   as written by moe_dispatch_q8 (16B)
 *   w_gateup   Wgu = [E][2I][H] int8 (rows 0..I-1 gate, I..2I-1 up) in the tile image of
 *              moe_pack_expert_weights (MOE_PROJ_GATEUP), 16B;  s_gateup [E][2I] fp32, 16B
 *   w_down     Wd = [E][H][I] int8 in the tile image of moe_pack_expert_weights
 *              (MOE_PROJ_DOWN), 16B;  s_down [E][H] fp32, 16B
 *   I          multiple of 64, <= 16384 (H a multiple of 128)
 *   ret        [T*k][H] bf16, 16B
 *   acc_gateup_dbg [T*k][2I] int32 or NULL, acc_down_dbg [T*k][H] int32 or NULL:
 *              when given, the raw int32 accumulators are written too (testing)
 *   scratch    ffn_scratch_bytes (16B)
 */
int moe_expert_ffn_q8(const void *disp_buf, const int32_t *slot_count, const int32_t *slot_offset,
                      const int32_t *slot_rows, const int32_t *slot_logical,
                      const int8_t *w_gateup, const float *s_gateup, const int8_t *w_down,
                      const float *s_down, int32_t I, const moe_geom_t *g, uint16_t *ret,
                      int32_t *acc_gateup_dbg, int32_t *acc_down_dbg, void *scratch,
                      size_t scratch_bytes, void *stream);

/*
 * The two stages of moe_expert_ffn_q8, for callers that schedule or time them
 * apart [XDS DeepSeek INT8 量化, P085, P088]; moe_expert_ffn_q8 is exactly
 * moe_expert_gateup_q8 followed by moe_expert_down_q8 on the same scratch.
 *   moe_expert_gateup_q8: the fused gate/up QMM and the SwiGLU epilogue; leaves h
 *     (fp32) and its per-row partial maxima in scratch.
 *   moe_expert_down_q8: token-wise INT8 of h (hq, hs) and the down QMM into ret.
 *     It must follow moe_expert_gateup_q8 on the same stream, scratch, geometry
 *     and slot arrays.
 * Arguments have the meaning given for moe_expert_ffn_q8.
 */
int moe_expert_gateup_q8(const void *disp_buf, const int32_t *slot_count,
                         const int32_t *slot_offset, const int32_t *slot_rows,
                         const int32_t *slot_logical, const int8_t *w_gateup,
                         const float *s_gateup, int32_t I, const moe_geom_t *g,
                         int32_t *acc_gateup_dbg, void *scratch, size_t scratch_bytes,
                         void *stream);
int moe_expert_down_q8(const int32_t *slot_count, const int32_t *slot_offset,
                       const int32_t *slot_logical, const int8_t *w_down, const float *s_down,
                       int32_t I, const moe_geom_t *g, uint16_t *ret, int32_t *acc_down_dbg,
                       void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_expert_down_q8_int8ret -- moe_expert_down_q8 with INT8 return rows
 * [XDS DeepSeek INT8 量化, P089: expert outputs are quantized to INT8 before
 * they travel back, the quantization fused into the transfer].  The bf16 value
 * y that moe_expert_down_q8 would return is quantized in the projection's
 * epilogue, one scale per MOE_RET_Q8_BLOCK columns of each row (the pages do
 * not fix the granularity; 256 columns is the projection's output tile):
 *   s = max |y| over the block / 127,  q = clamp(round_half_even(y / s), +-127)
 *   (fp32 divisions; an all-zero block gives s = 0, q = 0).
 *   ret_q8  [T*k][ret_q8_row_bytes] (moe_plan_sizes): row slot_offset[p] + i
 *           holds H int8 codes, then ceil(H / 256) fp32 scales, then padding
 *           to a whole number of 128-byte lines; 16B (a 128-byte aligned
 *           buffer keeps every 256-column block of codes on whole lines).
 * Combine these rows with mode MOE_RET_Q8_BLOCKS.  Geometries with relays are
 * not supported (MOE_ERR_UNSUPPORTED): the E2A hop moves bf16 rows.
 * Other arguments, preconditions and errors as moe_expert_down_q8.
 */
int moe_expert_down_q8_int8ret(const int32_t *slot_count, const int32_t *slot_offset,
                               const int32_t *slot_logical, const int8_t *w_down,
                               const float *s_down, int32_t I, const moe_geom_t *g, void *ret_q8,
                               int32_t *acc_down_dbg, void *scratch, size_t scratch_bytes,
                               void *stream);

/*
 * moe_quant_returns_q8 -- token-wise INT8 expert returns [XDS DeepSeek INT8 量化:
 * P085 gives activations one scale per token, P089 quantizes the expert outputs
 * to INT8 before they travel back, the quantization fused into that transfer].
 * Each dense bf16 return row y (as written by moe_expert_down_q8) gets the
 * token rule of moe_dispatch_q8 over the whole row:
 *   s = max_c |y[c]| / 127 (fp32),  q[c] = clamp(round_half_even(y[c] / s), +-127)
 *   (fp32 quotients; an all-zero row gives s = 0 and q = 0).
 * This is the send side of the return path: it reads each return row once and
 * writes the row that travels, half the bytes of the bf16 row.
 *   ret         [T*k][H] bf16, 16B (rows [0, slot_offset[P]) are converted)
 *   slot_offset [P+1] as written by moe_dispatch_q8 (read on the device)
 *   ret_q8      [T*k][ret_q8_row_bytes] (moe_plan_sizes), 16B: row i holds the H
 *               codes, then the fp32 scale at byte H, then zeros up to the end of
 *               the scale's 128-byte line (written so that the line is stored
 *               whole); any bytes after that are left as they were
 * Combine these rows with mode MOE_RET_Q8_ROWS.  Geometries with relays are not
 * supported (MOE_ERR_UNSUPPORTED): the E2A hop moves bf16 rows.
 * Errors: MOE_ERR_INVALID_ARG (NULL or misaligned pointers), MOE_ERR_UNSUPPORTED.
 */
int moe_quant_returns_q8(const uint16_t *ret, const int32_t *slot_offset, const moe_geom_t *g,
                         void *ret_q8, void *stream);

/*
 * moe_relay_returns -- E2A second hop of the two-hop trampoline [XDS 解耦 A2A,
 * P045, Fig. 8: E2A runs the A2E path in reverse].  With g->relays = R > 0, the
 * return row of every route whose slot lives on a partition d >= R is copied
 * from ret[ret_row] to the staging rows that follow the T*k return rows
 * (ret[T*k + ret_row]), and comb_row [T][k] is written with the row the
 * combine must read: ret_row for direct routes, T*k + ret_row for relayed ones.
 *   ret      [2*T*k][H] bf16 (return_bytes of moe_plan_sizes), 16B
 */
int moe_relay_returns(uint16_t *ret, const int32_t *phys_ids, const int32_t *slot_partition,
                      const int32_t *ret_row, const moe_geom_t *g, int32_t *comb_row,
                      void *stream);

/*
 * moe_combine -- gather each token's k returns, dequantize, gate-weighted sum
 * [XDS 合设 A2A, COMBINE procedure; CMI EP320 FusedCombine (all k contributions,
 * dequantize, weight by the gate)]:
 *   out[t][c] = sum_{j = 0..k-1} w[t][j] * v_j[c]   (fp32, ascending j, no FMA)
 *   mode Q8_FROM_DISPATCH: src = disp_buf, row = disp_row; v = f32(q) * scale
 *                          (identity experts: the dispatched message is the value)
 *   mode BF16:             src = ret [rows][H] bf16, row = ret_row (or comb_row)
 *   mode Q8_BLOCKS:        src = ret_q8 (moe_expert_down_q8_int8ret), row = ret_row;
 *                          v = f32(q[c]) * scale[c / 256] [XDS DeepSeek INT8 量化, P089]
 *   mode Q8_ROWS:          src = ret_q8 (moe_quant_returns_q8), row = ret_row;
 *                          v = f32(q[c]) * scale (one per row) [XDS P085, P089]
 *   topk_w  [T][k] fp32;  out [T][H] fp32 or bf16 (out_dtype, RNE), 16B.
 *   Routes with row < 0 contribute nothing.
 */
int moe_combine(moe_ret_mode_t mode, const void *src, const int32_t *row, const float *topk_w,
                const moe_geom_t *g, moe_dtype_t out_dtype, void *out, void *stream);

/*
 * moe_probe_mfma_i8 -- measurement support, not a step of the MoE path: the
 * int8 matrix-core rate the device sustains, the ceiling the expert GEMMs are
 * measured against beside the published peak (which assumes the top clock).
 * Launches `blocks` workgroups of 256 threads; every wavefront issues
 * 4 * iters v_mfma_i32_32x32x32_i8 (32x32x32 = 65536 int8 operations each) on
 * register operands and writes one checksum per thread:
 *   out  [blocks * 256] int32, device (caller-owned)
 * Errors: MOE_ERR_INVALID_ARG (blocks or iters <= 0, NULL out).
 */
int moe_probe_mfma_i8(int32_t blocks, int32_t iters, int32_t *out, void *stream);

/* Human-readable name of a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_TOPK_H */
