/*
 * miep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel core:
 * layout histogram, normal-mode dispatch with its handle, cached dispatch,
 * combine (with optional bias rows), the two-level relay (dispatch through
 * one buffer per group of 8 ranks and the two-level combine), low-latency
 * (expert-major, optionally FP8) dispatch and combine, and the low-latency
 * rank mask.
 *
 * One GPU plays every rank: the R logical ranks are partitions of one
 * device's HBM, and the S source partitions are the token blocks that the
 * R ranks would each send.  No inter-GPU transport is involved.
 *
 * Pages the calls follow (titles as published):
 *   [Ch4]  "Chapter 4  V1: layout, dispatch and combine", sections 4.1-4.5
 *   [NvLL] "DeepEP Normal vs Low-Latency dual-mode analysis"
 *   [Phil] "Normal vs Low-Latency: two communication philosophies in
 *          DeepEP V1 / V2 / DeepGEMM"
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless a parameter says "host", owned by
 *     the caller; the library keeps no pointer after the call returns and
 *     allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; the caller orders and synchronises.
 *   - Integer matrices are row-major int32 unless noted; booleans are one
 *     byte, 0 or 1.  bf16 data is passed as its 16-bit patterns.
 *   - Every call returns miep_status and miep_last_error() describes a
 *     failure (thread-local, host memory owned by the library).  Argument
 *     errors (EINVAL, EUNSUPPORTED) are found before anything is enqueued;
 *     an EHIP from a call that launches several kernels may leave its
 *     earlier kernels enqueued.  No call aborts, traps or prints.
 *   - Device-side bounds: rows at or past `recv_capacity` are never
 *     written; top-k entries outside [0, num_experts) are treated as masked.
 *   - Errors the host cannot see at call time (a receive side larger than
 *     its fixed capacity) are reported through a caller-owned device status
 *     word: the call writes 0 or the miep_status code, and
 *     miep_check_status() reads it back synchronously.
 */
#ifndef MIEP_H
#define MIEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum miep_status {
  MIEP_OK = 0,
  MIEP_EINVAL = 1,       /* a bad argument: null pointer, size or flag */
  MIEP_EUNSUPPORTED = 2, /* valid, but outside what the kernels handle (e.g. R > 256, misaligned x) */
  MIEP_EHIP = 3,         /* the HIP runtime refused a launch */
  MIEP_ECAPACITY = 4     /* device status: the receive rows exceeded a fixed capacity (rows past it were dropped) */
} miep_status;

/* Payload kinds of a normal-mode dispatch. */
typedef enum miep_xkind {
  MIEP_X_BF16 = 0,          /* x: [N][H] bf16; rows travel as 2H bytes                         */
  MIEP_X_FP8 = 1,           /* x: [N][H] E4M3 codes + x_scales [N][H/128] fp32 (pre-quantised)  */
  MIEP_X_BF16_CAST_FP8 = 2  /* x: [N][H] bf16, cast per 128 channels to E4M3 + fp32 scales      */
} miep_xkind;

/* Sizes of one normal-mode problem.  N = num_src * num_tokens tokens. */
typedef struct miep_problem {
  int32_t num_src;          /* S: source partitions (the sending ranks), <= 2^20         */
  int32_t num_tokens;       /* T: tokens per source partition                             */
  int32_t hidden;           /* H: channels per token, <= 2^24                             */
  int32_t num_topk;         /* K: experts per token, <= 64; a dispatch needs
                               N * min(K, R) <= 2^31-1 (int32 receive rows)                */
  int32_t num_experts;      /* E: experts; expert e lives on rank e / (E / R)              */
  int32_t num_ranks;        /* R: receiving ranks, 1..256; R > 8 needs R % 8 == 0          */
  int32_t num_channels;     /* C: channels splitting each source's tokens (ceil(T/C) each), <= 1024 */
  int32_t expert_alignment; /* a >= 1: per-expert receive counts rounded up to a multiple  */
} miep_problem;

/* The normal-mode handle ([Ch4] 4.2: a reverse-routing record, reused by
 * cached dispatch and combine).  All arrays are caller-owned device memory;
 * miep_dispatch fills every non-const member, is_token_in_rank is its input.
 *   rank_prefix_matrix[s][r]            inclusive over sources: rows rank r receives from sources 0..s
 *   channel_prefix_matrix[s][r][c]      inclusive over channels: tokens of source s, channels 0..c, sent to r
 *   recv_channel_prefix_matrix[r][s][c] rank r's row count before source s plus channel_prefix_matrix[s][r][c]
 *   recv_rank_offset[r]                 first receive row of rank r; [R] = total rows (may exceed capacity)
 *   recv_src_idx[row]                   token index t (within its source) of each receive row
 *   is_token_in_rank[n][r]              layout membership, n = s*T + t
 *   send_head[n][r]                     row of token n inside rank r's block, or -1
 * Rank r's rows are recv rows [recv_rank_offset[r], recv_rank_offset[r+1]),
 * ordered by (source, token).  The handle stays valid while the arrays live
 * and the routing is unchanged. */
typedef struct miep_handle {
  int32_t* rank_prefix_matrix;         /* [S][R]    */
  int32_t* channel_prefix_matrix;      /* [S][R][C] */
  int32_t* recv_channel_prefix_matrix; /* [R][S][C] */
  int32_t* recv_rank_offset;           /* [R + 1]   */
  int32_t* recv_src_idx;               /* [recv_capacity] */
  const uint8_t* is_token_in_rank;     /* [N][R]    */
  int32_t* send_head;                  /* [N][R]    */
  int64_t recv_capacity;               /* rows allocated in every receive-side array */
} miep_handle;

/* get_dispatch_layout -- [Ch4] 4.1: from the top-k routing compute the
 * tokens per rank, per RDMA rank (groups of 8 ranks, [NvLL] RDMA rank
 * translation), per expert, and the token-in-rank membership.
 *   topk_idx                 [N][K] int64, negative = masked
 *   num_tokens_per_rank      [S][R]   out
 *   num_tokens_per_rdma_rank [S][R/8] out; must be NULL when R <= 8, non-NULL when R > 8
 *   num_tokens_per_expert    [S][E]   out (counts top-k entries)
 *   is_token_in_rank         [N][R]   out (0/1 bytes)
 * Errors: EINVAL for a null required pointer or bad sizes (E % R != 0,
 * R > 8 with R % 8 != 0); EUNSUPPORTED for R > 256 or E > 8192. */
miep_status miep_get_dispatch_layout(const miep_problem* p, const int64_t* topk_idx,
                                     int32_t* num_tokens_per_rank, int32_t* num_tokens_per_rdma_rank,
                                     int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank, void* stream);

/* dispatch -- [Ch4] 4.1 fresh branch: notify (the prefix matrices) then
 * pack every token into each rank that receives it, rank-major.
 *   x                  [N][H] per x_kind (16-byte aligned; H % 8 == 0, FP8 kinds H % 128 == 0)
 *   x_scales           [N][H/128] fp32 for MIEP_X_FP8, else ignored
 *   round_scale        for MIEP_X_BF16_CAST_FP8: power-of-two scales
 *   use_ue8m0          ([Ch4] 4.3 flag) also emit each power-of-two scale 2^e as
 *                      its exponent byte e + 127; needs MIEP_X_BF16_CAST_FP8 with
 *                      round_scale (else EINVAL).  The fp32 scales are written too.
 *   topk_idx           [N][K] int64, nullable (then no recv_topk_* output)
 *   topk_weights       [N][K] fp32, nullable
 *   num_tokens_per_rank   [S][R] from get_dispatch_layout (source of the rank prefixes)
 *   num_tokens_per_expert [S][E] from get_dispatch_layout, nullable
 *   recv_x             [cap][H] bf16, or [cap][H] E4M3 codes for the FP8 kinds
 *   recv_x_scales      [cap][H/128] fp32 for the FP8 kinds
 *   recv_x_scales_ue8m0 [cap][H/128] uint8, required with use_ue8m0, else ignored
 *   recv_topk_idx      [cap][K] int64: local expert id (e - r*E/R) where expert e is on the row's rank, else -1
 *   recv_topk_weights  [cap][K] fp32: the weight there, else 0
 *   num_recv_tokens_per_expert [R][E/R] out, nullable: per-expert receive count rounded up to expert_alignment
 *   status             one int32 of device memory, nullable: set to 0, or to
 *                      MIEP_ECAPACITY when the receive rows exceed recv_capacity
 *   h                  the handle (all members required; cap = h->recv_capacity)
 * Size the receive side exactly with sum(num_tokens_per_rank) (never
 * overflows), or with a worst case (the num_worst_tokens mode of [Ch4] 4.1):
 * recv_rank_offset[R] reports the true total either way, and rows at or past
 * the capacity are neither written nor, later, combined -- a token whose row
 * fell past it loses that contribution in miep_combine.  A dispatch whose
 * status reads MIEP_ECAPACITY must be redone with a larger capacity before
 * its handle is used. */
miep_status miep_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                          int32_t round_scale, int32_t use_ue8m0, const int64_t* topk_idx, const float* topk_weights,
                          const int32_t* num_tokens_per_rank, const int32_t* num_tokens_per_expert, void* recv_x,
                          float* recv_x_scales, uint8_t* recv_x_scales_ue8m0, int64_t* recv_topk_idx,
                          float* recv_topk_weights, int32_t* num_recv_tokens_per_expert, int32_t* status,
                          const miep_handle* h, void* stream);

/* cached_dispatch -- [Ch4] 4.1 cached branch: with a handle from an earlier
 * dispatch of the same routing, move only x (and its scales); there are no
 * top-k arguments.  Arguments as in miep_dispatch (use_ue8m0 and
 * recv_x_scales_ue8m0 likewise); only h->send_head, h->recv_rank_offset and
 * h->recv_capacity are read. */
miep_status miep_cached_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                 int32_t round_scale, int32_t use_ue8m0, const miep_handle* h, void* recv_x,
                                 float* recv_x_scales, uint8_t* recv_x_scales_ue8m0, void* stream);

/* check_status -- host-side read of a status word written by miep_dispatch
 * or miep_relay_dispatch: waits for `stream` (synchronous), copies the word
 * and returns it (MIEP_OK or MIEP_ECAPACITY).  EINVAL for a null pointer,
 * EHIP if the copy fails. */
miep_status miep_check_status(const int32_t* status, void* stream);

/* combine -- [Ch4] 4.2 and 4.4: send expert outputs back through the handle
 * and add them per source token in fp32 (no gate weights applied), and
 * separately add the received top-k weights.  Contributions are added in
 * ascending rank order; a token no rank received combines to zero.  Only
 * rows below h->recv_capacity are read (after an overflowed dispatch the
 * rows past it are missing from the sums).
 * [Ch4] 4.2 also unpacks a bias into two rows for the combine without a
 * formula; here each given bias row is added to its token's fp32 sum after
 * the received contributions, bias_0 first (a token no rank received then
 * combines to its bias).
 *   y                     [cap][H] bf16 expert outputs in the receive layout
 *   recv_topk_weights     [cap][K] fp32, nullable
 *   bias_0, bias_1        [N][H] bf16 each, nullable, 16-byte aligned
 *   combined_x            [N][H] bf16 out (round to nearest even)
 *   combined_topk_weights [N][K] fp32 out, nullable (required if recv_topk_weights is given)
 * Reads h->send_head, h->recv_rank_offset, h->recv_capacity. */
miep_status miep_combine(const miep_problem* p, const uint16_t* y, const float* recv_topk_weights,
                         const uint16_t* bias_0, const uint16_t* bias_1, const miep_handle* h,
                         uint16_t* combined_x, float* combined_topk_weights, void* stream);

/* The two-level relay's handle ([NvLL] normal-mode internode dispatch:
 * RDMA to the destination node, then forwarding over NVLink inside it;
 * [Ch4] 4.2: the internode handle adds RDMA prefixes and source metadata).
 * Groups g = 0..G-1 of 8 ranks (ranks 8g..8g+7, the RDMA rank translation)
 * stand for the nodes.  All arrays are caller-owned device memory filled by
 * miep_relay_dispatch:
 *   rdma_rank_prefix_matrix[s][g]            inclusive over sources: group rows group g receives from sources 0..s
 *   rdma_channel_prefix_matrix[s][g][c]      inclusive over channels: tokens of source s, channels 0..c, sent to group g
 *   recv_rdma_channel_prefix_matrix[g][s][c] group g's row count before source s plus rdma_channel_prefix_matrix[s][g][c]
 *   recv_rdma_offset[g]                      first group row of group g; [G] = total group rows
 *   send_rdma_head[n][g]                     row of token n inside group g's block, or -1
 *   rdma_src_idx[row]                        source token n = s*T + t of each group row
 *   send_nvl_head[row][j]                    row of the group row inside rank 8g+j's receive block, or -1
 * A token goes to group g when it goes to any of the group's ranks; group
 * g's rows are [recv_rdma_offset[g], recv_rdma_offset[g+1]), in (source,
 * token) order.  send_head, send_rdma_head and send_nvl_head must be
 * 16-byte aligned, is_token_in_rank 8-byte aligned. */
typedef struct miep_relay_handle {
  int32_t* rdma_rank_prefix_matrix;         /* [S][G]    */
  int32_t* rdma_channel_prefix_matrix;      /* [S][G][C] */
  int32_t* recv_rdma_channel_prefix_matrix; /* [G][S][C] */
  int32_t* recv_rdma_offset;                /* [G + 1]   */
  int32_t* send_rdma_head;                  /* [N][G]    */
  int32_t* rdma_src_idx;                    /* [rdma_capacity] */
  int32_t* send_nvl_head;                   /* [rdma_capacity][8] */
  int64_t rdma_capacity;                    /* group rows allocated in rdma_x, rdma_src_idx, send_nvl_head */
} miep_relay_handle;

/* relay_dispatch -- the normal dispatch through the two-level relay: each
 * token is written once per destination group into the group rows (rdma_x;
 * the FP8 cast of MIEP_X_BF16_CAST_FP8 happens once, before this first hop),
 * then every group row is forwarded to each of the group's ranks that
 * receive the token.  The receive side (recv_x, recv_x_scales,
 * recv_topk_*, num_recv_tokens_per_expert and the handle h) is exactly that
 * of miep_dispatch with the same arguments; rh describes the group rows.
 *   num_tokens_per_rdma_rank [S][G] from get_dispatch_layout (required)
 *   rdma_x        [rdma_capacity][H] bf16, or E4M3 codes for the FP8 kinds (16-byte aligned)
 *   rdma_x_scales [rdma_capacity][H/128] fp32 for the FP8 kinds
 * Other arguments as in miep_dispatch.  Needs R % 8 == 0 and R > 8.  Group
 * rows at or past rh->rdma_capacity are neither written nor forwarded;
 * recv_rdma_offset[G] reports the true total.  `status` (nullable) reads
 * MIEP_ECAPACITY when either the group rows or the receive rows exceed
 * their capacity, else 0. */
miep_status miep_relay_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                int32_t round_scale, const int64_t* topk_idx, const float* topk_weights,
                                const int32_t* num_tokens_per_rank, const int32_t* num_tokens_per_rdma_rank,
                                const int32_t* num_tokens_per_expert, void* rdma_x, float* rdma_x_scales,
                                void* recv_x, float* recv_x_scales, int64_t* recv_topk_idx,
                                float* recv_topk_weights, int32_t* num_recv_tokens_per_expert, int32_t* status,
                                const miep_handle* h, const miep_relay_handle* rh, void* stream);

/* relay_cached_dispatch -- [Ch4] 4.1 cached branch through the relay: with
 * the handles of an earlier miep_relay_dispatch of the same routing, move
 * only x (and its scales) through the group rows to the ranks' rows; no
 * top-k arguments.  Reads h->send_head's placement only through rh
 * (send_rdma_head, recv_rdma_offset, send_nvl_head) and h->recv_rank_offset;
 * arguments as in miep_relay_dispatch. */
miep_status miep_relay_cached_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                       int32_t round_scale, const miep_handle* h, const miep_relay_handle* rh,
                                       void* rdma_x, float* rdma_x_scales, void* recv_x, float* recv_x_scales,
                                       void* stream);

/* relay_combine -- the two-level combine, the reverse of miep_relay_dispatch
 * ([NvLL] normal mode reduces inside the node first, then once more across
 * nodes; [Ch4] 4.4: additions only, weights reduced separately).  First
 * level: each group row sums, in fp32 from its first term, the rows of the
 * group's ranks j ascending that hold it, into rdma_y: rounded to bf16 (the
 * type a partial travels in), or kept fp32 when partial_f32 is set (twice
 * the partial bytes; the result is then one fp32 sum rounded once, which
 * stays within bf16 rounding of the fp32 reference even where partials
 * cancel); the received top-k weights likewise in fp32 into rdma_w.
 * Second level: each source token sums its groups' partials g ascending in
 * fp32, then bias_0 and bias_1 as in miep_combine, rounded once more to
 * bf16.  A token no rank received combines to zero (or its bias).
 *   y                     [cap][H] bf16 expert outputs in the receive layout
 *   recv_topk_weights     [cap][K] fp32, nullable
 *   bias_0, bias_1        [N][H] bf16, nullable
 *   partial_f32           0: bf16 partials, 1: fp32 partials
 *   rdma_y                [rdma_capacity][H] bf16 (or fp32) scratch (out: the partials), 16-byte aligned
 *   rdma_w                [rdma_capacity][K] fp32 scratch, required if recv_topk_weights is given
 *   combined_x            [N][H] bf16 out
 *   combined_topk_weights [N][K] fp32 out, nullable (required if recv_topk_weights is given)
 * Reads h->recv_rank_offset, h->recv_capacity and rh's heads and offsets. */
miep_status miep_relay_combine(const miep_problem* p, const uint16_t* y, const float* recv_topk_weights,
                               const uint16_t* bias_0, const uint16_t* bias_1, const miep_handle* h,
                               const miep_relay_handle* rh, int32_t partial_f32, void* rdma_y, float* rdma_w,
                               uint16_t* combined_x, float* combined_topk_weights, void* stream);

/* Sizes of one low-latency problem, seen from the receiving rank dest_rank. */
typedef struct miep_ll_problem {
  int32_t num_ranks;   /* R: source ranks (all ranks send), 1..1024          */
  int32_t num_tokens;  /* T: tokens per source rank, T <= max_tokens          */
  int32_t max_tokens;  /* M: num_max_dispatch_tokens_per_rank (slot capacity) */
  int32_t hidden;      /* H: H % 8 == 0; with FP8, H % 128 == 0               */
  int32_t num_topk;    /* K */
  int32_t num_experts; /* E: E % R == 0; L = E / R local experts per rank     */
  int32_t dest_rank;   /* d: the receiving rank modelled                      */
} miep_ll_problem;

/* Bytes of one low-latency message ([Phil] message format): a 16-byte
 * header (int32 source token index + 3 reserved int32, zero here), then
 * either H E4M3 bytes and H/128 fp32 scales, or 2H bf16 bytes, rounded up
 * to a multiple of 16 bytes (FP8 with H % 512 != 0: up to 12 padding bytes,
 * left unwritten).  Host-only; -1 for hidden <= 0. */
int64_t miep_ll_msg_bytes(int32_t hidden, int32_t use_fp8);

/* low_latency_dispatch -- [NvLL] low-latency dispatch (send loop, receive
 * layout) and [Ch4] 4.3 outputs.  Send side: every top-k entry of a source
 * token that names one of rank d's local experts becomes one message,
 * written expert-major to slot (l, s, j) of msg_buf; j counts such entries
 * of source s in (token, k) order.  Receive side: for each local expert l
 * the (l, s) blocks are packed in ascending s.
 *   x              [R*T][H] bf16;  topk_idx [R*T][K] int64 (negative = masked)
 *   use_fp8        cast per 128 channels (round_scale: power-of-two scales;
 *                  use_ue8m0 additionally emits exponent bytes, requires round_scale)
 *   msg_buf        [L][R][M] messages of miep_ll_msg_bytes() (16-byte aligned) -- scratch standing in for the transport
 *   msg_count      [L][R] int32 out: messages per (local expert, source), capped at M
 *   packed_recv_x  [L][R*M][H] E4M3 codes, or bf16 without FP8 (rows past the count untouched)
 *   packed_recv_x_scales [L][R*M][H/128] fp32 (FP8 only)
 *   packed_recv_x_scales_ue8m0 [L][R*M][H/128] uint8 exponent + 127, nullable (FP8 + use_ue8m0 only)
 *   packed_recv_src_info [L][R*M] int32: source token index of each row
 *   packed_recv_layout_range [L][R] int64: (first row << 32) | count
 *   packed_recv_count [L] int32: rows per local expert
 *   cumulative_local_expert_recv_stats [L] int32, nullable: += packed_recv_count
 *   mask_buffer    [R] int32, nullable: rank masking ([NvLL] low-latency
 *                  send loop and receive wait), nonzero = masked.  If rank d
 *                  or source s is masked, no message travels from s to d:
 *                  the (l, s) blocks hold 0 rows.
 * Errors: EINVAL for bad sizes or flags, FP8 with H % 128 != 0, or a null
 * required pointer; EUNSUPPORTED for R > 1024, M > 4096, K > 64,
 * H % 8 != 0, or misaligned x / msg_buf / packed_recv_x. */
miep_status miep_ll_dispatch(const miep_ll_problem* q, const uint16_t* x, const int64_t* topk_idx, int32_t use_fp8,
                             int32_t round_scale, int32_t use_ue8m0, void* msg_buf, int32_t* msg_count,
                             void* packed_recv_x, float* packed_recv_x_scales, uint8_t* packed_recv_x_scales_ue8m0,
                             int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                             int32_t* packed_recv_count, int32_t* cumulative_local_expert_recv_stats,
                             const int32_t* mask_buffer, void* stream);

/* low_latency_dispatch_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): miep_ll_dispatch without the message buffer and counts.
 * Same arguments and the same receive side (packed_recv_*, cumulative stats,
 * rank mask) as miep_ll_dispatch; the messages, which only stand in for the
 * transport, are not materialised, and the per-(local expert, source)
 * message counts that its two kernels share live in a device array of the
 * library (65536 int32 per device, held until the process ends).
 * It allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * Every call on one device shares that array: calls that overlap on one
 * device (concurrent streams) race and must be ordered by the caller; each
 * call overwrites every count it reads, so nothing needs clearing.
 * Errors: as miep_ll_dispatch; EUNSUPPORTED when num_experts (L * R counts)
 * exceeds 65536; EHIP if the device address of the array cannot be found. */
miep_status miep_ll_dispatch_noalloc(const miep_ll_problem* q, const uint16_t* x, const int64_t* topk_idx,
                                     int32_t use_fp8, int32_t round_scale, int32_t use_ue8m0, void* packed_recv_x,
                                     float* packed_recv_x_scales, uint8_t* packed_recv_x_scales_ue8m0,
                                     int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                                     int32_t* packed_recv_count, int32_t* cumulative_local_expert_recv_stats,
                                     const int32_t* mask_buffer, void* stream);

/* low_latency_combine -- [Ch4] 4.3 and [NvLL] name it beside the
 * low-latency dispatch without its arithmetic.  Here it is the reverse of
 * miep_ll_dispatch seen from rank d: each source token (s, t) gets back the
 * rows of d's local experts that its top-k entries were sent to (the slot
 * rule of the dispatch: the j-th entry of source s naming expert d*L + l,
 * in (token, k) order, is row l*R*M + begin(l, s) + j), each multiplied by
 * the entry's gate weight when topk_weights is given, summed in fp32 in
 * ascending k and rounded once to bf16.  Entries dropped at the slot cap or
 * by rank masking (slot >= count) contribute nothing; a token without a row
 * combines to +0.0.
 *   y                       [L][R*M][H] bf16 expert outputs, packed like packed_recv_x (16-byte aligned)
 *   packed_recv_src_info    [L][R*M] int32 from miep_ll_dispatch
 *   packed_recv_layout_range [L][R] int64 from miep_ll_dispatch
 *   topk_idx                [R*T][K] int64, the routing given to miep_ll_dispatch
 *   topk_weights            [R*T][K] fp32, nullable (then rows are summed unweighted)
 *   combined_x              [R*T][H] bf16 out (16-byte aligned)
 * A handle from another routing is not detected: a row whose src_info does
 * not name the token is skipped, and every access stays inside y.
 * Errors: as miep_ll_dispatch for sizes; EINVAL for a null required pointer. */
miep_status miep_ll_combine(const miep_ll_problem* q, const uint16_t* y, const int32_t* packed_recv_src_info,
                            const int64_t* packed_recv_layout_range, const int64_t* topk_idx,
                            const float* topk_weights, uint16_t* combined_x, void* stream);

/* Rank mask buffer helpers ([NvLL]: the low-latency buffer's mask can be
 * queried, updated and cleaned; a rank is masked when it stops answering).
 * mask_buffer is [num_ranks] int32 device memory owned by the caller.
 *   update: mask_buffer[rank] = value (nonzero = masked)
 *   clean:  every entry = 0
 *   query:  out[r] = mask_buffer[r] for every r (out: [num_ranks] int32 device)
 * Small kernels (no memset or copy nodes), enqueued on `stream`.
 * Errors: EINVAL for a null pointer, num_ranks <= 0 or rank out of range. */
miep_status miep_mask_update(int32_t* mask_buffer, int32_t num_ranks, int32_t rank, int32_t value, void* stream);
miep_status miep_mask_clean(int32_t* mask_buffer, int32_t num_ranks, void* stream);
miep_status miep_mask_query(const int32_t* mask_buffer, int32_t num_ranks, int32_t* out, void* stream);

/* Description of the last failure on this thread ("" if none). Host-only. */
const char* miep_last_error(void);

/* Library version string. Host-only. */
const char* miep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIEP_H */
