// api.cpp -- the C ABI declared in include/miep.h: argument validation,
// launch-geometry choice and the kernel launches.  Host code only.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "miep.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

miep_status fail(miep_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

miep_status ok() {
  g_err[0] = '\0';
  return MIEP_OK;
}

miep_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MIEP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Cache-policy codes of the relay's launches.  The forwarding pack and the
// group-level combine: non-temporal loads and stores at device scope
// (measured on the 64-rank FP8 relay: dispatch 464 -> 454 us, two-level
// combine 784 -> 750 us against the direct path's codes).  Per launch, the
// first hop keeps plain loads of x (its group rows still stream out) and the
// token-level combine keeps device-scope write-back stores for its output,
// the direct pack's and combine's codes (relay dispatch 430 -> 424 us,
// two-level combine 739 -> 715 us).
constexpr int kRelayCpol = 7;
constexpr int kRelayHop1Cpol = 6;
constexpr int kRelayTokenCpol = 5;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

miep_status check_problem(const miep_problem* p) {
  if (!p) return fail(MIEP_EINVAL, "problem is NULL");
  if (p->num_src < 0 || p->num_tokens < 0) return fail(MIEP_EINVAL, "num_src and num_tokens must be >= 0");
  if (p->hidden <= 0 || p->num_topk <= 0 || p->num_experts <= 0 || p->num_ranks <= 0 || p->num_channels <= 0)
    return fail(MIEP_EINVAL, "hidden, num_topk, num_experts, num_ranks, num_channels must be > 0");
  if (p->expert_alignment <= 0) return fail(MIEP_EINVAL, "expert_alignment must be >= 1");
  if (p->num_experts % p->num_ranks != 0) return fail(MIEP_EINVAL, "num_experts must be a multiple of num_ranks");
  if (p->num_ranks > 8 && p->num_ranks % 8 != 0)
    return fail(MIEP_EINVAL, "num_ranks > 8 must be a multiple of 8 (RDMA groups of 8 ranks)");
  if (p->num_ranks > miep::kMaxRanks) return fail(MIEP_EUNSUPPORTED, "num_ranks > %d", miep::kMaxRanks);
  if (p->num_experts > miep::kMaxExperts) return fail(MIEP_EUNSUPPORTED, "num_experts > %d", miep::kMaxExperts);
  if (p->num_topk > 64) return fail(MIEP_EUNSUPPORTED, "num_topk > 64");
  if (static_cast<int64_t>(p->num_src) * p->num_tokens > (1ll << 31) - 1)
    return fail(MIEP_EUNSUPPORTED, "more than 2^31-1 tokens");
  if (p->num_src > (1 << 20)) return fail(MIEP_EUNSUPPORTED, "num_src > 2^20");
  if (p->num_channels > 1024) return fail(MIEP_EUNSUPPORTED, "num_channels > 1024");
  if (p->hidden > (1 << 24)) return fail(MIEP_EUNSUPPORTED, "hidden > 2^24");
  return ok();
}

// A dispatch's receive rows (and their prefixes in the handle) are int32: a
// token reaches at most min(K, R) ranks, so N * min(K, R) bounds the total.
miep_status check_rows(const miep_problem* p) {
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  const int64_t fan = p->num_topk < p->num_ranks ? p->num_topk : p->num_ranks;
  if (N * fan > (1ll << 31) - 1)
    return fail(MIEP_EUNSUPPORTED, "num_src * num_tokens * min(num_topk, num_ranks) > 2^31-1 (int32 receive rows)");
  return ok();
}

static_assert(miep::kStatusCapacity == MIEP_ECAPACITY, "device status code must match the header");

// use_ue8m0 needs power-of-two scales from the fused cast, and somewhere to put the bytes
miep_status check_ue8m0(int32_t x_kind, int32_t round_scale, int32_t use_ue8m0, const uint8_t* out, int64_t cap) {
  if (!use_ue8m0) return MIEP_OK;
  if (x_kind != MIEP_X_BF16_CAST_FP8 || !round_scale)
    return fail(MIEP_EINVAL, "use_ue8m0 needs x_kind MIEP_X_BF16_CAST_FP8 with round_scale");
  if (cap > 0 && !out) return fail(MIEP_EINVAL, "recv_x_scales_ue8m0 is NULL with use_ue8m0");
  return MIEP_OK;
}

miep_status check_payload(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales) {
  if (x_kind != MIEP_X_BF16 && x_kind != MIEP_X_FP8 && x_kind != MIEP_X_BF16_CAST_FP8)
    return fail(MIEP_EINVAL, "unknown x_kind %d", x_kind);
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (N > 0 && !x) return fail(MIEP_EINVAL, "x is NULL");
  if (!aligned16(x)) return fail(MIEP_EUNSUPPORTED, "x must be 16-byte aligned");
  if (p->hidden % 8 != 0) return fail(MIEP_EUNSUPPORTED, "hidden must be a multiple of 8 (16-byte rows)");
  if (x_kind != MIEP_X_BF16) {
    if (p->hidden % miep::kFp8Group != 0) return fail(MIEP_EINVAL, "FP8 payloads need hidden % 128 == 0");
    if (x_kind == MIEP_X_BF16_CAST_FP8 && p->hidden > 65536)
      return fail(MIEP_EUNSUPPORTED, "the fused FP8 cast supports hidden <= 65536");
    if (x_kind == MIEP_X_FP8 && N > 0 && !x_scales) return fail(MIEP_EINVAL, "x_scales is NULL for MIEP_X_FP8");
  }
  return ok();
}

// Arrays of zero elements may be NULL (empty tensors carry no storage).
miep_status check_handle(const miep_problem* p, const miep_handle* h, bool full) {
  if (!h) return fail(MIEP_EINVAL, "handle is NULL");
  if (h->recv_capacity < 0 || h->recv_capacity > (1ll << 31) - 1)
    return fail(MIEP_EINVAL, "recv_capacity must be in [0, 2^31-1]");
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (!h->recv_rank_offset) return fail(MIEP_EINVAL, "handle recv_rank_offset is NULL");
  if (N > 0 && !h->send_head) return fail(MIEP_EINVAL, "handle send_head is NULL");
  if (full) {
    if (p->num_src > 0 && (!h->rank_prefix_matrix || !h->channel_prefix_matrix || !h->recv_channel_prefix_matrix))
      return fail(MIEP_EINVAL, "handle prefix matrices are NULL");
    if (h->recv_capacity > 0 && !h->recv_src_idx) return fail(MIEP_EINVAL, "handle recv_src_idx is NULL");
    if (N > 0 && !h->is_token_in_rank) return fail(MIEP_EINVAL, "handle is_token_in_rank is NULL");
  }
  return ok();
}

miep::PackArgs pack_args(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                         int32_t round_scale, const miep_handle* h, void* recv_x, float* recv_x_scales) {
  miep::PackArgs a{};
  a.N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  a.T = p->num_tokens;
  a.H = p->hidden;
  a.K = p->num_topk;
  a.E = p->num_experts;
  a.R = p->num_ranks;
  a.L = p->num_experts / p->num_ranks;
  a.kind = x_kind;
  a.round_scale = round_scale;
  a.capacity = h->recv_capacity;
  a.x = x;
  a.x_scales = x_scales;
  a.send_head = h->send_head;
  a.off = h->recv_rank_offset;
  a.recv_x = recv_x;
  a.recv_x_scales = recv_x_scales;
  return a;
}

// The relay's group-row arrays (G = R / 8 groups).
miep_status check_relay(const miep_problem* p, const miep_relay_handle* rh) {
  if (!rh) return fail(MIEP_EINVAL, "relay handle is NULL");
  if (p->num_ranks % 8 != 0 || p->num_ranks <= 8)
    return fail(MIEP_EUNSUPPORTED, "the relay needs num_ranks > 8 and a multiple of 8");
  if (rh->rdma_capacity < 0 || rh->rdma_capacity > (1ll << 31) - 1)
    return fail(MIEP_EINVAL, "rdma_capacity out of range");
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (!rh->recv_rdma_offset) return fail(MIEP_EINVAL, "relay recv_rdma_offset is NULL");
  if (N > 0 && !rh->send_rdma_head) return fail(MIEP_EINVAL, "relay send_rdma_head is NULL");
  if (rh->rdma_capacity > 0 && (!rh->send_nvl_head || !rh->rdma_src_idx))
    return fail(MIEP_EINVAL, "relay send_nvl_head / rdma_src_idx is NULL");
  if (!aligned16(rh->send_nvl_head) || !aligned16(rh->send_rdma_head))
    return fail(MIEP_EUNSUPPORTED, "send_nvl_head and send_rdma_head must be 16-byte aligned");
  return MIEP_OK;
}

miep::NotifyArgs notify_args(const miep_problem* p, const miep_handle* h, const int32_t* ntpr, const int32_t* ntpe,
                             int32_t* nrte) {
  miep::NotifyArgs na{};
  na.S = p->num_src;
  na.T = p->num_tokens;
  na.R = p->num_ranks;
  na.C = p->num_channels;
  na.E = p->num_experts;
  na.L = p->num_experts / p->num_ranks;
  na.align = p->expert_alignment;
  na.tcdiv = miep::make_fastdiv(p->num_tokens > 0 ? (p->num_tokens + p->num_channels - 1) / p->num_channels : 1);
  na.nonempty = p->num_tokens > 0 ? (p->num_tokens + na.tcdiv.d - 1) / na.tcdiv.d : 0;
  na.in_rank = h->is_token_in_rank;
  na.ntpr = ntpr;
  na.ntpe = ntpe;
  na.rpm = h->rank_prefix_matrix;
  na.cpm = h->channel_prefix_matrix;
  na.rcpm = h->recv_channel_prefix_matrix;
  na.off = h->recv_rank_offset;
  na.send_head = h->send_head;
  na.nrte = nrte;
  return na;
}

// Sizes of a low-latency problem (shared by dispatch and combine).
miep_status check_ll_problem(const miep_ll_problem* q) {
  if (!q) return fail(MIEP_EINVAL, "problem is NULL");
  const int R = q->num_ranks, T = q->num_tokens, M = q->max_tokens, H = q->hidden, K = q->num_topk,
            E = q->num_experts, d = q->dest_rank;
  if (R <= 0 || T < 0 || M <= 0 || H <= 0 || K <= 0 || E <= 0) return fail(MIEP_EINVAL, "sizes must be positive");
  if (T > M) return fail(MIEP_EINVAL, "num_tokens > max_tokens");
  if (E % R != 0) return fail(MIEP_EINVAL, "num_experts must be a multiple of num_ranks");
  if (d < 0 || d >= R) return fail(MIEP_EINVAL, "dest_rank out of range");
  if (R > 1024) return fail(MIEP_EUNSUPPORTED, "num_ranks > 1024");
  if (M > 4096) return fail(MIEP_EUNSUPPORTED, "max_tokens > 4096");
  if (K > 64) return fail(MIEP_EUNSUPPORTED, "num_topk > 64");
  if (H % 8 != 0) return fail(MIEP_EUNSUPPORTED, "hidden must be a multiple of 8");
  if (static_cast<int64_t>(E) * M > (1ll << 31) - 1) return fail(MIEP_EUNSUPPORTED, "num_experts * max_tokens >= 2^31");
  return MIEP_OK;
}

}  // namespace

namespace miep {
const Tuning& tuning() {
  static const Tuning t = {env_int("MIEP_PACK_VPL", 0),     env_int("MIEP_PACK_SLICES", 0),
                           env_int("MIEP_COMBINE_VPL", 0),  env_int("MIEP_COMBINE_SLICES", 0),
                           env_int("MIEP_COMBINE_MAXR", 0),
                           env_int("MIEP_PACK_NT", -1),    env_int("MIEP_COMBINE_NT", -1),
                           env_int("MIEP_LL_SPLIT", 0),     env_int("MIEP_LL_VPL", 0),
                           env_int("MIEP_CAST_TPB", -1),    env_int("MIEP_LLC_VPL", 0),
                           env_int("MIEP_LLC_SLICES", 0),   env_int("MIEP_LLC_NT", -1),
                           env_int("MIEP_LL_NT", -1),       env_int("MIEP_PACK_RECORDS", -1),
                           env_int("MIEP_LL_TPB", 0),       env_int("MIEP_LL_COUNT_SRC", -1),
                           env_int("MIEP_NOTIFY_CHAN", -1), env_int("MIEP_BIAS_NT", -1)};
  return t;
}
}  // namespace miep

extern "C" {

const char* miep_last_error(void) { return g_err; }

const char* miep_version(void) { return "miep 0.1 gfx950"; }

int64_t miep_ll_msg_bytes(int32_t hidden, int32_t use_fp8) {
  if (hidden <= 0) return -1;
  const int64_t used = 16 + (use_fp8 ? static_cast<int64_t>(hidden) + 4ll * (hidden / miep::kFp8Group) : 2ll * hidden);
  return (used + 15) / 16 * 16;   // 16-byte message stride
}

miep_status miep_get_dispatch_layout(const miep_problem* p, const int64_t* topk_idx, int32_t* num_tokens_per_rank,
                                     int32_t* num_tokens_per_rdma_rank, int32_t* num_tokens_per_expert,
                                     uint8_t* is_token_in_rank, void* stream) {
  miep_status st = check_problem(p);
  if (st != MIEP_OK) return st;
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (p->num_src > 0 && (!num_tokens_per_rank || !num_tokens_per_expert))
    return fail(MIEP_EINVAL, "num_tokens_per_rank / num_tokens_per_expert NULL");
  if (N > 0 && (!topk_idx || !is_token_in_rank)) return fail(MIEP_EINVAL, "topk_idx / is_token_in_rank NULL");
  if (p->num_ranks > 8 && p->num_src > 0 && !num_tokens_per_rdma_rank)
    return fail(MIEP_EINVAL, "num_tokens_per_rdma_rank required when num_ranks > 8");
  if (p->num_ranks <= 8 && num_tokens_per_rdma_rank)
    return fail(MIEP_EINVAL, "num_tokens_per_rdma_rank must be NULL when num_ranks <= 8");
  if ((reinterpret_cast<uintptr_t>(is_token_in_rank) & 3u) != 0)
    return fail(MIEP_EUNSUPPORTED, "is_token_in_rank must be 4-byte aligned");
  miep::LayoutArgs a{};
  a.S = p->num_src;
  a.T = p->num_tokens;
  a.K = p->num_topk;
  a.E = p->num_experts;
  a.R = p->num_ranks;
  a.L = p->num_experts / p->num_ranks;
  a.Ldiv = miep::make_fastdiv(a.L);
  a.topk_idx = topk_idx;
  a.ntpr = num_tokens_per_rank;
  a.ntp_rdma = num_tokens_per_rdma_rank;
  a.ntpe = num_tokens_per_expert;
  a.in_rank = is_token_in_rank;
  return hip_status(miep::launch_layout(a, static_cast<hipStream_t>(stream)), "layout launch");
}

miep_status miep_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                          int32_t round_scale, int32_t use_ue8m0, const int64_t* topk_idx, const float* topk_weights,
                          const int32_t* num_tokens_per_rank, const int32_t* num_tokens_per_expert, void* recv_x,
                          float* recv_x_scales, uint8_t* recv_x_scales_ue8m0, int64_t* recv_topk_idx,
                          float* recv_topk_weights, int32_t* num_recv_tokens_per_expert, int32_t* status,
                          const miep_handle* h, void* stream) {
  miep_status st = check_problem(p);
  if (st == MIEP_OK) st = check_rows(p);
  if (st != MIEP_OK) return st;
  if ((st = check_payload(p, x, x_kind, x_scales)) != MIEP_OK) return st;
  if ((st = check_handle(p, h, true)) != MIEP_OK) return st;
  if ((st = check_ue8m0(x_kind, round_scale, use_ue8m0, recv_x_scales_ue8m0, h->recv_capacity)) != MIEP_OK) return st;
  if (p->num_src > 0 && !num_tokens_per_rank) return fail(MIEP_EINVAL, "num_tokens_per_rank is NULL");
  if (h->recv_capacity > 0 && !recv_x) return fail(MIEP_EINVAL, "recv_x is NULL");
  if (!aligned16(recv_x)) return fail(MIEP_EUNSUPPORTED, "recv_x must be 16-byte aligned");
  if (x_kind != MIEP_X_BF16 && h->recv_capacity > 0 && !recv_x_scales)
    return fail(MIEP_EINVAL, "recv_x_scales is NULL for an FP8 dispatch");
  if (topk_idx && h->recv_capacity > 0 && !recv_topk_idx) return fail(MIEP_EINVAL, "recv_topk_idx is NULL");
  if (topk_weights && !topk_idx) return fail(MIEP_EINVAL, "topk_weights given without topk_idx");
  if (topk_weights && h->recv_capacity > 0 && !recv_topk_weights)
    return fail(MIEP_EINVAL, "recv_topk_weights is NULL");
  if (num_recv_tokens_per_expert && !num_tokens_per_expert)
    return fail(MIEP_EINVAL, "num_recv_tokens_per_expert needs num_tokens_per_expert");
  if (p->num_ranks % 4 == 0 && (reinterpret_cast<uintptr_t>(h->send_head) & 15u) != 0)
    return fail(MIEP_EUNSUPPORTED, "send_head must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(h->is_token_in_rank) & 3u) != 0)
    return fail(MIEP_EUNSUPPORTED, "is_token_in_rank must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);

  miep::NotifyArgs na = notify_args(p, h, num_tokens_per_rank, num_tokens_per_expert, num_recv_tokens_per_expert);
  na.status = status;
  na.capacity = h->recv_capacity;
  if (p->num_src == 0) {
    // no sources: every receive offset is 0, every expert count is 0, nothing overflows
    hipError_t e = miep::launch_fill_zero(h->recv_rank_offset, p->num_ranks + 1, s);
    if (e == hipSuccess && num_recv_tokens_per_expert)
      e = miep::launch_fill_zero(num_recv_tokens_per_expert, p->num_experts, s);
    if (e == hipSuccess && status) e = miep::launch_fill_zero(status, 1, s);
    return hip_status(e, "dispatch (no sources)");
  }
  hipError_t e = miep::launch_notify(na, s);
  if (e != hipSuccess) return hip_status(e, "notify launch");

  miep::PackArgs a = pack_args(p, x, x_kind, x_scales, round_scale, h, recv_x, recv_x_scales);
  a.recv_ue = use_ue8m0 ? recv_x_scales_ue8m0 : nullptr;
  a.meta = 1;
  a.S = p->num_src;
  a.rpm = h->rank_prefix_matrix;
  a.in_rank = h->is_token_in_rank;
  a.topk_idx = topk_idx;
  a.topk_weights = topk_weights;
  a.recv_topk_idx = topk_idx ? recv_topk_idx : nullptr;
  a.recv_topk_weights = topk_weights ? recv_topk_weights : nullptr;
  a.recv_src_idx = h->recv_src_idx;
  if (!topk_idx) a.K = 0;
  return hip_status(miep::launch_pack(a, s), "pack launch");
}

miep_status miep_cached_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                 int32_t round_scale, int32_t use_ue8m0, const miep_handle* h, void* recv_x,
                                 float* recv_x_scales, uint8_t* recv_x_scales_ue8m0, void* stream) {
  miep_status st = check_problem(p);
  if (st != MIEP_OK) return st;
  if ((st = check_payload(p, x, x_kind, x_scales)) != MIEP_OK) return st;
  if ((st = check_handle(p, h, false)) != MIEP_OK) return st;
  if ((st = check_ue8m0(x_kind, round_scale, use_ue8m0, recv_x_scales_ue8m0, h->recv_capacity)) != MIEP_OK) return st;
  if (h->recv_capacity > 0 && !recv_x) return fail(MIEP_EINVAL, "recv_x is NULL");
  if (!aligned16(recv_x)) return fail(MIEP_EUNSUPPORTED, "recv_x must be 16-byte aligned");
  if (x_kind != MIEP_X_BF16 && h->recv_capacity > 0 && !recv_x_scales)
    return fail(MIEP_EINVAL, "recv_x_scales is NULL for an FP8 dispatch");
  miep::PackArgs a = pack_args(p, x, x_kind, x_scales, round_scale, h, recv_x, recv_x_scales);
  a.recv_ue = use_ue8m0 ? recv_x_scales_ue8m0 : nullptr;
  a.meta = 0;
  a.K = 0;
  return hip_status(miep::launch_pack(a, static_cast<hipStream_t>(stream)), "cached pack launch");
}

miep_status miep_check_status(const int32_t* status, void* stream) {
  if (!status) return fail(MIEP_EINVAL, "status is NULL");
  int32_t v = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&v, status, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "status read");
  if (v == MIEP_OK) return ok();
  if (v == MIEP_ECAPACITY)
    return fail(MIEP_ECAPACITY, "the receive side needed more rows than its fixed capacity; rows past it were dropped");
  return fail(MIEP_EINVAL, "status word holds %d, not a status a dispatch writes", v);
}

miep_status miep_combine(const miep_problem* p, const uint16_t* y, const float* recv_topk_weights,
                         const uint16_t* bias_0, const uint16_t* bias_1, const miep_handle* h,
                         uint16_t* combined_x, float* combined_topk_weights, void* stream) {
  miep_status st = check_problem(p);
  if (st != MIEP_OK) return st;
  if ((st = check_handle(p, h, false)) != MIEP_OK) return st;
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (p->hidden % 8 != 0) return fail(MIEP_EUNSUPPORTED, "hidden must be a multiple of 8 (16-byte rows)");
  if (h->recv_capacity > 0 && !y) return fail(MIEP_EINVAL, "y is NULL");
  if (N > 0 && !combined_x) return fail(MIEP_EINVAL, "combined_x is NULL");
  if (!aligned16(y) || !aligned16(combined_x)) return fail(MIEP_EUNSUPPORTED, "y and combined_x must be 16-byte aligned");
  if (!aligned16(bias_0) || !aligned16(bias_1)) return fail(MIEP_EUNSUPPORTED, "bias rows must be 16-byte aligned");
  if (recv_topk_weights && N > 0 && !combined_topk_weights)
    return fail(MIEP_EINVAL, "combined_topk_weights is NULL while recv_topk_weights is given");
  miep::CombineArgs a{};
  a.N = N;
  a.H = p->hidden;
  a.K = p->num_topk;
  a.R = p->num_ranks;
  a.capacity = h->recv_capacity;
  a.y = y;
  a.w = recv_topk_weights;
  a.bias0 = N > 0 ? bias_0 : nullptr;
  a.bias1 = N > 0 ? bias_1 : nullptr;
  a.send_head = h->send_head;
  a.off = h->recv_rank_offset;
  a.out = combined_x;
  a.out_w = combined_topk_weights;
  return hip_status(miep::launch_combine(a, static_cast<hipStream_t>(stream)), "combine launch");
}

miep_status miep_relay_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                int32_t round_scale, const int64_t* topk_idx, const float* topk_weights,
                                const int32_t* num_tokens_per_rank, const int32_t* num_tokens_per_rdma_rank,
                                const int32_t* num_tokens_per_expert, void* rdma_x, float* rdma_x_scales,
                                void* recv_x, float* recv_x_scales, int64_t* recv_topk_idx,
                                float* recv_topk_weights, int32_t* num_recv_tokens_per_expert, int32_t* status,
                                const miep_handle* h, const miep_relay_handle* rh, void* stream) {
  miep_status st = check_problem(p);
  if (st == MIEP_OK) st = check_rows(p);
  if (st != MIEP_OK) return st;
  if ((st = check_payload(p, x, x_kind, x_scales)) != MIEP_OK) return st;
  if ((st = check_handle(p, h, true)) != MIEP_OK) return st;
  if ((st = check_relay(p, rh)) != MIEP_OK) return st;
  const int G = p->num_ranks / 8;
  if (p->num_src > 0 && (!num_tokens_per_rank || !num_tokens_per_rdma_rank))
    return fail(MIEP_EINVAL, "num_tokens_per_rank / num_tokens_per_rdma_rank is NULL");
  if (h->recv_capacity > 0 && !recv_x) return fail(MIEP_EINVAL, "recv_x is NULL");
  if (rh->rdma_capacity > 0 && !rdma_x) return fail(MIEP_EINVAL, "rdma_x is NULL");
  if (!aligned16(recv_x) || !aligned16(rdma_x)) return fail(MIEP_EUNSUPPORTED, "recv_x and rdma_x must be 16-byte aligned");
  if (x_kind != MIEP_X_BF16 && ((h->recv_capacity > 0 && !recv_x_scales) || (rh->rdma_capacity > 0 && !rdma_x_scales)))
    return fail(MIEP_EINVAL, "recv_x_scales / rdma_x_scales is NULL for an FP8 dispatch");
  if (topk_idx && h->recv_capacity > 0 && !recv_topk_idx) return fail(MIEP_EINVAL, "recv_topk_idx is NULL");
  if (topk_weights && !topk_idx) return fail(MIEP_EINVAL, "topk_weights given without topk_idx");
  if (topk_weights && h->recv_capacity > 0 && !recv_topk_weights)
    return fail(MIEP_EINVAL, "recv_topk_weights is NULL");
  if (num_recv_tokens_per_expert && !num_tokens_per_expert)
    return fail(MIEP_EINVAL, "num_recv_tokens_per_expert needs num_tokens_per_expert");
  if (!aligned16(h->send_head)) return fail(MIEP_EUNSUPPORTED, "send_head must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(h->is_token_in_rank) & 7u) != 0)
    return fail(MIEP_EUNSUPPORTED, "is_token_in_rank must be 8-byte aligned for the relay");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->num_src == 0) {
    hipError_t e = miep::launch_fill_zero(h->recv_rank_offset, p->num_ranks + 1, s);
    if (e == hipSuccess) e = miep::launch_fill_zero(rh->recv_rdma_offset, G + 1, s);
    if (e == hipSuccess && num_recv_tokens_per_expert)
      e = miep::launch_fill_zero(num_recv_tokens_per_expert, p->num_experts, s);
    if (e == hipSuccess && status) e = miep::launch_fill_zero(status, 1, s);
    return hip_status(e, "relay dispatch (no sources)");
  }
  // the ranks' handle (the receive side is the direct dispatch's)
  miep::NotifyArgs na = notify_args(p, h, num_tokens_per_rank, num_tokens_per_expert, num_recv_tokens_per_expert);
  na.status = status;
  na.capacity = h->recv_capacity;
  hipError_t e = miep::launch_notify(na, s);
  if (e != hipSuccess) return hip_status(e, "notify launch");
  // the groups' prefix matrices, offsets and send_rdma_head
  miep::NotifyArgs ng = na;
  ng.R = G;
  ng.group_w = 8;
  ng.E = 0;
  ng.ntpr = num_tokens_per_rdma_rank;
  ng.ntpe = nullptr;
  ng.nrte = nullptr;
  ng.rpm = rh->rdma_rank_prefix_matrix;
  ng.cpm = rh->rdma_channel_prefix_matrix;
  ng.rcpm = rh->recv_rdma_channel_prefix_matrix;
  ng.off = rh->recv_rdma_offset;
  ng.send_head = rh->send_rdma_head;
  ng.capacity = rh->rdma_capacity;
  ng.status_or = 1;                  // keeps the first notify's status word, ORs in the group rows' overflow
  e = miep::launch_notify(ng, s);
  if (e != hipSuccess) return hip_status(e, "group notify launch");
  miep::RelayMetaArgs rm{};
  rm.N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  rm.G = G;
  rm.R = p->num_ranks;
  rm.rdma_capacity = rh->rdma_capacity;
  rm.send_rdma_head = rh->send_rdma_head;
  rm.rdma_off = rh->recv_rdma_offset;
  rm.send_head = h->send_head;
  rm.rdma_src_idx = rh->rdma_src_idx;
  rm.send_nvl_head = rh->send_nvl_head;
  e = miep::launch_relay_meta(rm, s);
  if (e != hipSuccess) return hip_status(e, "relay meta launch");
  // first hop: every token once into each destination group's rows
  miep::PackArgs a1 = pack_args(p, x, x_kind, x_scales, round_scale, h, rdma_x, rdma_x_scales);
  a1.R = G;
  a1.send_head = rh->send_rdma_head;
  a1.off = rh->recv_rdma_offset;
  a1.capacity = rh->rdma_capacity;
  a1.meta = 0;
  a1.cpol = kRelayHop1Cpol;
  e = miep::launch_pack(a1, s);
  if (e != hipSuccess) return hip_status(e, "relay pack launch");
  // second hop: every group row to the group's receiving ranks, with metadata
  const int fwd_kind = x_kind == MIEP_X_BF16 ? MIEP_X_BF16 : MIEP_X_FP8;
  miep::PackArgs a2 = pack_args(p, rdma_x, fwd_kind, rdma_x_scales, 0, h, recv_x, recv_x_scales);
  a2.N = rh->rdma_capacity;
  a2.R = 8;
  a2.send_head = rh->send_nvl_head;
  a2.meta = 1;
  a2.topk_idx = topk_idx;
  a2.topk_weights = topk_weights;
  a2.recv_topk_idx = topk_idx ? recv_topk_idx : nullptr;
  a2.recv_topk_weights = topk_weights ? recv_topk_weights : nullptr;
  a2.recv_src_idx = h->recv_src_idx;
  if (!topk_idx) a2.K = 0;
  a2.count = rh->recv_rdma_offset + G;
  a2.group_off = rh->recv_rdma_offset;
  a2.groups = G;
  a2.group_w = 8;
  a2.src_tok = rh->rdma_src_idx;
  a2.cpol = kRelayCpol;
  return hip_status(miep::launch_pack(a2, s), "relay forward launch");
}

miep_status miep_relay_cached_dispatch(const miep_problem* p, const void* x, int32_t x_kind, const float* x_scales,
                                       int32_t round_scale, const miep_handle* h, const miep_relay_handle* rh,
                                       void* rdma_x, float* rdma_x_scales, void* recv_x, float* recv_x_scales,
                                       void* stream) {
  miep_status st = check_problem(p);
  if (st != MIEP_OK) return st;
  if ((st = check_payload(p, x, x_kind, x_scales)) != MIEP_OK) return st;
  if ((st = check_handle(p, h, false)) != MIEP_OK) return st;
  if ((st = check_relay(p, rh)) != MIEP_OK) return st;
  const int G = p->num_ranks / 8;
  if (h->recv_capacity > 0 && !recv_x) return fail(MIEP_EINVAL, "recv_x is NULL");
  if (rh->rdma_capacity > 0 && !rdma_x) return fail(MIEP_EINVAL, "rdma_x is NULL");
  if (!aligned16(recv_x) || !aligned16(rdma_x)) return fail(MIEP_EUNSUPPORTED, "recv_x and rdma_x must be 16-byte aligned");
  if (x_kind != MIEP_X_BF16 && ((h->recv_capacity > 0 && !recv_x_scales) || (rh->rdma_capacity > 0 && !rdma_x_scales)))
    return fail(MIEP_EINVAL, "recv_x_scales / rdma_x_scales is NULL for an FP8 dispatch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  miep::PackArgs a1 = pack_args(p, x, x_kind, x_scales, round_scale, h, rdma_x, rdma_x_scales);
  a1.R = G;
  a1.send_head = rh->send_rdma_head;
  a1.off = rh->recv_rdma_offset;
  a1.capacity = rh->rdma_capacity;
  a1.meta = 0;
  a1.cpol = kRelayHop1Cpol;
  hipError_t e = miep::launch_pack(a1, s);
  if (e != hipSuccess) return hip_status(e, "relay pack launch");
  const int fwd_kind = x_kind == MIEP_X_BF16 ? MIEP_X_BF16 : MIEP_X_FP8;
  miep::PackArgs a2 = pack_args(p, rdma_x, fwd_kind, rdma_x_scales, 0, h, recv_x, recv_x_scales);
  a2.N = rh->rdma_capacity;
  a2.R = 8;
  a2.send_head = rh->send_nvl_head;
  a2.meta = 0;
  a2.count = rh->recv_rdma_offset + G;
  a2.group_off = rh->recv_rdma_offset;
  a2.groups = G;
  a2.group_w = 8;
  a2.cpol = kRelayCpol;
  return hip_status(miep::launch_pack(a2, s), "relay forward launch");
}

miep_status miep_relay_combine(const miep_problem* p, const uint16_t* y, const float* recv_topk_weights,
                               const uint16_t* bias_0, const uint16_t* bias_1, const miep_handle* h,
                               const miep_relay_handle* rh, int32_t partial_f32, void* rdma_y, float* rdma_w,
                               uint16_t* combined_x, float* combined_topk_weights, void* stream) {
  miep_status st = check_problem(p);
  if (st != MIEP_OK) return st;
  if ((st = check_handle(p, h, false)) != MIEP_OK) return st;
  if ((st = check_relay(p, rh)) != MIEP_OK) return st;
  const int G = p->num_ranks / 8;
  const int64_t N = static_cast<int64_t>(p->num_src) * p->num_tokens;
  if (p->hidden % 8 != 0) return fail(MIEP_EUNSUPPORTED, "hidden must be a multiple of 8 (16-byte rows)");
  if (h->recv_capacity > 0 && !y) return fail(MIEP_EINVAL, "y is NULL");
  if (rh->rdma_capacity > 0 && !rdma_y) return fail(MIEP_EINVAL, "rdma_y is NULL");
  if (N > 0 && !combined_x) return fail(MIEP_EINVAL, "combined_x is NULL");
  if (!aligned16(y) || !aligned16(rdma_y) || !aligned16(combined_x) || !aligned16(bias_0) || !aligned16(bias_1))
    return fail(MIEP_EUNSUPPORTED, "y, rdma_y, combined_x and bias rows must be 16-byte aligned");
  if (recv_topk_weights && ((rh->rdma_capacity > 0 && !rdma_w) || (N > 0 && !combined_topk_weights)))
    return fail(MIEP_EINVAL, "rdma_w / combined_topk_weights is NULL while recv_topk_weights is given");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // first level: each group row sums its group's ranks' rows
  miep::CombineArgs c1{};
  c1.N = rh->rdma_capacity;
  c1.H = p->hidden;
  c1.K = p->num_topk;
  c1.R = 8;
  c1.capacity = h->recv_capacity;
  c1.y = y;
  c1.w = recv_topk_weights;
  c1.send_head = rh->send_nvl_head;
  c1.off = h->recv_rank_offset;
  c1.out = static_cast<uint16_t*>(rdma_y);
  c1.out_f32 = partial_f32 ? 1 : 0;
  c1.out_w = recv_topk_weights ? rdma_w : nullptr;
  c1.count = rh->recv_rdma_offset + G;
  c1.group_off = rh->recv_rdma_offset;
  c1.groups = G;
  c1.group_w = 8;
  c1.cpol = kRelayCpol;
  hipError_t e = miep::launch_combine(c1, s);
  if (e != hipSuccess) return hip_status(e, "relay combine (group level) launch");
  // second level: each token sums its groups' partial rows, then the bias
  miep::CombineArgs c2{};
  c2.N = N;
  c2.H = p->hidden;
  c2.K = p->num_topk;
  c2.R = G;
  c2.capacity = rh->rdma_capacity;
  c2.y = static_cast<const uint16_t*>(rdma_y);
  c2.in_f32 = partial_f32 ? 1 : 0;
  c2.w = recv_topk_weights ? rdma_w : nullptr;
  c2.bias0 = N > 0 ? bias_0 : nullptr;
  c2.bias1 = N > 0 ? bias_1 : nullptr;
  c2.send_head = rh->send_rdma_head;
  c2.off = rh->recv_rdma_offset;
  c2.out = combined_x;
  c2.out_w = combined_topk_weights;
  c2.cpol = kRelayTokenCpol;
  return hip_status(miep::launch_combine(c2, s), "relay combine (token level) launch");
}

}  // extern "C"

namespace {

// Checks and arguments of a low-latency dispatch.  with_msgs: the caller's
// message buffer and counts (msg_buf, msg_count) are required; otherwise
// they are null and the caller fills a.msg_count.
miep_status ll_dispatch_args(const miep_ll_problem* q, const uint16_t* x, const int64_t* topk_idx, int32_t use_fp8,
                             int32_t round_scale, int32_t use_ue8m0, void* msg_buf, int32_t* msg_count,
                             void* packed_recv_x, float* packed_recv_x_scales, uint8_t* packed_recv_x_scales_ue8m0,
                             int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                             int32_t* packed_recv_count, int32_t* cumulative_local_expert_recv_stats,
                             const int32_t* mask_buffer, bool with_msgs, miep::LLArgs* out) {
  miep_status st = check_ll_problem(q);
  if (st != MIEP_OK) return st;
  const int R = q->num_ranks, T = q->num_tokens, M = q->max_tokens, H = q->hidden, K = q->num_topk,
            E = q->num_experts, d = q->dest_rank;
  if (use_ue8m0 && !round_scale) return fail(MIEP_EINVAL, "use_ue8m0 requires round_scale");
  if (use_ue8m0 && !use_fp8) return fail(MIEP_EINVAL, "use_ue8m0 requires use_fp8");
  if (use_fp8 && H % miep::kFp8Group != 0)
    return fail(MIEP_EINVAL, "FP8 low-latency messages need hidden % 128 == 0 (whole scale groups)");
  if ((T > 0 && (!x || !topk_idx)) || (with_msgs && (!msg_buf || !msg_count)) || !packed_recv_x ||
      !packed_recv_src_info || !packed_recv_layout_range || !packed_recv_count)
    return fail(MIEP_EINVAL, "a required pointer is NULL");
  if (use_fp8 && !packed_recv_x_scales) return fail(MIEP_EINVAL, "packed_recv_x_scales is NULL with use_fp8");
  if (!aligned16(x) || !aligned16(msg_buf) || !aligned16(packed_recv_x))
    return fail(MIEP_EUNSUPPORTED, "x, msg_buf and packed_recv_x must be 16-byte aligned");
  miep::LLArgs& a = *out;
  a = miep::LLArgs{};
  a.R = R;
  a.T = T;
  a.M = M;
  a.H = H;
  a.K = K;
  a.E = E;
  a.L = E / R;
  a.d = d;
  a.use_fp8 = use_fp8 ? 1 : 0;
  a.round_scale = round_scale ? 1 : 0;
  a.use_ue8m0 = use_ue8m0 ? 1 : 0;
  a.msg_bytes = miep_ll_msg_bytes(H, use_fp8);
  a.x = x;
  a.topk_idx = topk_idx;
  a.msg = static_cast<uint8_t*>(msg_buf);
  a.msg_count = msg_count;
  a.prx = packed_recv_x;
  a.prs = packed_recv_x_scales;
  a.prue = (use_fp8 && use_ue8m0) ? packed_recv_x_scales_ue8m0 : nullptr;
  a.src_info = packed_recv_src_info;
  a.layout_range = packed_recv_layout_range;
  a.count = packed_recv_count;
  a.cumulative = cumulative_local_expert_recv_stats;
  a.mask = mask_buffer;
  return ok();
}

}  // namespace

extern "C" {

miep_status miep_ll_dispatch(const miep_ll_problem* q, const uint16_t* x, const int64_t* topk_idx, int32_t use_fp8,
                             int32_t round_scale, int32_t use_ue8m0, void* msg_buf, int32_t* msg_count,
                             void* packed_recv_x, float* packed_recv_x_scales, uint8_t* packed_recv_x_scales_ue8m0,
                             int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                             int32_t* packed_recv_count, int32_t* cumulative_local_expert_recv_stats,
                             const int32_t* mask_buffer, void* stream) {
  miep::LLArgs a;
  miep_status st = ll_dispatch_args(q, x, topk_idx, use_fp8, round_scale, use_ue8m0, msg_buf, msg_count,
                                    packed_recv_x, packed_recv_x_scales, packed_recv_x_scales_ue8m0,
                                    packed_recv_src_info, packed_recv_layout_range, packed_recv_count,
                                    cumulative_local_expert_recv_stats, mask_buffer, true, &a);
  if (st != MIEP_OK) return st;
  return hip_status(miep::launch_ll(a, static_cast<hipStream_t>(stream)), "low-latency launch");
}

miep_status miep_ll_dispatch_noalloc(const miep_ll_problem* q, const uint16_t* x, const int64_t* topk_idx,
                                     int32_t use_fp8, int32_t round_scale, int32_t use_ue8m0, void* packed_recv_x,
                                     float* packed_recv_x_scales, uint8_t* packed_recv_x_scales_ue8m0,
                                     int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                                     int32_t* packed_recv_count, int32_t* cumulative_local_expert_recv_stats,
                                     const int32_t* mask_buffer, void* stream) {
  miep::LLArgs a;
  miep_status st = ll_dispatch_args(q, x, topk_idx, use_fp8, round_scale, use_ue8m0, nullptr, nullptr,
                                    packed_recv_x, packed_recv_x_scales, packed_recv_x_scales_ue8m0,
                                    packed_recv_src_info, packed_recv_layout_range, packed_recv_count,
                                    cumulative_local_expert_recv_stats, mask_buffer, false, &a);
  if (st != MIEP_OK) return st;
  if (static_cast<int64_t>(a.L) * a.R > miep::kLLScratchCounts)
    return fail(MIEP_EUNSUPPORTED, "the allocation-free low-latency dispatch holds at most %d (local expert, source) "
                "counts; this problem needs %lld (num_experts)", miep::kLLScratchCounts,
                static_cast<long long>(a.L) * a.R);
  int32_t* counts = nullptr;
  hipError_t e = miep::ll_scratch_counts(&counts);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  a.msg = nullptr;
  a.msg_count = counts;
  return hip_status(miep::launch_ll(a, static_cast<hipStream_t>(stream)), "low-latency launch");
}

miep_status miep_ll_combine(const miep_ll_problem* q, const uint16_t* y, const int32_t* packed_recv_src_info,
                            const int64_t* packed_recv_layout_range, const int64_t* topk_idx,
                            const float* topk_weights, uint16_t* combined_x, void* stream) {
  miep_status st = check_ll_problem(q);
  if (st != MIEP_OK) return st;
  if (!y || !packed_recv_src_info || !packed_recv_layout_range || (q->num_tokens > 0 && (!topk_idx || !combined_x)))
    return fail(MIEP_EINVAL, "a required pointer is NULL");
  if (!aligned16(y) || !aligned16(combined_x)) return fail(MIEP_EUNSUPPORTED, "y and combined_x must be 16-byte aligned");
  miep::LLCombineArgs a{};
  a.R = q->num_ranks;
  a.T = q->num_tokens;
  a.M = q->max_tokens;
  a.H = q->hidden;
  a.K = q->num_topk;
  a.E = q->num_experts;
  a.L = q->num_experts / q->num_ranks;
  a.d = q->dest_rank;
  a.y = y;
  a.src_info = packed_recv_src_info;
  a.layout_range = packed_recv_layout_range;
  a.topk_idx = topk_idx;
  a.w = topk_weights;
  a.out = combined_x;
  return hip_status(miep::launch_ll_combine(a, static_cast<hipStream_t>(stream)), "low-latency combine launch");
}

miep_status miep_mask_update(int32_t* mask_buffer, int32_t num_ranks, int32_t rank, int32_t value, void* stream) {
  if (!mask_buffer || num_ranks <= 0) return fail(MIEP_EINVAL, "mask_buffer is NULL or num_ranks <= 0");
  if (rank < 0 || rank >= num_ranks) return fail(MIEP_EINVAL, "rank out of range");
  return hip_status(miep::launch_mask_set(mask_buffer, rank, value, static_cast<hipStream_t>(stream)), "mask launch");
}

miep_status miep_mask_clean(int32_t* mask_buffer, int32_t num_ranks, void* stream) {
  if (!mask_buffer || num_ranks <= 0) return fail(MIEP_EINVAL, "mask_buffer is NULL or num_ranks <= 0");
  return hip_status(miep::launch_fill_zero(mask_buffer, num_ranks, static_cast<hipStream_t>(stream)), "mask launch");
}

miep_status miep_mask_query(const int32_t* mask_buffer, int32_t num_ranks, int32_t* out, void* stream) {
  if (!mask_buffer || !out || num_ranks <= 0) return fail(MIEP_EINVAL, "a pointer is NULL or num_ranks <= 0");
  return hip_status(miep::launch_copy_i32(mask_buffer, out, num_ranks, static_cast<hipStream_t>(stream)), "mask launch");
}

}  // extern "C"
