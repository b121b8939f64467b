// kernels.h -- internal launch interface between the C ABI (api.cpp) and the
// gfx950 kernels.  Host code only sees these argument structs and launchers;
// every launcher enqueues on the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miep {

constexpr int kWave = 64;          // CDNA wavefront width
// A grid dimension counts its work-items in 32 bits: the largest number of
// workgroups of `threads` threads one 1-D launch may ask for.  Launches past
// it return hipErrorInvalidConfiguration instead of a truncated grid.
constexpr int64_t max_blocks(int64_t threads) { return ((int64_t(1) << 32) - 1) / threads; }
constexpr int kFp8Group = 128;     // channels per FP8 scale
constexpr int kMaxRanks = 256;     // logical ranks supported by one call
constexpr int kMaxExperts = 8192;  // experts (LDS histogram bound)
constexpr int kStatusCapacity = 4; // device status word value of MIEP_ECAPACITY

// Division by a launch constant without the ~30-instruction integer divide:
// floor(n / d) = (n * m) >> 40 with m = ceil(2^40 / d).  Writing m = (2^40 +
// e) / d with 0 <= e < d, the product overshoots n/d by n*e / (d * 2^40) <
// n / 2^40, which stays below the 1/d gap to the next integer whenever
// n * d < 2^40.  Uses: expert / experts-per-rank (both <= 8192, always
// exact) and token / tokens-per-channel (exact for T <= 2^20, which the
// kernels check before taking it).
struct FastDiv {
  uint64_t m;
  int d;
};
inline FastDiv make_fastdiv(int d) {
  FastDiv f;
  f.d = d > 0 ? d : 1;
  f.m = ((1ull << 40) + static_cast<uint64_t>(f.d) - 1) / static_cast<uint64_t>(f.d);
  return f;
}

// ---- layout histogram (one workgroup per source partition)
struct LayoutArgs {
  int S, T, K, E, R, L;
  FastDiv Ldiv;             // experts per rank
  const int64_t* topk_idx;  // [S*T][K]
  int32_t* ntpr;            // [S][R]
  int32_t* ntp_rdma;        // [S][R/8] or null
  int32_t* ntpe;            // [S][E]
  uint8_t* in_rank;         // [S*T][R]
};
hipError_t launch_layout(const LayoutArgs& a, hipStream_t st);

// ---- notify: prefix matrices, receive offsets, send_head (one workgroup per
// group of channels of a source, or per source where that kernel's conditions
// do not hold)
// group_w == 0: the destinations are the R ranks of in_rank's rows.
// group_w == 8: the destinations are R groups of 8 ranks (rows of R*8
// bytes); a token goes to a group when it goes to any of its ranks.
struct NotifyArgs {
  int S, T, R, C, E, L, align;
  int group_w;
  FastDiv tcdiv;            // tokens per channel, ceil(T / C)
  int nonempty;             // channels holding tokens, ceil(T / tcdiv.d)
  const uint8_t* in_rank;   // [S*T][R] (or [S*T][R*group_w])
  const int32_t* ntpr;      // [S][R]
  const int32_t* ntpe;      // [S][E] or null
  int32_t* rpm;             // [S][R]
  int32_t* cpm;             // [S][R][C]
  int32_t* rcpm;            // [R][S][C]
  int32_t* off;             // [R+1]
  int32_t* send_head;       // [S*T][R]
  int32_t* nrte;            // [R][L] or null
  // Device status word (null: none): workgroup 0 writes kStatusCapacity when
  // the receive rows exceed `capacity`, else 0 -- or, with status_or, writes
  // only on an overflow (a second notify of the same call keeps the first's).
  int32_t* status = nullptr;
  int64_t capacity = 0;
  int status_or = 0;
};
hipError_t launch_notify(const NotifyArgs& a, hipStream_t st);
// Zero-fill of an int32 array by a kernel (no memset node in captured graphs).
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t st);

// ---- pack: send_head-driven copy of every token to each receiving rank
enum PackKind { kPackBf16 = 0, kPackFp8 = 1, kPackCastFp8 = 2 };
struct PackArgs {
  int64_t N;      // tokens
  int T, H, K, E, L, R;
  int kind;       // PackKind
  int round_scale;
  int meta;       // write recv_src_idx / recv_topk_* (fresh dispatch)
  int64_t capacity;
  const void* x;
  const float* x_scales;
  const int64_t* topk_idx;
  const float* topk_weights;
  const int32_t* send_head;
  const int32_t* off;
  void* recv_x;
  float* recv_x_scales;
  uint8_t* recv_ue = nullptr;  // [cap][H/128] exponent bytes of power-of-two scales (fused cast), or null
  int64_t* recv_topk_idx;
  float* recv_topk_weights;
  int32_t* recv_src_idx;
  // Forwarding from group rows (all null / 0 for a direct dispatch):
  const int32_t* count;      // device row count; rows n >= *count are skipped
  const int32_t* group_off;  // [groups+1] first row of each group; lane j of row n's group g is rank g*group_w + j
  int groups, group_w;
  const int32_t* src_tok;    // [N] source token of row n (top-k metadata, recv_src_idx)
  int cpol = -1;             // cache-policy code of this launch (-1: the default)
  // Receive records of a fresh direct dispatch in their own wavefronts (one
  // per (source, rank)): needs the rank prefix matrix and the membership.
  int S = 0;
  const int32_t* rpm = nullptr;       // [S][R] inclusive rows per rank from sources 0..s
  const uint8_t* in_rank = nullptr;   // [S*T][R]
  int rec_waves = 0, rec_blocks = 0;  // set by launch_pack
  int rec_parts = 1;                  // record wavefronts per (source, rank), each taking every rec_parts-th part
  int rec_last = 0;                   // record workgroups at the end of the grid instead of the front
};
hipError_t launch_pack(const PackArgs& a, hipStream_t st);

// ---- combine: send_head-driven gather and fp32 sum back to token order
struct CombineArgs {
  int64_t N;
  int H, K, R;
  int64_t capacity;
  const uint16_t* y;
  const float* w;            // [cap][K] or null
  const uint16_t* bias0;     // [N][H] or null
  const uint16_t* bias1;     // [N][H] or null
  const int32_t* send_head;
  const int32_t* off;
  uint16_t* out;             // [N][H]
  float* out_w;              // [N][K] or null
  // Group-level reduction (all null / 0 for a direct combine): rows n >=
  // *count are skipped; lane j of row n's group g reads rank g*group_w + j.
  const int32_t* count;
  const int32_t* group_off;  // [groups+1]
  int groups, group_w;
  int cpol = -1;             // cache-policy code of this launch (-1: the default)
  // Row element types (the two-level combine's fp32 partials): y is fp32
  // [cap][H] when in_f32, out is fp32 [N][H] when out_f32 (no rounding).
  int in_f32 = 0, out_f32 = 0;
  int bias_nt = 0;           // bias rows loaded non-temporally (set by launch_combine)
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// ---- relay: per group row, its source token and its rows in the group's ranks
struct RelayMetaArgs {
  int64_t N;                  // source tokens
  int G, R;                   // groups of 8, ranks
  int64_t rdma_capacity;
  const int32_t* send_rdma_head;  // [N][G]
  const int32_t* rdma_off;        // [G+1]
  const int32_t* send_head;       // [N][R]
  int32_t* rdma_src_idx;          // [rdma_capacity]
  int32_t* send_nvl_head;         // [rdma_capacity][8]
};
hipError_t launch_relay_meta(const RelayMetaArgs& a, hipStream_t st);

// ---- low-latency: per-block message counts, then messages and packed rows in one pass
struct LLArgs {
  int R, T, M, H, K, E, L, d;
  int use_fp8, round_scale, use_ue8m0;
  int64_t msg_bytes;
  const uint16_t* x;
  const int64_t* topk_idx;
  uint8_t* msg;              // [L][R][M] messages, or null: not materialised
  int32_t* msg_count;        // [L][R]
  void* prx;                 // [L][R*M][H] codes or bf16
  float* prs;                // [L][R*M][H/128]
  uint8_t* prue;             // [L][R*M][H/128] or null
  int32_t* src_info;         // [L][R*M]
  int64_t* layout_range;     // [L][R]
  int32_t* count;            // [L]
  int32_t* cumulative;       // [L] or null
  const int32_t* mask;       // [R] nonzero = masked rank, or null
};
hipError_t launch_ll(const LLArgs& a, hipStream_t st);
// The allocation-free variant's count buffer: a file-scope device array of
// kLLScratchCounts int32 (one copy per device); its device address for the
// current device, looked up once per device.
constexpr int kLLScratchCounts = 65536;
constexpr int kMaxDevices = 64;
hipError_t ll_scratch_counts(int32_t** out);

// ---- low-latency combine: rank d's expert outputs back to source-token order
struct LLCombineArgs {
  int R, T, M, H, K, E, L, d;
  const uint16_t* y;             // [L][R*M][H]
  const int32_t* src_info;       // [L][R*M]
  const int64_t* layout_range;   // [L][R]
  const int64_t* topk_idx;       // [R*T][K]
  const float* w;                // [R*T][K] or null
  uint16_t* out;                 // [R*T][H]
};
hipError_t launch_ll_combine(const LLCombineArgs& a, hipStream_t st);

// ---- rank mask helpers: set one entry (launch_mask_set), clear all
// (launch_fill_zero), copy out (launch_copy_i32); tiny kernels
hipError_t launch_mask_set(int32_t* mask, int rank, int value, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t st);

// Optional launch-geometry overrides read once from the environment
// (MIEP_PACK_VPL, MIEP_PACK_SLICES, MIEP_COMBINE_VPL, MIEP_COMBINE_SLICES,
// MIEP_COMBINE_MAXR, MIEP_PACK_NT, MIEP_COMBINE_NT, MIEP_LL_SPLIT,
// MIEP_LL_VPL, MIEP_CAST_TPB, MIEP_LLC_VPL, MIEP_LLC_SLICES, MIEP_LLC_NT,
// MIEP_LL_NT, MIEP_PACK_RECORDS, MIEP_LL_TPB, MIEP_LL_COUNT_SRC,
// MIEP_NOTIFY_CHAN, MIEP_BIAS_NT):
// used by geometry sweeps, never required.
// combine_maxr: source rows whose loads are issued together.
// pack_nt / combine_nt: cache policy of the row traffic, bit 0 =
// non-temporal loads, bit 1 = non-temporal stores, bit 2 = device-scope
// (sc1) stores; -1 (unset) leaves it to the launch.  Defaults, measured on
// MI355X: over the whole normal step (layout, dispatch, combine back to
// back) pack 6 (plain loads of x, non-temporal device-scope stores) and
// combine 5 (non-temporal loads of the expert outputs, device-scope
// stores); setting both or neither of the non-temporal bits costs ~20% in
// either kernel.  The relay's forwarding pack and group-level combine take 7
// (its group rows are written once and read once more right after); its
// first hop and token-level combine keep the direct path's 6 and 5.  ll_split: workgroups per
// low-latency (expert, source) block.  cast_tpb: fused FP8 cast with one
// token per workgroup (1), or 1 KiB slices (0 or -1, the default).
// llc_vpl / llc_slices / llc_nt: low-latency combine vectors per lane,
// slices per token and cache-policy code (as pack_nt); ll_nt: the
// low-latency send's cache-policy code.  pack_records: 0 writes a fresh
// dispatch's receive records from the payload wavefronts instead of the
// record wavefronts (-1, the default: record wavefronts where supported).
// ll_tpb: threads per low-latency send workgroup (256, 512 or 1024; 0 =
// chosen per call); ll_count_src: 0 counts messages with one workgroup per
// (l, s) block instead of one per source (-1, the default).  notify_chan: 0
// runs the per-source notify everywhere, n > 0 caps the channels per
// workgroup of the channel-group notify (-1, the default: as many whole
// channels as fit in one wavefront, where supported).  bias_nt: 1 loads the
// combine's bias rows non-temporally, 0 with the default policy (-1, the
// default: non-temporally when a bias is larger than half the 256 MiB
// last-level cache, which it then could not hold anyway).
struct Tuning {
  int pack_vpl, pack_slices, combine_vpl, combine_slices, combine_maxr, pack_nt, combine_nt, ll_split, ll_vpl,
      cast_tpb, llc_vpl, llc_slices, llc_nt, ll_nt, pack_records, ll_tpb, ll_count_src, notify_chan, bias_nt;
};
const Tuning& tuning();

}  // namespace miep
