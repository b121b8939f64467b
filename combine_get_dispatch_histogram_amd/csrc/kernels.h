// kernels.h -- internal launch interface between the C ABI (api.cpp) and the
// gfx950 kernels.  Host code only sees these argument structs and launchers;
// every launcher enqueues on the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miep {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kFp8Group = 128;     // channels per FP8 scale
constexpr int kMaxRanks = 256;     // logical ranks supported by one call
constexpr int kMaxExperts = 8192;  // experts (LDS histogram bound)

// ---- layout histogram (one workgroup per source partition)
struct LayoutArgs {
  int S, T, K, E, R, L;
  const int64_t* topk_idx;  // [S*T][K]
  int32_t* ntpr;            // [S][R]
  int32_t* ntp_rdma;        // [S][R/8] or null
  int32_t* ntpe;            // [S][E]
  uint8_t* in_rank;         // [S*T][R]
};
hipError_t launch_layout(const LayoutArgs& a, hipStream_t st);

// ---- notify: prefix matrices, receive offsets, send_head (one workgroup per source)
struct NotifyArgs {
  int S, T, R, C, E, L, align;
  const uint8_t* in_rank;   // [S*T][R]
  const int32_t* ntpr;      // [S][R]
  const int32_t* ntpe;      // [S][E] or null
  int32_t* rpm;             // [S][R]
  int32_t* cpm;             // [S][R][C]
  int32_t* rcpm;            // [R][S][C]
  int32_t* off;             // [R+1]
  int32_t* send_head;       // [S*T][R]
  int32_t* nrte;            // [R][L] or null
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
  int64_t* recv_topk_idx;
  float* recv_topk_weights;
  int32_t* recv_src_idx;
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
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// ---- low-latency: expert-major send, then receive-side unpack
struct LLArgs {
  int R, T, M, H, K, E, L, d;
  int use_fp8, round_scale, use_ue8m0;
  int64_t msg_bytes;
  const uint16_t* x;
  const int64_t* topk_idx;
  uint8_t* msg;
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
// MIEP_LL_VPL, MIEP_CAST_TPB, MIEP_LLC_VPL, MIEP_LLC_SLICES): used by
// geometry sweeps, never required.
// combine_maxr: source rows whose loads are issued together.
// pack_nt: bit 0 = non-temporal payload loads, bit 1 = non-temporal stores;
// combine_nt: bit 0 = non-temporal loads of the expert outputs, bit 1 =
// non-temporal stores of the combined rows.  ll_split: workgroups per
// low-latency (expert, source) block.  cast_tpb: fused FP8 cast with one
// token per workgroup (1), 1 KiB slices (0), or chosen per call (-1).
// llc_vpl / llc_slices: low-latency combine vectors per lane and slices per
// token.
struct Tuning {
  int pack_vpl, pack_slices, combine_vpl, combine_slices, combine_maxr, pack_nt, combine_nt, ll_split, ll_vpl,
      cast_tpb, llc_vpl, llc_slices;
};
const Tuning& tuning();

}  // namespace miep
