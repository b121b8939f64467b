// ll.hip -- low-latency dispatch on one GPU, seen from one receiving rank.
//
// "DeepEP Normal vs Low-Latency dual-mode analysis", low-latency dispatch:
// each token is cast (optionally to FP8 with per-128-channel scales) and
// one message per top-k expert entry >= 0 goes straight to the rank owning
// that expert; the receiver keeps messages expert-major, at slot
// (local_expert, src_rank, i), and packs local expert l's rows from row
// l * R * M.  "Normal vs Low-Latency: two communication philosophies in
// DeepEP V1 / V2 / DeepGEMM": a message is one 16-byte header (the source
// token index plus three reserved ints) and the payload (H E4M3 bytes and
// H/128 fp32 scales, or 2H bf16 bytes).  "Chapter 4  V1: layout, dispatch
// and combine", section 4.3: the call returns the packed rows, scales,
// per-expert counts, source info and layout range.
//
// Where the transport fills slots in atomic arrival order, these kernels
// fix the order: slot j of (l, s) is the j-th top-k entry of source s that
// names expert d*L + l, in (token, k) order, so the output is
// deterministic.  Two kernels:
//   count: one workgroup per source s counts, for each of d's local
//          experts, the top-k entries naming it (an LDS histogram), and
//          writes the (l, s) message counts;
//   send:  a few workgroups per (l, s) block (kLLSplit of 256 threads; 3 of
//          512 threads for wide FP8 rows) repeat the (tiny) slot scan, take
//          the block's packed range from the counts of the earlier sources,
//          and cast and write each message and its packed row in one pass
//          (16-byte loads and stores), so nothing is read back.
#include <mutex>

#include "device.h"
#include "kernels.h"

namespace miep {

// Scratch of the allocation-free low-latency dispatch: the per-(local
// expert, source) message counts that the count kernel hands to the send
// kernel, for callers that pass no message buffer.  One copy per device,
// held until the process ends; every call on a device overwrites all L*R
// counts it uses before reading them, so nothing needs clearing.
static __device__ __align__(256) int32_t scratch[kLLScratchCounts];

hipError_t ll_scratch_counts(int32_t** out) {
  // the array's name is a host-side stand-in: its device address comes from
  // the runtime, once per device, with that device current
  static std::mutex mu;
  static int32_t* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

constexpr int kLLThreads = 256;
constexpr int kLLSplit = 8;  // default workgroups sharing one (l, s) block's messages
constexpr int kLLMaxSlots = 4096;

// The slot scan of block (l, s): every top-k entry of source s that names
// expert d*L + l, in (token, k) order, takes the next slot.  Thread t of the
// workgroup handles token t (8 entries loaded at a time); a wavefront scan
// plus an LDS carry across wavefronts and 256-token chunks gives each entry
// its slot.  With `slot_tok`, slot j < M records its token.  Returns the
// number of matching entries (uncapped), the same in every thread.
template <int TPB>
__device__ __forceinline__ int ll_slot_scan(const LLArgs& a, int l, int s, int32_t* slot_tok, int32_t* wsum,
                                            int32_t* carry_s) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int64_t target = static_cast<int64_t>(a.d) * a.L + l;
  const int64_t* idx = a.topk_idx + static_cast<int64_t>(s) * a.T * a.K;
  // a masked destination is not sent to, a masked source is not received from
  const bool masked = a.mask != nullptr && (a.mask[a.d] != 0 || a.mask[s] != 0);
  if (a.T <= TPB) {
    // one chunk: every thread sums the wavefront totals itself (two
    // barriers: the totals, then the slot list)
    const int t = tid;
    uint64_t kmask = 0;
    if (t < a.T && !masked) {
      const int64_t* row = idx + static_cast<int64_t>(t) * a.K;
      for (int k0 = 0; k0 < a.K; k0 += 8) {
        int64_t e8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e8[j] = k0 + j < a.K ? row[k0 + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) kmask |= static_cast<uint64_t>(e8[j] == target) << (k0 + j);
      }
    }
    const int cnt = __popcll(kmask);
    const int inc = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int tot = 0, before = 0;
#pragma unroll
    for (int q = 0; q < TPB / kWave; ++q) {
      const int v = wsum[q];
      tot += v;
      before += q < w ? v : 0;
    }
    if (slot_tok != nullptr) {
      int j = before + inc - cnt;
      for (uint64_t km = kmask; km != 0; km &= km - 1) {
        if (j < a.M) slot_tok[j] = t;
        ++j;
      }
    }
    __syncthreads();
    return tot;
  }
  // the carry is first read after the first barrier of the loop, so its
  // reset needs no barrier of its own (the top-k loads go out at once)
  if (tid == 0) *carry_s = 0;
  for (int t0 = 0; t0 < a.T; t0 += TPB) {
    const int t = t0 + tid;
    uint64_t kmask = 0;                           // entries k of token t that name the expert
    if (t < a.T && !masked) {
      const int64_t* row = idx + static_cast<int64_t>(t) * a.K;
      for (int k0 = 0; k0 < a.K; k0 += 8) {       // 8 independent loads in flight
        int64_t e8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e8[j] = k0 + j < a.K ? row[k0 + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) kmask |= static_cast<uint64_t>(e8[j] == target) << (k0 + j);
      }
    }
    const int cnt = __popcll(kmask);
    const int inc = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    if (slot_tok != nullptr) {
      int j = *carry_s + inc - cnt;
      for (int q = 0; q < w; ++q) j += wsum[q];
      for (uint64_t km = kmask; km != 0; km &= km - 1) {   // one slot per matching entry, k ascending
        if (j < a.M) slot_tok[j] = t;
        ++j;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int tot = *carry_s;
      for (int q = 0; q < TPB / kWave; ++q) tot += wsum[q];
      *carry_s = tot;
    }
    __syncthreads();
  }
  return a.T > 0 ? *carry_s : 0;
}

// Per-(l, s) message counts, capped at M (one workgroup per block).
__global__ __launch_bounds__(kLLThreads) void ll_count_kernel(LLArgs a) {
  __shared__ int32_t wsum[kLLThreads / kWave];
  __shared__ int32_t carry_s;
  const int l = blockIdx.x / a.R;
  const int s = blockIdx.x % a.R;
  const int n = ll_slot_scan<kLLThreads>(a, l, s, nullptr, wsum, &carry_s);
  if (threadIdx.x == 0) a.msg_count[l * a.R + s] = n < a.M ? n : a.M;
}

// Per-(l, s) message counts, capped at M, one workgroup per source s: every
// thread takes tokens t, t + blockDim, ... and counts, in an LDS histogram
// over d's L local experts, the top-k entries naming each of them (a
// source's top-k rows are read once instead of once per local expert).
__global__ __launch_bounds__(kLLThreads) void ll_count_src_kernel(LLArgs a) {
  extern __shared__ int32_t hist[];               // [L]
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  for (int l = tid; l < a.L; l += blockDim.x) hist[l] = 0;
  const bool masked = a.mask != nullptr && (a.mask[a.d] != 0 || a.mask[s] != 0);
  const int64_t lo = static_cast<int64_t>(a.d) * a.L;
  __syncthreads();
  if (!masked) {
    const int64_t* idx = a.topk_idx + static_cast<int64_t>(s) * a.T * a.K;
    for (int t = tid; t < a.T; t += blockDim.x) {
      const int64_t* row = idx + static_cast<int64_t>(t) * a.K;
      for (int k0 = 0; k0 < a.K; k0 += 8) {       // 8 independent loads in flight
        int64_t e8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e8[j] = k0 + j < a.K ? row[k0 + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (e8[j] >= lo && e8[j] < lo + a.L) atomicAdd(&hist[e8[j] - lo], 1);
      }
    }
  }
  __syncthreads();
  for (int l = tid; l < a.L; l += blockDim.x) {
    const int n = hist[l];
    a.msg_count[l * a.R + s] = n < a.M ? n : a.M;
  }
}

// Messages and their packed receive rows.  Workgroup (l, s, y) repeats the
// slot scan, takes block (l, s)'s first packed row from the counts of the
// earlier sources, and serves every kLLSplit-th (message, slice) task: the
// slice is loaded once (16-byte loads), cast, and written both to the
// message (the transport buffer) and to the packed row, so the receive side
// never reads the messages back.  Without a message buffer (a.msg null)
// only the packed rows are written.
template <int VPL, int NT, int TPB>
__global__ __launch_bounds__(TPB) void ll_send_kernel(LLArgs a) {
  __shared__ int32_t slot_tok[kLLMaxSlots];  // message j -> source token
  __shared__ int32_t wsum[TPB / kWave];
  __shared__ int32_t carry_s;
  const int l = blockIdx.x / a.R;
  const int s = blockIdx.x % a.R;
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: row bases stay scalar
  // first packed row of the block: messages of the earlier sources for
  // expert l, summed by every wavefront; the first 64 counts are loaded
  // unconditionally (clamped index) so that they are in flight with the
  // scan's top-k loads, and masked only after the scan
  const int p_raw = a.msg_count[l * a.R + (lane < a.R ? lane : a.R - 1)];
  const int cnt = ll_slot_scan<TPB>(a, l, s, slot_tok, wsum, &carry_s);   // synchronises the workgroup
  const int n = cnt < a.M ? cnt : a.M;
  int part = lane < s ? p_raw : 0;
  for (int q = lane + kWave; q < s; q += kWave) part += a.msg_count[l * a.R + q];
  const int begin = readlane(wave_inclusive_scan(part), kWave - 1);
  if (tid == 0 && blockIdx.y == 0) {             // once per (l, s), not per split workgroup
    a.layout_range[l * a.R + s] = (static_cast<int64_t>(begin) << 32) | static_cast<int64_t>(static_cast<uint32_t>(n));
    if (s == a.R - 1) {
      a.count[l] = begin + n;
      if (a.cumulative) a.cumulative[l] += begin + n;
    }
  }

  // one wavefront per (message, row slice).  A lane's unit is one 16-byte
  // vector of 8 bf16, or with FP8 a pair of them (16 channels -> 16 codes in
  // one 16-byte store; a 128-channel group is 8 lanes).
  const int nv = a.H / 8;
  const int units = a.use_fp8 ? nv / 2 : nv;
  const int span = kWave * VPL;
  const int nsl = (units + span - 1) / span;
  const int G = a.H / kFp8Group;
  const int64_t pb = a.use_fp8 ? a.H : 2 * static_cast<int64_t>(a.H);   // packed row bytes
  const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(a.x) + static_cast<int64_t>(s) * a.T * 2 * a.H;
  const bool keep = a.msg != nullptr;                       // messages materialised
  for (int task = blockIdx.y * (TPB / kWave) + w; task < n * nsl; task += gridDim.y * (TPB / kWave)) {
    const int j = task / nsl;
    const int u0 = (task - j * nsl) * span;
    const int t = slot_tok[j];
    uint8_t* msg = keep ? a.msg + ((static_cast<int64_t>(l) * a.R + s) * a.M + j) * a.msg_bytes : nullptr;
    const int64_t row = static_cast<int64_t>(l) * a.R * a.M + begin + j;
    uint8_t* prow = static_cast<uint8_t*>(a.prx) + row * pb;
    if (u0 == 0 && lane == 0) {
      if (keep) *reinterpret_cast<int4*>(msg) = make_int4(t, 0, 0, 0);
      a.src_info[row] = t;
    }
    const uint8_t* xrow = xsrc + static_cast<int64_t>(t) * 2 * a.H;
    if (a.use_fp8) {
      v4u d[VPL][2];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int p = u0 + i * kWave + lane;
        if (p < units) {
          d[i][0] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(p) * 32);
          d[i][1] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(p) * 32 + 16);
        }
      }
      float* scales = keep ? reinterpret_cast<float*>(msg + 16 + a.H) : nullptr;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int p = u0 + i * kWave + lane;
        const float amax = group8_max(p < units ? fmaxf(absmax8(d[i][0]), absmax8(d[i][1])) : 0.0f);
        float sci;
        const float sc = fp8_scales(amax, a.round_scale != 0, &sci);
        if (p < units) {
          const v4u q = cast16(d[i][0], d[i][1], sc);
          if (keep) stb16<store_cpol(NT)>(msg, 16 + static_cast<uint32_t>(p) * 16, q);
          stb16<store_cpol(NT)>(prow, static_cast<uint32_t>(p) * 16, q);
          if ((lane & 7) == 0) {
            if (keep) scales[p / 8] = sci;
            a.prs[row * G + p / 8] = sci;
            if (a.prue) a.prue[row * G + p / 8] = static_cast<uint8_t>((__float_as_uint(sci) >> 23) & 0xFFu);
          }
        }
      }
    } else {
      v4u d[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int v = u0 + i * kWave + lane;
        if (v < nv) d[i] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(v) * 16);
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int v = u0 + i * kWave + lane;
        if (v < nv) {
          if (keep) stb16<store_cpol(NT)>(msg, 16 + static_cast<uint32_t>(v) * 16, d[i]);
          stb16<store_cpol(NT)>(prow, static_cast<uint32_t>(v) * 16, d[i]);
        }
      }
    }
  }
}

// count: one workgroup per source (an LDS histogram over the L local
// experts; measured on the low-latency workload 12.55 -> 12.15 us for count +
// send) when L fits in LDS, else one per (l, s) block.  send: tpb threads
// per workgroup (512 with 3 workgroups per block for wide FP8 rows: 11.95 us).
template <int VPL, int NT>
static hipError_t launch_ll_cfg(const LLArgs& a, int blocks, int split, int tpb, hipStream_t st) {
  if (tuning().ll_count_src != 0 && a.L <= 16384)
    hipLaunchKernelGGL(ll_count_src_kernel, dim3(a.R), dim3(kLLThreads), sizeof(int32_t) * a.L, st, a);
  else
    hipLaunchKernelGGL(ll_count_kernel, dim3(blocks), dim3(kLLThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (tpb) {
    case 512: hipLaunchKernelGGL((ll_send_kernel<VPL, NT, 512>), dim3(blocks, split), dim3(512), 0, st, a); break;
    case 1024: hipLaunchKernelGGL((ll_send_kernel<VPL, NT, 1024>), dim3(blocks, split), dim3(1024), 0, st, a); break;
    default: hipLaunchKernelGGL((ll_send_kernel<VPL, NT, kLLThreads>), dim3(blocks, split), dim3(kLLThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <int VPL>
static hipError_t launch_ll_vpl(const LLArgs& a, int blocks, int split, int tpb, hipStream_t st) {
  // cache policy: plain loads of x, non-temporal stores of the messages and
  // packed rows (measured on the low-latency workload: 12.95 us against
  // 13.5 us with the plain policy)
  switch (tuning().ll_nt >= 0 ? tuning().ll_nt & 7 : 2) {
    case 1: return launch_ll_cfg<VPL, 1>(a, blocks, split, tpb, st);
    case 2: return launch_ll_cfg<VPL, 2>(a, blocks, split, tpb, st);
    case 3: return launch_ll_cfg<VPL, 3>(a, blocks, split, tpb, st);
    case 4: return launch_ll_cfg<VPL, 4>(a, blocks, split, tpb, st);
    case 5: return launch_ll_cfg<VPL, 5>(a, blocks, split, tpb, st);
    case 6: return launch_ll_cfg<VPL, 6>(a, blocks, split, tpb, st);
    case 7: return launch_ll_cfg<VPL, 7>(a, blocks, split, tpb, st);
    default: return launch_ll_cfg<VPL, 0>(a, blocks, split, tpb, st);
  }
}

hipError_t launch_ll(const LLArgs& a, hipStream_t st) {
  const int blocks = a.L * a.R;
  if (blocks == 0) return hipSuccess;
  const Tuning& tu = tuning();
  // bf16: two 16-byte vectors per lane per task when a row is a multiple of
  // 128 vectors, 8 workgroups per (l, s) block (measured best).  FP8: rows of
  // at least 128 pairs of vectors take two pairs (32 channels) per lane with
  // 6 workgroups per block (the last slice of a row may be partial; measured
  // on the low-latency workload: 12.6 us against 13.0 us with one pair and 8
  // workgroups, which fill every wavefront slot of the chip exactly), shorter
  // rows one pair when a row is 64 pairs' multiple
  const bool fp8_wide = a.use_fp8 && a.H / 16 >= 2 * kWave;
  const int tpb = tu.ll_tpb > 0 ? tu.ll_tpb : (fp8_wide ? 512 : kLLThreads);
  const int split = tu.ll_split > 0 ? tu.ll_split : (fp8_wide ? (tpb == 512 ? 3 : 6) : kLLSplit);
  int vpl;
  if (tu.ll_vpl > 0)
    vpl = tu.ll_vpl;
  else if (a.use_fp8)
    vpl = fp8_wide ? 2 : ((a.H / 16) % kWave == 0 ? 1 : 8);
  else
    vpl = (a.H / 8) % (2 * kWave) == 0 ? 2 : 8;
  switch (vpl) {
    case 1: return launch_ll_vpl<1>(a, blocks, split, tpb, st);
    case 2: return launch_ll_vpl<2>(a, blocks, split, tpb, st);
    case 4: return launch_ll_vpl<4>(a, blocks, split, tpb, st);
    default: return launch_ll_vpl<8>(a, blocks, split, tpb, st);
  }
}

// ---------------------------------------------------------------------------
// Low-latency combine, the reverse of the dispatch above seen from rank d:
// every source token (s, t) gets back the rows of d's experts that its top-k
// entries were sent to, summed in fp32 in ascending k (each row times the
// entry's gate weight when weights are given) and rounded once to bf16.
//
// One wavefront per (group of P = 64 / K tokens, row slice); lane p*K + k
// holds entry k of the group's token p, so one load brings in the routing
// of P tokens.  Most tokens have no entry on rank d: their zero rows are
// stored once the entries' slots are found.  For an entry on local expert l the lane finds its slot in
// the (l, s) block from the dispatch's slot rule: the block's rows hold
// source tokens in (token, k) order, so the slot is the number of rows that
// name an earlier token (a binary search of the block's src_info) plus the
// number of the token's earlier entries for the same expert.  A slot at or
// past the block's count was dropped at the cap (or the rank was masked) and
// is skipped; so is a row whose src_info does not name the token (a handle
// from another routing).  The rows are then gathered in lane order, which is
// (token, k) order, MAXR rows' loads in flight, and each token's sum is
// stored when the walk moves past it.
// bf16 (round to nearest even) of one token's fp32 sums for the slice at v0
template <int VPL, int SP>
__device__ __forceinline__ void store_sum(uint8_t* orow, const float (&acc)[VPL][8], int v0, int nv, int lane) {
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int v = v0 + j * kWave + lane;
    if (v < nv) {
      v4u o;
      o.x = pack_bf16x2(acc[j][0], acc[j][1]);
      o.y = pack_bf16x2(acc[j][2], acc[j][3]);
      o.z = pack_bf16x2(acc[j][4], acc[j][5]);
      o.w = pack_bf16x2(acc[j][6], acc[j][7]);
      stb16<SP>(orow, static_cast<uint32_t>(v) * 16, o);
    }
  }
}

template <int VPL, int MAXR, int NT>
__global__ __launch_bounds__(256) void ll_combine_kernel(LLCombineArgs a, int nslices) {
  const int lane = lane_id();
  const int64_t gw = wave_index();
  const int K = a.K;
  const int P = kWave / K;                                 // tokens per group
  const int64_t N = static_cast<int64_t>(a.R) * a.T;
  const int64_t g = gw / nslices;
  const int slice = static_cast<int>(gw - g * nslices);
  const int64_t n0 = g * P;
  if (n0 >= N) return;
  const int np = N - n0 < P ? static_cast<int>(N - n0) : P;   // tokens in this group
  const int64_t lo = static_cast<int64_t>(a.d) * a.L;
  const int64_t block_rows = static_cast<int64_t>(a.R) * a.M;
  const uint64_t seg = K == kWave ? ~0ull : ((1ull << K) - 1);

  // routing of the group: lane p*K + k <- entry k of token n0 + p
  const int p = lane / K;
  const int k = lane - p * K;
  const bool mine = p < np;
  const int64_t n = n0 + p;
  int le = -1;                     // local expert of the entry, or -1
  float wk = 1.0f;                 // its gate weight
  if (mine) {
    const int64_t e = a.topk_idx[n * K + k];
    if (e >= lo && e < lo + a.L) le = static_cast<int>(e - lo);
    if (a.w) wk = a.w[n * K + k];
  }
  const uint64_t local = ballot(le >= 0);
  uint64_t tok_local = 0;          // tokens with an entry on rank d
  for (int q = 0; q < np; ++q)
    if ((local >> (q * K)) & seg) tok_local |= 1ull << q;

  const int nv = a.H / 8;
  const int64_t row_bytes = 2 * static_cast<int64_t>(a.H);
  uint8_t* out = reinterpret_cast<uint8_t*>(a.out);
  const int span = kWave * VPL;

  // zero rows of the tokens without an entry on rank d: at once when the
  // group has no other work, else after the slot search below, whose
  // dependent loads would otherwise queue behind these stores
  auto zero_rows = [&](uint64_t skip) {
    for (int v0 = slice * span; v0 < nv; v0 += nslices * span)
      for (int q = 0; q < np; ++q) {
        if ((skip >> q) & 1ull) continue;
        uint8_t* orow = out + (n0 + q) * row_bytes;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int v = v0 + j * kWave + lane;
          if (v < nv) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(v) * 16, v4u{0u, 0u, 0u, 0u});
        }
      }
  };
  if (tok_local == 0) {
    zero_rows(0);
    return;
  }

  // slot of every local entry: earlier entries of the token naming the same
  // expert, plus rows of the (l, s) block naming an earlier token
  int occ = 0;
  for (int j = 1; j < K; ++j) {
    const int other = __shfl(le, lane - j < 0 ? 0 : lane - j, kWave);
    occ += (j <= k && le >= 0 && other == le) ? 1 : 0;
  }
  int row = -1;                    // packed row of the entry, or -1
  if (le >= 0) {
    const int s = static_cast<int>(n / a.T);
    const int t = static_cast<int>(n - static_cast<int64_t>(s) * a.T);
    const int64_t lr = a.layout_range[static_cast<int64_t>(le) * a.R + s];
    const int64_t begin = lr >> 32;
    int64_t cnt = lr & 0xFFFFFFFFll;
    if (begin < 0 || begin + cnt > block_rows) cnt = 0;   // not a range the dispatch writes
    const int32_t* si = a.src_info + le * block_rows + begin;
    int64_t b = 0, e = cnt;                               // first row naming a token >= t
    while (b < e) {
      const int64_t mid = (b + e) >> 1;
      if (si[mid] < t) b = mid + 1; else e = mid;
    }
    const int64_t j = b + occ;
    if (j < cnt && si[j] == t) row = static_cast<int>(le * block_rows + begin + j);
  }
  zero_rows(tok_local);          // (measured: 12.56 -> 12.2 us on the low-latency workload)
  const uint64_t valid = ballot(row >= 0);
  uint64_t tok_valid = 0;
  for (int q = 0; q < np; ++q)
    if ((valid >> (q * K)) & seg) tok_valid |= 1ull << q;

  const uint8_t* y = reinterpret_cast<const uint8_t*>(a.y);
  const bool weighted = a.w != nullptr;
  for (int v0 = slice * span; v0 < nv; v0 += nslices * span) {
    // tokens whose every local entry was dropped combine to zero
    for (int q = 0; q < np; ++q) {
      if (((tok_local & ~tok_valid) >> q) & 1ull) {
        uint8_t* orow = out + (n0 + q) * row_bytes;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int v = v0 + j * kWave + lane;
          if (v < nv) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(v) * 16, v4u{0u, 0u, 0u, 0u});
        }
      }
    }
    float acc[VPL][8];
    int cur = -1;                  // token whose sum is in acc
    uint64_t m = valid;
    while (m) {
      int64_t rows[MAXR];
      float ws[MAXR];
      int tq[MAXR];
      int nb = 0;
#pragma unroll
      for (int q = 0; q < MAXR; ++q) {
        rows[q] = 0;
        ws[q] = 1.0f;
        tq[q] = 0;
        if (m) {
          const int bl = __builtin_ctzll(m);
          m &= m - 1;
          rows[q] = readlane(row, bl);
          ws[q] = __int_as_float(readlane(__float_as_int(wk), bl));
          tq[q] = bl / K;
          nb = q + 1;
        }
      }
      v4u dv[MAXR][VPL];
#pragma unroll
      for (int q = 0; q < MAXR; ++q) {
        if (q < nb) {
          const uint8_t* yrow = y + rows[q] * row_bytes;
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const int v = v0 + j * kWave + lane;
            if (v < nv) dv[q][j] = ldb16<load_cpol(NT)>(yrow, static_cast<uint32_t>(v) * 16);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < MAXR; ++q) {
        if (q < nb) {
          const bool first = tq[q] != cur;
          if (first && cur >= 0) store_sum<VPL, store_cpol(NT)>(out + (n0 + cur) * row_bytes, acc, v0, nv, lane);
          cur = tq[q];
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            float f[8] = {bf16_lo(dv[q][j].x), bf16_hi(dv[q][j].x), bf16_lo(dv[q][j].y), bf16_hi(dv[q][j].y),
                          bf16_lo(dv[q][j].z), bf16_hi(dv[q][j].z), bf16_lo(dv[q][j].w), bf16_hi(dv[q][j].w)};
            if (weighted) {
#pragma unroll
              for (int c = 0; c < 8; ++c) f[c] = f[c] * ws[q];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[j][c] = first ? f[c] : acc[j][c] + f[c];
          }
        }
      }
    }
    if (cur >= 0) store_sum<VPL, store_cpol(NT)>(out + (n0 + cur) * row_bytes, acc, v0, nv, lane);
  }
}

template <int VPL, int MAXR, int NT>
static hipError_t launch_ll_combine_cfg(const LLCombineArgs& a, int nslices, hipStream_t st) {
  const int P = kWave / a.K;
  const int64_t groups = (static_cast<int64_t>(a.R) * a.T + P - 1) / P;
  const int64_t blocks = (groups * nslices + 3) / 4;
  if (blocks > max_blocks(256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((ll_combine_kernel<VPL, MAXR, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                     nslices);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_ll_combine_nt(const LLCombineArgs& a, int vpl, int nslices, hipStream_t st) {
  switch (vpl) {
    case 2: return launch_ll_combine_cfg<2, 8, NT>(a, nslices, st);
    case 4: return launch_ll_combine_cfg<4, 4, NT>(a, nslices, st);
    default: return launch_ll_combine_cfg<1, 8, NT>(a, nslices, st);
  }
}

hipError_t launch_ll_combine(const LLCombineArgs& a, hipStream_t st) {
  if (static_cast<int64_t>(a.R) * a.T == 0) return hipSuccess;
  const Tuning& tu = tuning();
  const int nv = a.H / 8;
  // default: four 16-byte vectors per lane per token (4 KiB row pieces; the
  // last slice of a row may be partial) for rows of at least 256 vectors
  // (measured on the low-latency workload: 12.6-12.7 us against 13.3 us with
  // two, 14.5 us with one), else two when a row is a multiple of 128
  // vectors, else one
  const int vpl = tu.llc_vpl > 0 ? tu.llc_vpl : (nv >= 4 * kWave ? 4 : (nv % (2 * kWave) == 0 ? 2 : 1));
  const int span = vpl * kWave;
  int nslices = tu.llc_slices > 0 ? tu.llc_slices : (nv + span - 1) / span;
  if (nslices < 1) nslices = 1;
  // cache policy: plain loads, device-scope stores (measured on the
  // low-latency workload: 13.3 us against 14.3 us with the plain policy)
  switch (tu.llc_nt >= 0 ? tu.llc_nt & 7 : 4) {
    case 1: return launch_ll_combine_nt<1>(a, vpl, nslices, st);
    case 2: return launch_ll_combine_nt<2>(a, vpl, nslices, st);
    case 3: return launch_ll_combine_nt<3>(a, vpl, nslices, st);
    case 4: return launch_ll_combine_nt<4>(a, vpl, nslices, st);
    case 5: return launch_ll_combine_nt<5>(a, vpl, nslices, st);
    case 6: return launch_ll_combine_nt<6>(a, vpl, nslices, st);
    case 7: return launch_ll_combine_nt<7>(a, vpl, nslices, st);
    default: return launch_ll_combine_nt<0>(a, vpl, nslices, st);
  }
}

// ---------------------------------------------------------------------------
// Rank mask helpers: one entry set, all entries cleared, or the mask copied
// out.  Tiny kernels rather than memset/memcpy nodes so that a captured
// stream replays them faithfully.
__global__ void mask_set_kernel(int32_t* mask, int rank, int value) {
  if (threadIdx.x == 0) mask[rank] = value;
}

__global__ void copy_i32_kernel(const int32_t* src, int32_t* dst, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = src[i];
}

hipError_t launch_mask_set(int32_t* mask, int rank, int value, hipStream_t st) {
  hipLaunchKernelGGL(mask_set_kernel, dim3(1), dim3(kWave), 0, st, mask, rank, value);
  return hipGetLastError();
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(copy_i32_kernel, dim3(blocks), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace miep
