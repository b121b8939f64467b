// pack.hip -- normal-mode dispatch payload movement (fresh and cached).
//
// "Chapter 4  V1: layout, dispatch and combine", section 4.1: every token
// goes to every rank whose experts it selected, rank-major, together with
// its source index and the top-k entries that rank owns; the cached branch
// moves only x (and its scales) along the same placement.  The optional
// per-128-channel FP8 cast is the one of the low-latency send loop ("DeepEP
// Normal vs Low-Latency dual-mode analysis").
//
// Push design: one wavefront per (token, row slice).  The slice is read
// from HBM once into registers (16-byte loads) and written to each of the
// rho receiving ranks' rows (16-byte stores), so HBM sees 1 read + rho
// writes per token -- the minimum.  Destinations come from send_head: lane
// r holds rank r's row, a ballot gives the destination set, and the wave
// walks it with scalar find-first-set + readlane, so every store is a fully
// coalesced 1 KiB wavefront store.  No atomics anywhere: placement was
// fixed by the notify scan.  Row traffic uses buffer instructions on the
// wave-uniform row base; by default x is read with the ordinary cache policy
// and the receive rows are written non-temporal at device scope.
//
// The small per-row records of a fresh dispatch (source index, the top-k
// entries the row's rank owns and their weights) are not written by the
// payload wavefronts, where each would leave as a scattered partial-line
// piece per (token, destination): extra wavefronts at the front of the same
// grid, a few per (source, rank) pair, walk the source's tokens in order and
// write the rank's consecutive receive rows with coalesced stores, while
// the payload wavefronts run.
#include "device.h"
#include "kernels.h"

namespace miep {

// First rank of the group that row n belongs to, for rows forwarded from
// group rows (group_off[g] <= n < group_off[g+1]); 0 for a direct dispatch.
// Wave-uniform: lane g loads group_off[g] and a ballot counts the groups
// that start at or before n.
__device__ __forceinline__ int group_rank_base(const int32_t* group_off, int groups, int group_w, int64_t n) {
  if (group_off == nullptr) return 0;
  const int lane = lane_id();
  const bool le = lane <= groups && group_off[lane] <= n;
  return (__popcll(ballot(le)) - 1) * group_w;
}

constexpr int kRecordMaxTokens = 1024;   // tokens per source for the record wavefronts
constexpr int kRecordChunks = kRecordMaxTokens / kWave;
constexpr int kRecordBatch = 8;          // store instructions per batch of gathered records
constexpr int kRecordMaxParts = 16;      // record wavefronts per (source, rank) at most

// Records of rank r's rows from source s (wavefronts (s, r, p), p <
// rec_parts, mw = (s * R + r) * rec_parts + p): the rows
// [off[r] + rpm[s-1][r], off[r] + rpm[s][r]) hold source s's tokens that go
// to r, in token order.  Every membership byte of the column is loaded at
// once (one load per lane per 64-token chunk, all in flight) and ballots
// list the members' tokens in this wavefront's LDS slot.  The members form
// parts of kRecordBatch * (64 / K) rows; wavefront p takes parts p,
// p + rec_parts, ... and gathers each part's top-k entries and weights with
// every load in flight before its stores: lane (j, k) writes entry k of row
// j, so each store covers 64 / K whole rows.  A wavefront's chain is one
// round trip for the membership plus one per part it takes (the host picks
// rec_parts from the rows a rank can expect, e.g. 8 wavefronts per
// (source, rank) at 8 ranks: one (source, rank) pair holds ~340 rows, whose
// six sequential batches had made the records outlast an FP8 payload).  The
// records are written with the streaming (non-temporal) policy: their lines
// are whole, and as ordinary dirty lines they cost the 64-rank FP8 dispatch
// ~27 us (measured: 216.6 -> 189.6 us).
__device__ __forceinline__ void pack_records(const PackArgs& a, int mw, int32_t* lst) {
  const int lane = lane_id();
  const int R = a.R, T = a.T, K = a.K;
  const int P = a.rec_parts;
  const int part = mw % P;
  const int sr = mw / P;
  const int s = sr / R;
  const int r = sr - s * R;
  const int part_rows = kRecordBatch * (kWave / (K > 0 ? K : 1));   // rows of one part (one batch)
  const int row0 = a.off[r] + (s > 0 ? a.rpm[(s - 1) * R + r] : 0);   // receive row of the first member
  const uint8_t* col = a.in_rank + static_cast<int64_t>(s) * T * R + r;
  const int nch = (T + kWave - 1) / kWave;
  uint8_t mb[kRecordChunks];
#pragma unroll
  for (int c = 0; c < kRecordChunks; ++c) {
    const int t = c * kWave + lane;
    mb[c] = (c < nch && t < T) ? col[static_cast<int64_t>(t) * R] : 0;
  }
  int nm = 0;                                       // members so far (uniform)
#pragma unroll
  for (int c = 0; c < kRecordChunks; ++c) {
    if (c < nch) {
      const bool member = mb[c] != 0;
      const uint64_t m = ballot(member);
      const int pos = nm + __popcll(m & lanemask_lt());
      const int t = c * kWave + lane;
      if (member) {
        lst[pos] = t;
        if ((pos / part_rows) % P == part && row0 + pos < a.capacity)   // this wavefront's parts
          __builtin_nontemporal_store(t, a.recv_src_idx + row0 + pos);
      }
      nm += __popcll(m);
    }
  }
  if (K == 0 || a.recv_topk_idx == nullptr || nm == 0) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the wavefront reads back its own list
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rows_per = kWave / K;                   // whole rows per store instruction
  const int j_l = lane / K;
  const int k_l = lane - j_l * K;
  const bool act = j_l < rows_per;
  const int64_t lo = static_cast<int64_t>(r) * a.L;
  const bool wts = a.recv_topk_weights != nullptr;
  for (int j0 = part * part_rows; j0 < nm; j0 += P * part_rows) {   // this wavefront's parts, one batch each
    int64_t e[kRecordBatch];
    float wv[kRecordBatch];
#pragma unroll
    for (int b = 0; b < kRecordBatch; ++b) {        // every load of the batch in flight together
      const int j = j0 + b * rows_per + j_l;
      const bool ok = act && j < nm;
      const int64_t n = static_cast<int64_t>(s) * T + (ok ? lst[j] : 0);
      e[b] = ok ? a.topk_idx[n * K + k_l] : -1;
      wv[b] = ok && wts ? a.topk_weights[n * K + k_l] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < kRecordBatch; ++b) {
      const int j = j0 + b * rows_per + j_l;
      const int64_t g = static_cast<int64_t>(row0) + j;
      if (act && j < nm && g < a.capacity) {
        const bool mine = e[b] >= lo && e[b] < lo + a.L && e[b] < a.E;
        __builtin_nontemporal_store(mine ? e[b] - lo : int64_t(-1), a.recv_topk_idx + g * K + k_l);
        if (wts) __builtin_nontemporal_store(mine ? wv[b] : 0.0f, a.recv_topk_weights + g * K + k_l);
      }
    }
  }
}

template <int KIND, int VPL, int MW, int NT>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a, int nslices) {
  __shared__ int32_t lst[256 / kWave][kRecordMaxTokens];   // record wavefronts: member tokens of the source
  const int lane = lane_id();
  // record workgroups: the first rec_blocks of the grid, or with rec_last the last ones
  const int rb = a.rec_last ? static_cast<int>(blockIdx.x) - static_cast<int>(gridDim.x - a.rec_blocks)
                            : static_cast<int>(blockIdx.x);
  if (rb >= 0 && rb < a.rec_blocks) {   // record wavefronts (uniform per workgroup)
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int mw = rb * (256 / kWave) + w;
    if (mw < a.rec_waves) pack_records(a, mw, lst[w]);
    return;
  }
  const int64_t gw = wave_index() - (a.rec_last ? 0 : static_cast<int64_t>(a.rec_blocks) * (256 / kWave));
  const int64_t n = gw / nslices;
  const int slice = static_cast<int>(gw - n * nslices);
  if (n >= a.N) return;
  if (a.count != nullptr && n >= *a.count) return;   // past the forwarded rows
  const int R = a.R;
  const int rbase = group_rank_base(a.group_off, a.groups, a.group_w, n);

  // destination rows: lane holds rank (rbase + 64*i + lane)
  int dst[MW];
  uint64_t dmask[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    const int r = kWave * i + lane;
    int row = -1;
    if (r < R) {
      const int sh = a.send_head[n * R + r];
      const int o = a.off[rbase + r];                // independent of sh: both loads in flight
      row = sh >= 0 ? o + sh : -1;
    }
    const bool ok = row >= 0 && row < a.capacity;
    dst[i] = row;
    dmask[i] = ballot(ok);
  }

  const int G = a.H / kFp8Group;
  // top-k entries, source index and pre-quantised scales, once per token (by
  // slice 0): loaded here, written after the payload so that their latency
  // hides behind the row traffic
  const bool inline_meta = a.meta && a.rec_waves == 0;   // else the record wavefronts write them
  const bool head = slice == 0 && (inline_meta || KIND == kPackFp8);
  int64_t tok = n;
  int64_t e = -1;
  float wk = 0.0f, sv = 0.0f;
  if (head) {
    tok = a.src_tok != nullptr ? a.src_tok[n] : n;   // the source token the row carries
    if (inline_meta && lane < a.K) {
      e = a.topk_idx[tok * a.K + lane];
      if (a.topk_weights) wk = a.topk_weights[tok * a.K + lane];
    }
    if (KIND == kPackFp8 && G <= kWave && lane < G) sv = a.x_scales[n * G + lane];
  }

  // payload: input vectors are 16 bytes (8 bf16 or 16 E4M3 codes)
  const int nv = KIND == kPackFp8 ? a.H / 16 : a.H / 8;
  const int64_t in_row_bytes = KIND == kPackFp8 ? a.H : 2 * static_cast<int64_t>(a.H);
  const int64_t out_row_bytes = KIND == kPackBf16 ? 2 * static_cast<int64_t>(a.H) : a.H;
  const uint8_t* xrow = static_cast<const uint8_t*>(a.x) + n * in_row_bytes;
  uint8_t* recv = static_cast<uint8_t*>(a.recv_x);
  const int span = kWave * VPL;
  if constexpr (KIND == kPackCastFp8) {
    // Fused cast: lane holds pairs of adjacent 16-byte vectors (16
    // channels), so a 128-channel group is 8 lanes and every code store is
    // one 16-byte vector per lane (1 KiB per wavefront).  nv is a multiple
    // of 16, so a group is either entirely in range or entirely out.
    const int np = nv / 2;
    for (int p0 = slice * span; p0 < np; p0 += nslices * span) {
      v4u d[VPL][2];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int pi = p0 + j * kWave + lane;
        if (pi < np) {
          d[j][0] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(pi) * 32);
          d[j][1] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(pi) * 32 + 16);
        }
      }
      v4u q[VPL];
      float sci[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int pi = p0 + j * kWave + lane;
        const float amax = group8_max(pi < np ? fmaxf(absmax8(d[j][0]), absmax8(d[j][1])) : 0.0f);
        const float sc = fp8_scales(amax, a.round_scale != 0, &sci[j]);
        if (pi < np) q[j] = cast16(d[j][0], d[j][1], sc);
      }
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        uint64_t m = dmask[i];
        while (m) {
          const int b = __builtin_ctzll(m);
          m &= m - 1;
          const int64_t row = readlane(dst[i], b);
          uint8_t* orow = recv + row * out_row_bytes;
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const int pi = p0 + j * kWave + lane;
            if (pi < np) {
              stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(pi) * 16, q[j]);
              if ((lane & 7) == 0) {
                a.recv_x_scales[row * G + pi / 8] = sci[j];
                if (a.recv_ue) a.recv_ue[row * G + pi / 8] = ue8m0_byte(sci[j]);
              }
            }
          }
        }
      }
    }
  } else {
    for (int v0 = slice * span; v0 < nv; v0 += nslices * span) {
      v4u d[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int v = v0 + j * kWave + lane;
        if (v < nv) d[j] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(v) * 16);
      }
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        uint64_t m = dmask[i];
        while (m) {
          const int b = __builtin_ctzll(m);
          m &= m - 1;
          const int64_t row = readlane(dst[i], b);
          uint8_t* orow = recv + row * out_row_bytes;
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const int v = v0 + j * kWave + lane;
            if (v < nv) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(v) * 16, d[j]);
          }
        }
      }
    }
  }
  // the token's metadata and pre-quantised scales, to every destination row
  if (head) {
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      uint64_t m = dmask[i];
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        const int r = rbase + kWave * i + b;
        const int64_t row = readlane(dst[i], b);
        if (inline_meta) {
          if (lane < a.K) {
            const bool mine = e >= 0 && e < a.E && static_cast<int>(e) / a.L == r;
            if (a.recv_topk_idx) a.recv_topk_idx[row * a.K + lane] = mine ? e - static_cast<int64_t>(r) * a.L : -1;
            if (a.recv_topk_weights) a.recv_topk_weights[row * a.K + lane] = mine ? wk : 0.0f;
          }
          if (lane == 0) a.recv_src_idx[row] = static_cast<int32_t>(tok % a.T);
        }
        if constexpr (KIND == kPackFp8) {
          if (G <= kWave) {
            if (lane < G) a.recv_x_scales[row * G + lane] = sv;
          } else {
            for (int g = lane; g < G; g += kWave) a.recv_x_scales[row * G + g] = a.x_scales[n * G + g];
          }
        }
      }
    }
  }
}

// Fused FP8 cast, one token per workgroup: wavefront w casts row slice w
// (64 lanes x VPL pairs of 16-byte vectors) and stores its codes to every
// destination, 16 bytes per lane; the row's H/128 scales are gathered in LDS
// and leave as one contiguous store per destination (scattered 16-byte scale
// pieces written by separate wavefronts cost a quarter of the kernel's time).
constexpr int kCastMaxGroups = 512;  // H <= 65536

template <int VPL, int MW, int NT>
__global__ __launch_bounds__(1024) void pack_cast_kernel(PackArgs a) {
  __shared__ float row_scales[kCastMaxGroups];
  const int lane = lane_id();
  const int slice = threadIdx.x / kWave;
  const int64_t n = blockIdx.x;
  const int R = a.R;
  int dst[MW];
  uint64_t dmask[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    const int r = kWave * i + lane;
    int row = -1;
    if (r < R) {
      const int sh = a.send_head[n * R + r];
      const int o = a.off[r];
      row = sh >= 0 ? o + sh : -1;
    }
    dst[i] = row;
    dmask[i] = ballot(row >= 0 && row < a.capacity);
  }
  const int G = a.H / kFp8Group;
  // the token's top-k entries: loaded now, written with the scales after the
  // payload, so their latency hides behind the row traffic instead of
  // holding up slice 0 (and through the barrier, the whole token)
  int64_t e = -1;
  float wk = 0.0f;
  if (slice == 0 && a.meta && lane < a.K) {
    e = a.topk_idx[n * a.K + lane];
    if (a.topk_weights) wk = a.topk_weights[n * a.K + lane];
  }
  // lane holds VPL pairs of adjacent 16-byte vectors (16 channels each), so
  // a 128-channel group is 8 lanes and each code store is 16 bytes per lane
  const int np = a.H / 16;
  const uint8_t* xrow = static_cast<const uint8_t*>(a.x) + n * 2 * static_cast<int64_t>(a.H);
  uint8_t* recv = static_cast<uint8_t*>(a.recv_x);
  const int p0 = slice * kWave * VPL;
  v4u d[VPL][2];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int pi = p0 + j * kWave + lane;
    if (pi < np) {
      d[j][0] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(pi) * 32);
      d[j][1] = ldb16<load_cpol(NT)>(xrow, static_cast<uint32_t>(pi) * 32 + 16);
    }
  }
  v4u q[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int pi = p0 + j * kWave + lane;
    const float amax = group8_max(pi < np ? fmaxf(absmax8(d[j][0]), absmax8(d[j][1])) : 0.0f);
    float sci;
    const float sc = fp8_scales(amax, a.round_scale != 0, &sci);
    if (pi < np) {
      q[j] = cast16(d[j][0], d[j][1], sc);
      if ((lane & 7) == 0) row_scales[pi / 8] = sci;
    }
  }
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    uint64_t m = dmask[i];
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1;
      uint8_t* orow = recv + static_cast<int64_t>(readlane(dst[i], b)) * a.H;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int pi = p0 + j * kWave + lane;
        if (pi < np) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(pi) * 16, q[j]);
      }
    }
  }
  __syncthreads();
  if (slice == 0) {
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      uint64_t m = dmask[i];
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        const int r = kWave * i + b;
        const int64_t row = readlane(dst[i], b);
        float* srow = a.recv_x_scales + row * G;
        for (int g = lane; g < G; g += kWave) srow[g] = row_scales[g];
        if (a.recv_ue) {
          uint8_t* urow = a.recv_ue + row * G;
          for (int g = lane; g < G; g += kWave) urow[g] = ue8m0_byte(row_scales[g]);
        }
        if (a.meta) {
          if (lane < a.K) {
            const bool mine = e >= 0 && e < a.E && static_cast<int>(e) / a.L == r;
            if (a.recv_topk_idx) a.recv_topk_idx[row * a.K + lane] = mine ? e - static_cast<int64_t>(r) * a.L : -1;
            if (a.recv_topk_weights) a.recv_topk_weights[row * a.K + lane] = mine ? wk : 0.0f;
          }
          if (lane == 0) a.recv_src_idx[row] = static_cast<int32_t>(n % a.T);
        }
      }
    }
  }
}

template <int VPL, int NT>
static hipError_t launch_pack_cast_vpl(const PackArgs& a, hipStream_t st) {
  const int np = a.H / 16;   // pairs of 16-byte input vectors
  const int waves = (np + kWave * VPL - 1) / (kWave * VPL);
  if (a.N > max_blocks(static_cast<int64_t>(waves) * kWave)) return hipErrorInvalidConfiguration;
  if (a.R <= 64)
    hipLaunchKernelGGL((pack_cast_kernel<VPL, 1, NT>), dim3(static_cast<unsigned>(a.N)), dim3(waves * kWave), 0, st,
                       a);
  else
    hipLaunchKernelGGL((pack_cast_kernel<VPL, 4, NT>), dim3(static_cast<unsigned>(a.N)), dim3(waves * kWave), 0, st,
                       a);
  return hipGetLastError();
}

// Smallest vector pairs per lane (at least `ppl_hint`) that fits the row in
// 16 wavefronts.
template <int NT>
static hipError_t launch_pack_cast(const PackArgs& a, int ppl_hint, hipStream_t st) {
  const int np = a.H / 16;
  if (ppl_hint <= 1 && np <= 16 * kWave) return launch_pack_cast_vpl<1, NT>(a, st);
  if (ppl_hint <= 2 && np <= 32 * kWave) return launch_pack_cast_vpl<2, NT>(a, st);
  if (ppl_hint <= 4 && np <= 64 * kWave) return launch_pack_cast_vpl<4, NT>(a, st);
  return launch_pack_cast_vpl<8, NT>(a, st);
}

template <int KIND, int VPL, int NT>
static hipError_t launch_pack_vpl(const PackArgs& a, int nslices, hipStream_t st) {
  const int64_t waves = a.N * nslices;
  const int64_t blocks = (waves + 3) / 4 + a.rec_blocks;
  if (blocks > max_blocks(256)) return hipErrorInvalidConfiguration;
  if (a.R <= 64)
    hipLaunchKernelGGL((pack_kernel<KIND, VPL, 1, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                       nslices);
  else
    hipLaunchKernelGGL((pack_kernel<KIND, VPL, 4, NT>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                       nslices);
  return hipGetLastError();
}

template <int KIND, int NT>
static hipError_t launch_pack_kind(const PackArgs& a, int vpl, int nslices, hipStream_t st) {
  switch (vpl) {
    case 1: return launch_pack_vpl<KIND, 1, NT>(a, nslices, st);
    case 2: return launch_pack_vpl<KIND, 2, NT>(a, nslices, st);
    case 4: return launch_pack_vpl<KIND, 4, NT>(a, nslices, st);
    case 7: return launch_pack_vpl<KIND, 7, NT>(a, nslices, st);
    default: return launch_pack_vpl<KIND, 8, NT>(a, nslices, st);
  }
}

template <int KIND>
static hipError_t launch_pack_nt(const PackArgs& a, int vpl, int nslices, int nt, hipStream_t st) {
  switch (nt) {
    case 0: return launch_pack_kind<KIND, 0>(a, vpl, nslices, st);
    case 1: return launch_pack_kind<KIND, 1>(a, vpl, nslices, st);
    case 2: return launch_pack_kind<KIND, 2>(a, vpl, nslices, st);
    case 3: return launch_pack_kind<KIND, 3>(a, vpl, nslices, st);
    case 4: return launch_pack_kind<KIND, 4>(a, vpl, nslices, st);
    case 5: return launch_pack_kind<KIND, 5>(a, vpl, nslices, st);
    case 7: return launch_pack_kind<KIND, 7>(a, vpl, nslices, st);
    default: return launch_pack_kind<KIND, 6>(a, vpl, nslices, st);
  }
}

hipError_t launch_pack(const PackArgs& a_in, hipStream_t st) {
  if (a_in.N == 0) return hipSuccess;
  const Tuning& tu = tuning();
  PackArgs a = a_in;
  // record wavefronts, rec_parts per (source, rank), for a fresh direct dispatch
  // whose sources hold at most kRecordMaxTokens tokens (a record wavefront
  // walks its source in 64-token chunks); forwarded group rows, longer
  // sources and the one-token-per-workgroup cast keep the records in their
  // payload wavefronts
  const bool cast_tpb = a.kind == kPackCastFp8 && tu.cast_tpb > 0;
  if (a.meta && a.group_off == nullptr && a.src_tok == nullptr && a.count == nullptr && a.rpm != nullptr &&
      a.in_rank != nullptr && !cast_tpb && tu.pack_records != 0 && a.T <= kRecordMaxTokens) {
    // parts per (source, rank) from the rows a rank can expect: a source's T
    // tokens reach at most min(K, R) ranks each, so a rank expects up to
    // T * min(K, R) / R rows from it (every wavefront loops over its parts,
    // so any routing is covered)
    const int part_rows = kRecordBatch * (kWave / (a.K > 0 ? a.K : 1));
    const int64_t expect = (static_cast<int64_t>(a.T) * (a.K < a.R ? a.K : a.R) + a.R - 1) / a.R;
    int parts = static_cast<int>((expect + part_rows - 1) / part_rows);
    parts = parts < 1 ? 1 : (parts > kRecordMaxParts ? kRecordMaxParts : parts);
    const int64_t rw = static_cast<int64_t>(a.S) * a.R * parts;
    a.rec_parts = parts;
    a.rec_waves = rw <= (int64_t(1) << 30) ? static_cast<int>(rw) : 0;   // else the payload wavefronts write them
    a.rec_blocks = (a.rec_waves + 3) / 4;
    a.rec_last = tu.pack_records == 2 ? 1 : 0;
  } else {
    a.rec_waves = 0;
    a.rec_blocks = 0;
  }
  const int nt = tu.pack_nt >= 0 ? tu.pack_nt & 7 : (a.cpol >= 0 ? a.cpol & 7 : 6);
  // per-lane unit: a 16-byte input vector, or for the fused cast a pair of
  // them (16 channels -> one 16-byte vector of codes)
  const int nv = a.kind == kPackFp8 ? a.H / 16 : (a.kind == kPackCastFp8 ? a.H / 16 : a.H / 8);
  // default geometry: one unit per lane, i.e. every wavefront writes one
  // 1 KiB piece of a row to each destination (hidden 7168 bf16 -> 14
  // wavefronts per token).  Measured on MI355X, writes spread as many small
  // per-wavefront pieces reach ~6.7 TB/s while 4-16 KiB per wavefront drop to
  // 5.4-5.9 TB/s.  Rows that are not a multiple of 64 units keep 8.
  // Forwarding from group rows has a longer per-wavefront prologue (row
  // count, group lookup, source token), so it moves 2 units per lane
  // (measured on the 64-rank FP8 relay: 514 -> 477 us per relay dispatch).
  const int base_vpl = a.group_off != nullptr ? 2 : 1;
  int vpl = tu.pack_vpl > 0 ? tu.pack_vpl : (nv % kWave == 0 ? base_vpl : 8);
  int span = vpl * kWave;
  int nslices = tu.pack_slices > 0 ? tu.pack_slices : (nv + span - 1) / span;
  if (nslices < 1) nslices = 1;
  switch (a.kind) {
    case kPackFp8: return launch_pack_nt<kPackFp8>(a, vpl, nslices, nt, st);
    case kPackCastFp8:
      // One token per workgroup (its H/128 scales gathered in LDS and stored
      // contiguously, the records written inline) only on request: with the
      // records in their own wavefronts the 1 KiB slices are faster also for
      // a fresh dispatch.  The token-per-workgroup kernel has no forwarding mode.
      if (cast_tpb && a.group_off == nullptr && a.count == nullptr && a.src_tok == nullptr) {
        const int hint = tu.pack_vpl > 0 ? tu.pack_vpl : 1;   // 1 pair = 2 vectors per lane
        switch (nt) {
          case 0: return launch_pack_cast<0>(a, hint, st);
          case 1: return launch_pack_cast<1>(a, hint, st);
          case 2: return launch_pack_cast<2>(a, hint, st);
          case 3: return launch_pack_cast<3>(a, hint, st);
          case 4: return launch_pack_cast<4>(a, hint, st);
          case 5: return launch_pack_cast<5>(a, hint, st);
          case 7: return launch_pack_cast<7>(a, hint, st);
          default: return launch_pack_cast<6>(a, hint, st);
        }
      }
      return launch_pack_nt<kPackCastFp8>(a, vpl, nslices, nt, st);
    default: return launch_pack_nt<kPackBf16>(a, vpl, nslices, nt, st);
  }
}

}  // namespace miep
