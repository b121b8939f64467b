// notify.hip -- the dispatch's notify step on one GPU: the handle's prefix
// matrices, the receive offsets, send_head and the aligned per-expert
// receive counts.
//
// "Chapter 4  V1: layout, dispatch and combine", sections 4.1-4.2: a fresh
// dispatch returns the rank prefix matrix, the channel prefix matrix, the
// receive-side channel prefix matrix, the source indices and send_head,
// which together form the reverse-routing handle.  Channels hold
// ceil(T/C) consecutive tokens of a source ("DeepEP Normal vs Low-Latency
// dual-mode analysis", V2 channel constants).  Across GPUs this step is an
// exchange of counts; with the ranks as partitions of one GPU it is a local
// scan.
//
// Two kernels, neither of which waits on another workgroup: rank bases
// (rows of rank r before source s) come from the layout's
// num_tokens_per_rank.
//  - notify_chan_kernel (rows of 8, 16, 32 or 64 ranks, channels of at most
//    256 tokens): one workgroup per run of whole channels of one source; the
//    earlier channels' rows per rank come from a byte-wise sum of their
//    membership rows (see the kernel's comment).
//  - notify_kernel (other shapes, and the relay's group notify): one
//    workgroup per source.  Within a wavefront of 64 tokens the per-rank
//    counts and prefixes come from one ballot per rank (rows of <= 8 ranks)
//    or from a bit transpose of the tokens' rank masks through LDS (wider
//    rows); each wavefront adds the earlier wavefronts' counts from LDS with
//    independent reads.
// send_head rows leave as 16-byte stores in both.  (An earlier split of a
// source over several workgroups that recounted its earlier tokens with
// ballots measured slower: 14.2 us with 64-token tiles against 8.7 us for
// the normal workload; the byte-wise sum is what made the split pay.)
#include "device.h"
#include "kernels.h"

namespace miep {

constexpr int kNotifyMaxWaves = 16;

// send_head rows leave in 16-byte stores.  Large send_head arrays (64 ranks:
// 4 MB for the 16384-token workload) are written with the streaming
// (non-temporal) policy: left as ordinary dirty lines they slowed the pack
// that follows by ~9 us (measured: notify then cached pack 193.6 us, 179.4 us
// with streaming stores, against 183.5 us for the two apart); small ones
// keep the default policy (8 ranks: streaming cost the next pack ~2 us).
template <bool NT>
__device__ __forceinline__ void store_head4(int32_t* base, int64_t idx, int4 v) {
  if constexpr (NT) {
    const u32x4 t = {static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y), static_cast<uint32_t>(v.z),
                     static_cast<uint32_t>(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(t, row_rsrc(base), static_cast<uint32_t>(idx * 4), 0, kCpolNt);
  } else {
    *reinterpret_cast<int4*>(base + idx) = v;
  }
}
constexpr int64_t kHeadStreamBytes = 1 << 20;   // send_head arrays above this size stream

// Nonzero bytes of a 32-bit word -> 4 bits (byte j -> bit j): fold each byte
// onto its low bit, then one multiply moves bits 0, 8, 16, 24 to 28..31 (the
// other partial products land on distinct lower bits, so nothing carries in).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t v) {
  v |= v >> 4;
  v |= v >> 2;
  v |= v >> 1;
  return ((v & 0x01010101u) * 0x10204080u) >> 28;
}

// Membership row of R <= 4*NW ranks (R % 4 == 0) kept as raw words between
// the loads and the decode, so that independent loads issued in between are
// in flight together.  R == 8 rows (8-byte aligned) take one 8-byte load.
template <int NW>
struct RowWords {
  uint32_t v[NW];
};
template <int NW>
__device__ __forceinline__ void issue_row_words(const uint8_t* row, int R, bool one8, RowWords<NW>& rw) {
  if (NW >= 2 && one8) {
    const uint64_t q = *reinterpret_cast<const uint64_t*>(row);
    rw.v[0] = static_cast<uint32_t>(q);
    rw.v[1] = static_cast<uint32_t>(q >> 32);
#pragma unroll
    for (int i = 2; i < NW; ++i) rw.v[i] = 0u;
  } else if (NW >= 16 && (R & 15) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    // 16-byte pieces (rows of 16, 32, 48 or 64 ranks), clamped like below
#pragma unroll
    for (int i = 0; i < NW; i += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + (4 * i < R ? 4 * i : R - 16));
      rw.v[i] = q.x;
      rw.v[i + 1] = q.y;
      rw.v[i + 2] = q.z;
      rw.v[i + 3] = q.w;
    }
  } else {
    // unconditional loads from clamped offsets (words past the row are
    // skipped by the decode): a load whose result is selected right away
    // gets its own wait from the compiler
#pragma unroll
    for (int i = 0; i < NW; ++i) rw.v[i] = *reinterpret_cast<const uint32_t*>(row + (4 * i < R ? 4 * i : R - 4));
  }
}
template <int NW>
__device__ __forceinline__ RankMask<1> decode_row_words(const RowWords<NW>& rw, int R) {
  uint64_t w = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (4 * i < R) w |= static_cast<uint64_t>(nonzero_bytes4(rw.v[i])) << (4 * i);
  RankMask<1> m;
  m.w[0] = w;
  return m;
}

// Destination set of token n: its rank row, or (GROUPED, group_w == 8) one
// bit per group of 8 ranks, set when any of the group's 8 bytes is set (one
// 8-byte load per group).  RB <= 8: rows of 4 or 8 bytes.
template <int MW, bool GROUPED, int RB>
__device__ __forceinline__ RankMask<MW> load_member(const NotifyArgs& a, int64_t n) {
  if constexpr (RB <= 8 && MW == 1 && !GROUPED) {
    if ((a.R & 3) != 0) return load_rank_row<1>(a.in_rank + n * a.R, a.R);   // byte rows
    RowWords<2> rw;
    issue_row_words<2>(a.in_rank + n * a.R, a.R, a.R == 8 && (reinterpret_cast<uintptr_t>(a.in_rank) & 7u) == 0, rw);
    return decode_row_words<2>(rw, a.R);
  } else if constexpr (!GROUPED) {
    return load_rank_row<MW>(a.in_rank + n * a.R, a.R);
  } else {
    const uint64_t* row = reinterpret_cast<const uint64_t*>(a.in_rank + n * a.R * 8);
    RankMask<MW> m;
    m.clear();
    for (int g = 0; g < a.R; ++g)
      if (row[g] != 0ull) m.set(g);
    return m;
  }
}

// The kernel is latency-bound (8 workgroups for the normal workload), and a
// wavefront issues about one instruction per 4 cycles, so its time is the
// length of its instruction chain plus its global round trips: no integer
// divides (wavefronts walk whole count rows; channel indices use FastDiv),
// one round trip for all the loads of the first token tile, and no serial
// scan across wavefronts (each wavefront sums the earlier ones' counts from
// LDS with independent reads).  RB bounds the ranks per row at compile time:
// 8 = rows of at most 8 ranks, one ballot per rank (unrolled); 64 = rows of
// up to 64 ranks (or groups), where the wavefront's membership masks go
// through LDS and lane r assembles rank r's 64-token bit column, which gives
// the rank's count and every in-wavefront prefix by popcount, and send_head
// leaves one token row at a time with the ranks side by side (contiguous
// stores); 256 = rows of up to 256 ranks, one ballot per rank.
template <int MW, bool GROUPED, int RB, bool HNT>
__global__ __launch_bounds__(1024) void notify_kernel(NotifyArgs a) {
  __shared__ int32_t base[kMaxRanks];                 // rows of rank r from sources < s
  __shared__ int32_t total[kMaxRanks];                // rows of rank r from all sources
  __shared__ int32_t run[kMaxRanks];                  // tokens of s in earlier tiles that go to r
  __shared__ int32_t wt[kNotifyMaxWaves][kMaxRanks];  // per-wavefront counts of the current tile

  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: source loops stay scalar
  const int nw = blockDim.x / kWave;
  const int R = a.R, T = a.T, C = a.C, S = a.S;

  constexpr bool kWide = MW == 1 && RB == 64;
  constexpr int kRankUnroll = RB <= 8 ? RB : 1;        // ballot loops: unrolled for rows of <= 8 ranks
  constexpr int kQuadUnroll = RB <= 8 ? RB / 4 : 1;
  extern __shared__ uint64_t dyn[];
  uint64_t* mk = dyn;                                  // [nw][64] membership masks (wide rows)
  // wide rows: [nw][64] masks (later the rank columns), then [nw][64] rank bases
  int32_t* eacc = reinterpret_cast<int32_t*>(dyn + (kWide ? nw * kWave : 0)) + (kWide ? nw * kWave : 0);
  const int ne = a.E > s ? (a.E - s + S - 1) / S : 0; // experts e = s + k*S
  const bool do_e = a.nrte != nullptr && a.ntpe != nullptr;

  // (1) rank totals / bases and the sums of the owned experts' counts:
  // wavefront w walks sources w, w + nw, ...; lane j of a 64-wide chunk
  // takes rank 64*i + j (and owned expert j), so the loads are whole rows.
  // The first batch is issued before the membership loads, so that a wait
  // the compiler places on those cannot hold the count loads back.
  int tot[MW], bas[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) tot[i] = bas[i] = 0;
  int eac = 0;
  const bool e_lane = do_e && lane < ne;
  // every load is unconditional, from a clamped (always valid) index, and
  // masked afterwards; a batch of B sources is chosen by a uniform branch
  const bool e_any = do_e && ne > 0;                  // expert s exists (E > s)
  const int32_t* ep = e_any ? a.ntpe : a.ntpr;
  const int kc = e_lane ? lane : 0;
  int vr[16][MW], ve[16];
  auto issue_counts = [&](int src0, int B) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < B) {
        const int src = src0 + u * nw;
        const int sc = src < S ? src : S - 1;
#pragma unroll
        for (int i = 0; i < MW; ++i) {
          const int r = kWave * i + lane;
          vr[u][i] = a.ntpr[sc * R + (r < R ? r : R - 1)];
        }
        ve[u] = ep[e_any ? static_cast<int64_t>(sc) * a.E + s + kc * S : 0];
      }
    }
  };
  auto add_counts = [&](int src0, int B) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u < B) {
        const int src = src0 + u * nw;
        const bool before = src < s;                  // (s < S, so also src < S)
#pragma unroll
        for (int i = 0; i < MW; ++i) {
          const int v = src < S && kWave * i + lane < R ? vr[u][i] : 0;
          tot[i] += v;
          bas[i] += before ? v : 0;
        }
        eac += e_lane && src < S ? ve[u] : 0;
      }
    }
  };
  const int need = w < S ? (S - w + nw - 1) / nw : 0;   // sources this wavefront walks
  const int b0 = need <= 1 ? 1 : (need <= 4 ? 4 : 16);
  if (need > 0) issue_counts(w, b0);

  // (2) the first token tile's membership row: loads issued, decoded later
  constexpr bool kLazy = MW == 1 && !GROUPED;
  constexpr int kNW = RB <= 8 ? 2 : 16;               // row words
  const bool lazy = kLazy && (R & 3) == 0;
  const bool one8 = R == 8 && (reinterpret_cast<uintptr_t>(a.in_rank) & 7u) == 0;
  RowWords<kNW> rw;
  RankMask<MW> first;
  first.clear();
  if (tid < T) {
    if (lazy) issue_row_words<kNW>(a.in_rank + (static_cast<int64_t>(s) * T + tid) * R, R, one8, rw);
    else first = load_member<MW, GROUPED, RB>(a, static_cast<int64_t>(s) * T + tid);
  }
  for (int r = tid; r < R; r += blockDim.x) {
    base[r] = 0;
    total[r] = 0;
    run[r] = 0;
  }
  for (int k = tid; k < ne; k += blockDim.x) eacc[k] = 0;
  if (need > 0) add_counts(w, b0);
  for (int src0 = w + 16 * nw; src0 < S; src0 += 16 * nw) {   // more than 16 sources per wavefront
    issue_counts(src0, 16);
    add_counts(src0, 16);
  }
  if constexpr (kLazy) {
    if (lazy && tid < T) first = decode_row_words<kNW>(rw, R);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    const int r = kWave * i + lane;
    if (r < R) {
      if (tot[i]) atomicAdd(&total[r], tot[i]);
      if (bas[i]) atomicAdd(&base[r], bas[i]);
    }
  }
  if (e_lane && eac) atomicAdd(&eacc[lane], eac);
  if (do_e) {                                         // owned experts past the first 64 (few sources)
    for (int k0 = kWave; k0 < ne; k0 += kWave) {
      const int k = k0 + lane;
      int acc = 0;
      if (k < ne)
        for (int src = w; src < S; src += nw) acc += a.ntpe[static_cast<int64_t>(src) * a.E + s + k * S];
      if (k < ne && acc) atomicAdd(&eacc[k], acc);
    }
  }
  __syncthreads();

  const int tc = a.tcdiv.d;
  const bool fast_tc = T <= (1 << 20);                // FastDiv is exact there
  int fin[MW];                                        // tokens of s per rank (wavefront 0, after the loop)
#pragma unroll
  for (int i = 0; i < MW; ++i) fin[i] = 0;
  for (int t0 = 0; t0 < T; t0 += blockDim.x) {
    const int t = t0 + tid;
    const bool valid = t < T;
    const int64_t n = static_cast<int64_t>(s) * T + t;
    RankMask<MW> m = first;
    if (t0 > 0) {
      m.clear();
      if (valid) m = load_member<MW, GROUPED, RB>(a, n);
    }
    // pass 1: per-wavefront counts, lane j of the wave keeps rank r0 + j
    uint64_t col = 0;                                 // wide rows: bit q = token q of this wavefront goes to rank `lane`
    if constexpr (kWide) {
      mk[w * kWave + lane] = m.w[0];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the wavefront reads back its own masks
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const ulonglong2* mw = reinterpret_cast<const ulonglong2*>(mk + w * kWave);
#pragma unroll 8
      for (int q = 0; q < kWave / 2; ++q) {           // broadcast reads, two masks each
        const ulonglong2 p = mw[q];
        col |= ((p.x >> lane) & 1ull) << (2 * q);
        col |= ((p.y >> lane) & 1ull) << (2 * q + 1);
      }
      if (lane < R) wt[w][lane] = __popcll(col);
    } else {
      for (int r0 = 0; r0 < R; r0 += kWave) {
        const int rend = R - r0 < kWave ? R - r0 : kWave;
        int mine = 0;
#pragma unroll kRankUnroll
        for (int j = 0; j < (RB < kWave ? RB : kWave); ++j) {
          if (j >= rend) break;
          const int c = __popcll(ballot(m.get(r0 + j) != 0));
          mine = lane == j ? c : mine;
        }
        if (lane < rend) wt[w][r0 + lane] = mine;
      }
    }
    __syncthreads();
    // this wavefront's exclusive base per rank within source s: earlier
    // tiles (run) plus the earlier wavefronts of this tile; all reads independent
    int pre[MW], tile[MW];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int r = kWave * i + lane;
      int acc = 0, all = 0;
      if (r < R) {
        acc = run[r];
        for (int q = 0; q < nw; ++q) {
          const int v = wt[q][r];
          acc += q < w ? v : 0;
          all += v;
        }
      }
      pre[i] = acc;
      tile[i] = all;
    }
    // pass 2: exclusive rank within source s -> send_head, channel prefixes.
    // Lane j holds rank r0 + j's bases in registers; per-rank values come by
    // readlane, so no lane walks a dependent LDS chain.
    const int ch = fast_tc ? fdiv(t, a.tcdiv) : t / tc;   // channel of token t
    const bool last_in_channel = valid && (t - ch * tc == tc - 1 || t == T - 1);
    const uint64_t clast = ballot(last_in_channel);
    if constexpr (kWide) {
      const int wt_l = pre[0];
      const int base_l = lane < R ? base[lane] : 0;
      const int pos_l = base_l + wt_l;
      const int tw0 = t0 + w * kWave;                 // first token of this wavefront
      const int nq = T - tw0 < kWave ? T - tw0 : kWave;
      int32_t* row0 = a.send_head + (static_cast<int64_t>(s) * T + tw0) * R;
      if ((R & 3) == 0) {
        // rows leave as 16-byte pieces: lane (tq, j) writes ranks 4j..4j+3 of
        // token q0 + tq, so one store instruction covers 64 / QP token rows
        // (QP = R/4 rounded up to a power of two); the rank lanes' columns and
        // bases go through this wavefront's LDS slot first
        uint64_t* cb = mk + w * kWave;
        int32_t* pb = reinterpret_cast<int32_t*>(mk + nw * kWave) + w * kWave;
        cb[lane] = col;
        pb[lane] = pos_l;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int ql = R >> 2;                        // lanes per token row
        const int lg = ql <= 1 ? 0 : 32 - __builtin_clz(static_cast<unsigned>(ql - 1));
        const int tq = lane >> lg, j = lane & ((1 << lg) - 1);
        const bool act = j < ql;
        uint64_t c4[4];
        int p4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          c4[k] = act ? cb[4 * j + k] : 0ull;
          p4[k] = act ? pb[4 * j + k] : 0;
        }
        for (int q0 = 0; q0 < nq; q0 += kWave >> lg) {
          const int q = q0 + tq;
          if (act && q < nq) {
            const uint64_t below = (1ull << q) - 1ull;
            int v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              v[k] = ((c4[k] >> q) & 1ull) ? p4[k] + __popcll(c4[k] & below) : -1;
            store_head4<HNT>(a.send_head, (static_cast<int64_t>(s) * T + tw0 + q) * R + 4 * j,
                             make_int4(v[0], v[1], v[2], v[3]));
          }
        }
      } else {
        for (int q = 0; q < nq; ++q) {                // token q's row: lane r writes rank r
          const bool bit = ((col >> q) & 1ull) != 0;
          const int v = bit ? pos_l + __popcll(col & ((1ull << q) - 1ull)) : -1;
          if (lane < R) row0[static_cast<int64_t>(q) * R + lane] = v;
        }
      }
      for (uint64_t cl = clast; cl != 0; cl &= cl - 1) {
        const int L = __builtin_ctzll(cl);
        const int cc = readlane(ch, L);
        const uint64_t upto = L == kWave - 1 ? ~0ull : ((2ull << L) - 1);   // tokens 0..L
        if (lane < R) {
          const int inc = wt_l + __popcll(col & upto);
          a.cpm[(static_cast<int64_t>(s) * R + lane) * C + cc] = inc;
          a.rcpm[(static_cast<int64_t>(lane) * S + s) * C + cc] = base_l + inc;
        }
      }
    }
    for (int i = 0; i < (kWide ? 0 : MW); ++i) {
      const int r0 = kWave * i;
      if (r0 >= R) break;
      const int rend = R - r0 < kWave ? R - r0 : kWave;
      const int wt_l = pre[i];
      const int base_l = lane < rend ? base[r0 + lane] : 0;
      const int pos_l = base_l + wt_l;
      uint64_t myb = 0;                                // lane j: this wavefront's ballot for rank r0 + j
#pragma unroll kQuadUnroll
      for (int j0 = 0; j0 < (RB < kWave ? RB : kWave); j0 += 4) {
        if (j0 >= rend) break;
        int v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + q;
          v[q] = -1;
          if (j < rend) {
            const bool bit = m.get(r0 + j) != 0;
            const uint64_t b = ballot(bit);
            myb = lane == j ? b : myb;
            const int pj = readlane(pos_l, j);        // with every lane active
            if (bit) v[q] = pj + __popcll(b & lanemask_lt());
          }
        }
        if (valid) {
          int32_t* dst = a.send_head + n * R + r0 + j0;
          if ((R & 3) == 0) {
            store_head4<HNT>(a.send_head, n * R + r0 + j0, make_int4(v[0], v[1], v[2], v[3]));
          } else {
            for (int q = 0; q < 4 && j0 + q < rend; ++q) dst[q] = v[q];
          }
        }
      }
      // channel prefixes: one wavefront-wide store per channel that ends on
      // a token of this wavefront (lane j writes rank r0 + j)
      for (uint64_t cl = clast; cl != 0; cl &= cl - 1) {
        const int L = __builtin_ctzll(cl);
        const int cc = readlane(ch, L);
        const uint64_t upto = L == kWave - 1 ? ~0ull : ((2ull << L) - 1);   // lanes 0..L
        if (lane < rend) {
          const int inc = wt_l + __popcll(myb & upto);
          const int r = r0 + lane;
          a.cpm[(static_cast<int64_t>(s) * R + r) * C + cc] = inc;
          a.rcpm[(static_cast<int64_t>(r) * S + s) * C + cc] = base_l + inc;
        }
      }
    }
    // carry into the next tile (wavefront 0's base is the carry itself);
    // after the last tile wavefront 0 keeps the source's totals in registers
#pragma unroll
    for (int i = 0; i < MW; ++i) fin[i] = pre[i] + tile[i];
    if (t0 + static_cast<int>(blockDim.x) < T) {
      __syncthreads();
      if (w == 0) {
#pragma unroll
        for (int i = 0; i < MW; ++i) {
          const int r = kWave * i + lane;
          if (r < R) run[r] = fin[i];
        }
      }
    }
  }

  // Everything below only stores, after the last barrier (a barrier's
  // fence waits for the wavefront's outstanding global stores).
  // Rank prefix row of this source; channels past the last token hold the total.
  if (w == 0) {
    const int nonempty = a.nonempty;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int r = kWave * i + lane;
      if (r < R) {
        const int b = base[r];
        a.rpm[static_cast<int64_t>(s) * R + r] = b + fin[i];
        for (int c = nonempty; c < C; ++c) {
          a.cpm[(static_cast<int64_t>(s) * R + r) * C + c] = fin[i];
          a.rcpm[(static_cast<int64_t>(r) * S + s) * C + c] = b + fin[i];
        }
      }
    }
  }
  // receive offsets: exclusive scan of the per-rank totals (workgroup 0)
  if (s == 0 && w == 0) {
    int carry = 0;
    for (int r0 = 0; r0 < R; r0 += kWave) {
      const int r = r0 + lane;
      const int v = r < R ? total[r] : 0;
      const int inc = wave_inclusive_scan(v);
      if (r < R) a.off[r] = carry + inc - v;
      carry += readlane(inc, kWave - 1);
    }
    if (lane == 0) {
      a.off[R] = carry;
      // capacity overflow (fixed-capacity receive side): rows past it are skipped by every writer
      if (a.status != nullptr) {
        const bool over = carry > a.capacity;
        if (!a.status_or) *a.status = over ? kStatusCapacity : 0;
        else if (over) *a.status = kStatusCapacity;
      }
    }
  }

  // per-expert receive counts, rounded up to the expert alignment (the sum
  // is at most S*T < 2^31, so sum + align - 1 fits 32 unsigned bits)
  if (do_e) {
    const uint32_t al = static_cast<uint32_t>(a.align);
    for (int k = tid; k < ne; k += blockDim.x) {
      const uint32_t sum = static_cast<uint32_t>(eacc[k]);
      a.nrte[s + k * S] = static_cast<int32_t>(al == 1u ? sum : (sum + al - 1u) / al * al);
    }
  }
}

// ---- one workgroup per group of channels of one source --------------------
//
// Rows of R = 8, 16, 32 or 64 ranks with channels of at most 256 tokens.  The
// per-source kernel above is bound by the length of one workgroup's chain;
// here a workgroup handles a run of whole channels of one source (as many as
// fit in one wavefront of 64 tokens, else one channel: 96 workgroups of two
// 22-token channels for the normal workload, 320 of five 11-token channels
// at 64 ranks) and takes everything that other workgroups would produce
// straight from the inputs, so that no workgroup waits on another:
//  - rows of rank r from sources before s: the sum of those sources'
//    num_tokens_per_rank rows;
//  - rows of rank r from the earlier channels of s: a byte-wise sum of their
//    tokens' membership rows, which are one contiguous byte range (16-byte
//    loads; byte b of the range belongs to rank b mod R, so every piece a
//    lane loads covers the same ranks and byte counters add without carries);
//  - its own tokens: ballots per rank (R = 8) or the bit transpose through
//    LDS (wider rows), as in the per-source kernel.
// Every load is issued before the first wait, and the cross-lane sums run in
// DPP row operations plus two lane exchanges, so a workgroup's chain is one
// round trip, a few dozen ALU instructions, one barrier and its stores.  The
// per-expert receive counts are spread over all workgroups.
constexpr int kChanMaxTokens = 256;   // tokens per channel (4 wavefronts)
constexpr int kChanMaxPieces = 127;   // 16-byte pieces per lane in the recount (byte counters, folded for R = 8)
constexpr int kChanBatch = 16;        // loads of one kind in flight per lane
constexpr int kChanEarlyE = 4;        // owned experts whose count loads join the first round trip

template <int R>
struct ChanRow {
  uint32_t v[R <= 8 ? 2 : R / 4];
};
template <int R>
__device__ __forceinline__ void chan_load_row(const uint8_t* row, ChanRow<R>& cr) {
  if constexpr (R == 8) {
    const uint64_t q = *reinterpret_cast<const uint64_t*>(row);
    cr.v[0] = static_cast<uint32_t>(q);
    cr.v[1] = static_cast<uint32_t>(q >> 32);
  } else {
#pragma unroll
    for (int i = 0; i < R / 16; ++i) {
      const uint4 q = reinterpret_cast<const uint4*>(row)[i];
      cr.v[4 * i] = q.x;
      cr.v[4 * i + 1] = q.y;
      cr.v[4 * i + 2] = q.z;
      cr.v[4 * i + 3] = q.w;
    }
  }
}
template <int R>
__device__ __forceinline__ uint64_t chan_row_mask(const ChanRow<R>& cr) {
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < (R <= 8 ? 2 : R / 4); ++i) m |= static_cast<uint64_t>(nonzero_bytes4(cr.v[i])) << (4 * i);
  return m;
}

// Sum of the lanes that agree modulo P (P = 1, 2, 4, 8 or 16) across the
// wavefront: DPP within each row of 16 lanes (quad permutes, then row shifts
// by 4 and 8 that fill with 0), then the four rows through two lane
// exchanges.  Lane 16 - P + j of every row ends up with class j's sum.
template <int P>
__device__ __forceinline__ uint32_t class_sum(uint32_t v) {
  int x = static_cast<int>(v);
  if constexpr (P == 1) x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if constexpr (P <= 2) x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if constexpr (P <= 4) x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  if constexpr (P <= 8) x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return static_cast<uint32_t>(x);
}

// Count rows (scalar per lane for R <= 16: lane -> rank tid % R; 16-byte
// quads for wider rows: lane -> ranks 4q..4q+3, q = tid % (R/4)) and
// membership pieces, B of each per lane, all loads issued before the first
// sum; indices past the ends are clamped to 0 (valid: the arrays are never
// empty here) and their values dropped.
template <int R, int B>
__device__ __forceinline__ void chan_sums(const int32_t* ntpr, int nq, const uint4* pc, int np, bool half_tail,
                                          int i0, int nthr, int tid, int4& acc, uint32_t (&bsum)[4]) {
  constexpr bool kQuad = R > 16;
  int4 v[B];
  uint4 pv[B];
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int i = i0 + u * nthr + tid;
    if constexpr (kQuad) v[u] = reinterpret_cast<const int4*>(ntpr)[i < nq ? i : 0];
    else v[u].x = ntpr[i < nq ? i : 0];
  }
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int i = i0 + u * nthr + tid;
    pv[u] = pc[i < np ? i : 0];
  }
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int i = i0 + u * nthr + tid;
    const bool okq = i < nq, okp = i < np;
    const bool cut = half_tail && i == np - 1;
    acc.x += okq ? v[u].x : 0;
    if constexpr (kQuad) {
      acc.y += okq ? v[u].y : 0;
      acc.z += okq ? v[u].z : 0;
      acc.w += okq ? v[u].w : 0;
    }
    bsum[0] += okp ? pv[u].x : 0u;
    bsum[1] += okp ? pv[u].y : 0u;
    bsum[2] += okp && !cut ? pv[u].z : 0u;
    bsum[3] += okp && !cut ? pv[u].w : 0u;
  }
}

template <int R, bool HNT>
__global__ __launch_bounds__(256) void notify_chan_kernel(NotifyArgs a, int cpw) {
  constexpr bool kQuad = R > 16;
  constexpr int kCP = kQuad ? R / 4 : R;          // count classes (lanes that agree mod kCP share a rank set)
  constexpr int kWin = R < 16 ? 8 : 16;           // ranks one lane's recount bytes cover
  constexpr int kNWin = R < 16 ? 1 : R / 16;      // recount classes
  __shared__ int32_t cnt_w[kNotifyMaxWaves][R];   // per wavefront: count rows of the summed sources
  __shared__ int32_t pre_w[kNotifyMaxWaves][R];   // per wavefront: member bytes of the earlier channels
  __shared__ int32_t own_w[kNotifyMaxWaves][R];   // per wavefront: its tokens per rank
  __shared__ uint64_t mk[kNotifyMaxWaves][kWave];    // wide rows: token masks, then rank columns
  __shared__ int32_t pk[kNotifyMaxWaves][kWave];     // wide rows: per-rank positions

  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nw = blockDim.x / kWave;
  const int nthr = blockDim.x;
  const int S = a.S, T = a.T, C = a.C;
  const int tc = a.tcdiv.d;
  const int c0 = static_cast<int>(blockIdx.x) * cpw;          // first channel of this workgroup
  const int c1 = c0 + cpw < a.nonempty ? c0 + cpw : a.nonempty;
  const int t0 = c0 * tc;                         // first token
  const int tend = c1 * tc < T ? c1 * tc : T;
  const int n_own = tend - t0;
  const bool first = s == 0 && blockIdx.x == 0;   // also computes the receive offsets and the status
  const int limit = first ? S : s;                // count rows summed (workgroup (0, 0): all, for the totals)
  const int64_t tok0 = static_cast<int64_t>(s) * T;

  // Every load below is unconditional, from a clamped (always valid) index,
  // and masked where it is summed: a load under a branch gets a wait of its
  // own from the compiler, which would serialise the round trips.
  // (1a) this thread's token
  ChanRow<R> cr;
  const bool mine = tid < n_own;
  chan_load_row<R>(a.in_rank + (tok0 + t0 + (mine ? tid : 0)) * R, cr);

  // (1b) owned experts e = b, b + nb, ... (b = workgroup index): lane j
  // loads source j's count of the first kChanEarlyE of them
  const bool do_e = a.nrte != nullptr && a.ntpe != nullptr;
  const int b = s * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
  const int nb = static_cast<int>(gridDim.x * gridDim.y);
  int ev[kChanEarlyE];
  if (do_e) {
    const int jc = lane < S ? lane : S - 1;
#pragma unroll
    for (int k = 0; k < kChanEarlyE; ++k) {
      const int e = b + k * nb;
      ev[k] = a.ntpe[static_cast<int64_t>(jc) * a.E + (e < a.E ? e : a.E - 1)];
    }
  }

  // (1c) count rows of sources < limit (elements, or 16-byte quads, i = tid,
  // tid + nthr, ...; nthr is a multiple of kCP, so the class is tid % kCP);
  // (1d) membership bytes of tokens [0, t0) of s: 16-byte pieces p = tid,
  // tid + nthr, ... (R = 8 with t0 odd: the last piece's second token is not
  // an earlier one)
  const int nq = limit * (kQuad ? R / 4 : R);
  const int64_t pbytes = static_cast<int64_t>(t0) * R;
  const int np = static_cast<int>((pbytes + 15) / 16);
  const bool half_tail = (pbytes & 15) != 0;
  const uint4* pc = reinterpret_cast<const uint4*>(a.in_rank + tok0 * R);
  int4 acc = make_int4(0, 0, 0, 0);
  uint32_t bsum[4] = {0u, 0u, 0u, 0u};
  const int nuq = (nq + nthr - 1) / nthr, nup = (np + nthr - 1) / nthr;
  const int nu = nuq > nup ? nuq : nup;           // loads per lane of the longer kind (wave-uniform)
  if (nu <= 1) {
    chan_sums<R, 1>(a.ntpr, nq, pc, np, half_tail, 0, nthr, tid, acc, bsum);
  } else if (nu <= 4) {
    chan_sums<R, 4>(a.ntpr, nq, pc, np, half_tail, 0, nthr, tid, acc, bsum);
  } else {
    for (int u0 = 0; u0 < nu; u0 += kChanBatch)
      chan_sums<R, kChanBatch>(a.ntpr, nq, pc, np, half_tail, u0 * nthr, nthr, tid, acc, bsum);
  }

  // (2) own tokens: per-wavefront rank counts (and, wide rows, rank columns)
  const uint64_t m = mine ? chan_row_mask<R>(cr) : 0ull;
  uint64_t bal[R <= 8 ? R : 1];                   // R = 8: ballot per rank
  uint64_t col = 0;                               // bit q: token q of the wavefront goes to rank `lane`
  if constexpr (R <= 8) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      bal[j] = ballot(((m >> j) & 1ull) != 0);
      col = lane == j ? bal[j] : col;
    }
  } else {
    mk[w][lane] = m;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const ulonglong2* mw = reinterpret_cast<const ulonglong2*>(&mk[w][0]);
#pragma unroll 8
    for (int q = 0; q < kWave / 2; ++q) {          // broadcast reads, two masks each
      const ulonglong2 pq = mw[q];
      col |= ((pq.x >> lane) & 1ull) << (2 * q);
      col |= ((pq.y >> lane) & 1ull) << (2 * q + 1);
    }
  }
  if (lane < R) own_w[w][lane] = __popcll(col);

  // (3) count rows: class sums; lanes 16 - kCP + j hold class j
  {
    const uint32_t x = class_sum<kCP>(static_cast<uint32_t>(acc.x));
    if constexpr (kQuad) {
      const uint32_t y = class_sum<kCP>(static_cast<uint32_t>(acc.y));
      const uint32_t z = class_sum<kCP>(static_cast<uint32_t>(acc.z));
      const uint32_t ww = class_sum<kCP>(static_cast<uint32_t>(acc.w));
      const int j = lane - (16 - kCP);
      if (j >= 0 && j < kCP) {
        cnt_w[w][4 * j] = static_cast<int32_t>(x);
        cnt_w[w][4 * j + 1] = static_cast<int32_t>(y);
        cnt_w[w][4 * j + 2] = static_cast<int32_t>(z);
        cnt_w[w][4 * j + 3] = static_cast<int32_t>(ww);
      }
    } else {
      const int j = lane - (16 - kCP);
      if (j >= 0 && j < kCP) cnt_w[w][j] = static_cast<int32_t>(x);
    }
  }

  // (4) membership bytes: 16-bit counters (even / odd bytes of each word),
  // class sums over the lanes that share a window
  constexpr int kWords = kWin / 2;
  uint32_t u16[kWords];
  if constexpr (R == 8) {
    const uint32_t f0 = bsum[0] + bsum[2], f1 = bsum[1] + bsum[3];   // bytes j and j + 8 are the same rank
    u16[0] = f0 & 0x00FF00FFu;
    u16[1] = (f0 >> 8) & 0x00FF00FFu;
    u16[2] = f1 & 0x00FF00FFu;
    u16[3] = (f1 >> 8) & 0x00FF00FFu;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u16[2 * i] = bsum[i] & 0x00FF00FFu;
      u16[2 * i + 1] = (bsum[i] >> 8) & 0x00FF00FFu;
    }
  }
#pragma unroll
  for (int i = 0; i < kWords; ++i) u16[i] = class_sum<kNWin>(u16[i]);
  {
    const int j = lane - (16 - kNWin);
    if (j >= 0 && j < kNWin) {
#pragma unroll
      for (int i = 0; i < kWords / 2; ++i) {      // word 2i: ranks 4i, 4i+2; word 2i+1: ranks 4i+1, 4i+3
        int32_t* d = &pre_w[w][kWin * j + 4 * i];
        d[0] = static_cast<int32_t>(u16[2 * i] & 0xFFFFu);
        d[2] = static_cast<int32_t>(u16[2 * i] >> 16);
        d[1] = static_cast<int32_t>(u16[2 * i + 1] & 0xFFFFu);
        d[3] = static_cast<int32_t>(u16[2 * i + 1] >> 16);
      }
    }
  }
  __syncthreads();

  // (5) lane r: rank r's bases
  int cnt = 0, pre = 0, own = 0, wp = 0;
  if (lane < R) {
    for (int q = 0; q < nw; ++q) {
      cnt += cnt_w[q][lane];
      pre += pre_w[q][lane];
      const int o = own_w[q][lane];
      own += o;
      wp += q < w ? o : 0;
    }
  }
  const int base_l = first ? 0 : cnt;             // rows of rank `lane` from sources < s
  const int pos_l = base_l + pre + wp;            // row of this wavefront's first member

  // (6) send_head rows of this wavefront's tokens
  if constexpr (R <= 8) {
    // rank j's position read from lane j with every lane active (inside the
    // branch below, the compiler may compute pos_l only on the active lanes)
    int posj[R];
#pragma unroll
    for (int j = 0; j < R; ++j) posj[j] = readlane(pos_l, j);
    if (mine) {
      int v[R];
#pragma unroll
      for (int j = 0; j < R; ++j) v[j] = ((m >> j) & 1ull) ? posj[j] + __popcll(bal[j] & lanemask_lt()) : -1;
      const int64_t n = tok0 + t0 + tid;
      store_head4<HNT>(a.send_head, n * R, make_int4(v[0], v[1], v[2], v[3]));
      store_head4<HNT>(a.send_head, n * R + 4, make_int4(v[4], v[5], v[6], v[7]));
    }
  } else {
    // lane (tq, j) writes ranks 4j..4j+3 of token q0 + tq: one store
    // instruction covers 64 / (R/4) token rows
    mk[w][lane] = col;
    pk[w][lane] = pos_l;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int kQ = R / 4;
    constexpr int kLg = R == 16 ? 2 : (R == 32 ? 3 : 4);   // log2(R / 4)
    const int tq = lane >> kLg, j = lane & (kQ - 1);
    uint64_t c4[4];
    int p4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c4[k] = mk[w][4 * j + k];
      p4[k] = pk[w][4 * j + k];
    }
    const int tw0 = w * kWave;                    // this wavefront's first token within the workgroup
    const int nqw = n_own - tw0 < kWave ? n_own - tw0 : kWave;
    for (int q0 = 0; q0 < nqw; q0 += kWave / kQ) {
      const int q = q0 + tq;
      if (q < nqw) {
        const uint64_t below = (1ull << q) - 1ull;
        int v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = ((c4[k] >> q) & 1ull) ? p4[k] + __popcll(c4[k] & below) : -1;
        store_head4<HNT>(a.send_head, (tok0 + t0 + tw0 + q) * R + 4 * j, make_int4(v[0], v[1], v[2], v[3]));
      }
    }
  }

  // (7) channel prefixes (inclusive of the channel): one store per rank for
  // every channel that ends on a token of this wavefront
  {
    const int t = t0 + tid;
    const int ch = T <= (1 << 20) ? fdiv(t, a.tcdiv) : t / tc;   // FastDiv is exact below 2^20
    const bool last_in_channel = mine && (t - ch * tc == tc - 1 || t == T - 1);
    const uint64_t clast = ballot(last_in_channel);
    for (uint64_t cl = clast; cl != 0; cl &= cl - 1) {
      const int L = __builtin_ctzll(cl);
      const int cc = readlane(ch, L);
      const uint64_t upto = L == kWave - 1 ? ~0ull : ((2ull << L) - 1);   // tokens 0..L of the wavefront
      if (lane < R) {
        const int inc = pre + wp + __popcll(col & upto);
        a.cpm[(static_cast<int64_t>(s) * R + lane) * C + cc] = inc;
        a.rcpm[(static_cast<int64_t>(lane) * S + s) * C + cc] = base_l + inc;
      }
    }
  }
  // the source's last workgroup: tail channels and the rank prefix
  if (w == 0 && lane < R && c1 == a.nonempty) {
    const int r = lane;
    const int inc = pre + own;
    a.rpm[static_cast<int64_t>(s) * R + r] = base_l + inc;
    for (int cc = c1; cc < C; ++cc) {
      a.cpm[(static_cast<int64_t>(s) * R + r) * C + cc] = inc;
      a.rcpm[(static_cast<int64_t>(r) * S + s) * C + cc] = base_l + inc;
    }
  }
  // receive offsets and the capacity status (workgroup (0, 0): cnt = totals)
  if (first && w == 0) {
    const int v = lane < R ? cnt : 0;
    const int incl = wave_inclusive_scan(v);
    if (lane < R) a.off[lane] = incl - v;
    const int sum = readlane(incl, kWave - 1);
    if (lane == 0) {
      a.off[R] = sum;
      if (a.status != nullptr) {
        const bool over = sum > a.capacity;
        if (!a.status_or) *a.status = over ? kStatusCapacity : 0;
        else if (over) *a.status = kStatusCapacity;
      }
    }
  }
  // (8) per-expert receive counts, rounded up to the alignment
  if (do_e && w == 0) {
    const uint32_t al = static_cast<uint32_t>(a.align);
    for (int k = 0; b + k * nb < a.E; ++k) {
      const int e = b + k * nb;
      int sum = 0;
      if (k < kChanEarlyE) {
#pragma unroll
        for (int kk = 0; kk < kChanEarlyE; ++kk) sum = kk == k && lane < S ? ev[kk] : sum;
      } else if (lane < S) {
        sum = a.ntpe[static_cast<int64_t>(lane) * a.E + e];
      }
      for (int src = kWave + lane; src < S; src += kWave) sum += a.ntpe[static_cast<int64_t>(src) * a.E + e];
      sum = static_cast<int>(class_sum<1>(static_cast<uint32_t>(sum)));
      if (lane == 15) {
        const uint32_t t = static_cast<uint32_t>(sum);
        a.nrte[e] = static_cast<int32_t>(al == 1u ? t : (t + al - 1u) / al * al);
      }
    }
  }
}

__global__ void fill_zero_kernel(int32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if ((n + 255) / 256 > max_blocks(256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

template <bool HNT>
static hipError_t launch_notify_cfg(const NotifyArgs& a, int threads, size_t lds, hipStream_t st) {
  if (a.group_w != 0 && a.R <= 8)   // groups: R <= 32 destinations
    hipLaunchKernelGGL((notify_kernel<1, true, 8, HNT>), dim3(a.S), dim3(threads), lds, st, a);
  else if (a.group_w != 0)
    hipLaunchKernelGGL((notify_kernel<1, true, 64, HNT>), dim3(a.S), dim3(threads), lds, st, a);
  else if (a.R <= 8)
    hipLaunchKernelGGL((notify_kernel<1, false, 8, HNT>), dim3(a.S), dim3(threads), lds, st, a);
  else if (a.R <= 64)
    hipLaunchKernelGGL((notify_kernel<1, false, 64, HNT>), dim3(a.S), dim3(threads), lds, st, a);
  else
    hipLaunchKernelGGL((notify_kernel<4, false, 256, HNT>), dim3(a.S), dim3(threads), lds, st, a);
  return hipGetLastError();
}

// Geometry of the per-channel-group kernel: threads per workgroup and
// channels per workgroup, or {0, 0} where its conditions do not hold (then
// the per-source kernel runs).
struct ChanGeom {
  int threads, cpw;
};
static ChanGeom chan_geom(const NotifyArgs& a) {
  const ChanGeom none{0, 0};
  if (tuning().notify_chan == 0 || a.group_w != 0) return none;
  if (a.R != 8 && a.R != 16 && a.R != 32 && a.R != 64) return none;
  if (a.T <= 0 || a.S <= 0 || a.S > 65535 || (static_cast<int64_t>(a.T) * a.R) % 16 != 0) return none;
  const int tc = a.tcdiv.d;
  if (tc <= 0 || tc > kChanMaxTokens || a.nonempty <= 0) return none;
  if (((reinterpret_cast<uintptr_t>(a.in_rank) | reinterpret_cast<uintptr_t>(a.ntpr) |
        reinterpret_cast<uintptr_t>(a.send_head)) & 15u) != 0)
    return none;
  // whole channels per workgroup: as many as fit in one wavefront (tuning:
  // notify_chan > 0 caps it)
  int cpw = tc <= kWave ? kWave / tc : 1;
  if (tuning().notify_chan > 0 && cpw > tuning().notify_chan) cpw = tuning().notify_chan;
  const int threads = (cpw * tc + kWave - 1) / kWave * kWave;
  const int64_t pieces = static_cast<int64_t>(a.T) * a.R / 16;
  if ((pieces + threads - 1) / threads > kChanMaxPieces) return none;
  return ChanGeom{threads, cpw};
}

template <bool HNT>
static hipError_t launch_notify_chan(const NotifyArgs& a, const ChanGeom& g, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.nonempty + g.cpw - 1) / g.cpw), static_cast<unsigned>(a.S));
  switch (a.R) {
    case 8: hipLaunchKernelGGL((notify_chan_kernel<8, HNT>), grid, dim3(g.threads), 0, st, a, g.cpw); break;
    case 16: hipLaunchKernelGGL((notify_chan_kernel<16, HNT>), grid, dim3(g.threads), 0, st, a, g.cpw); break;
    case 32: hipLaunchKernelGGL((notify_chan_kernel<32, HNT>), grid, dim3(g.threads), 0, st, a, g.cpw); break;
    default: hipLaunchKernelGGL((notify_chan_kernel<64, HNT>), grid, dim3(g.threads), 0, st, a, g.cpw); break;
  }
  return hipGetLastError();
}

hipError_t launch_notify(const NotifyArgs& a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  const int64_t head_bytes = static_cast<int64_t>(a.S) * a.T * a.R * 4;
  const bool hnt = head_bytes > kHeadStreamBytes && head_bytes < (1ll << 31);
  const ChanGeom g = chan_geom(a);
  if (g.threads > 0) return hnt ? launch_notify_chan<true>(a, g, st) : launch_notify_chan<false>(a, g, st);
  int threads = ((a.T + kWave - 1) / kWave) * kWave;
  threads = threads < kWave ? kWave : (threads > kNotifyMaxWaves * kWave ? kNotifyMaxWaves * kWave : threads);
  const int ne_max = (a.E + a.S - 1) / a.S;  // experts owned by workgroup 0 (the most)
  const bool wide = a.R > 8 && a.R <= 64;   // the notify_kernel<1, *, 64> instantiations
  const size_t lds = sizeof(int32_t) * static_cast<size_t>(ne_max > 0 ? ne_max : 1) +
                     (wide ? (sizeof(uint64_t) + sizeof(int32_t)) * static_cast<size_t>(threads) : 0);
  // rows of <= 8 ranks (or groups): one unrolled ballot per rank; wider
  // rows: the LDS bit transpose (measured on the 64-rank workload: 64-rank
  // notify 18.0 -> 15.3 us with it, while 8 groups took 7.3 us with ballots
  // against 11.1 us transposed)
  // streaming send_head stores (buffer offsets are 32 bits: arrays below 2 GiB)
  if (hnt) return launch_notify_cfg<true>(a, threads, lds, st);
  return launch_notify_cfg<false>(a, threads, lds, st);
}

}  // namespace miep
