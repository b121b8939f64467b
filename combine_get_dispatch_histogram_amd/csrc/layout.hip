// layout.hip -- get_dispatch_layout on gfx950.
//
// "Chapter 4  V1: layout, dispatch and combine", section 4.1: the layout
// turns the top-k expert indices into per-rank, per-RDMA-rank and
// per-expert token counts plus the token-in-rank membership matrix.
// Expert e lives on rank e / (E/R) and negative entries are skipped ("DeepEP
// Normal vs Low-Latency dual-mode analysis", low-latency send loop); ranks
// group into RDMA ranks of 8 (same page, RDMA rank translation and the
// 8-peer NVLink constant).
//
// One workgroup owns one source partition, so every count is produced by a
// single workgroup: no global atomics, no zero-fill launch.  Each thread
// reads one token's K indices (16-byte loads), builds the rank bitmask in
// registers (expert -> rank by multiply-shift), writes the membership row
// with 4-byte stores and counts its experts in LDS; rank and RDMA-group
// counts are wavefront ballots, one LDS add per rank per wavefront (integer
// adds, order-independent).
#include "device.h"
#include "kernels.h"

namespace miep {

// 4 mask bits -> 4 bytes of 0/1 (bit i -> byte i): one multiply places bits
// 0..3 at bits 0, 8, 16, 24 (the four partial products occupy disjoint bit
// ranges, so nothing carries).
__device__ __forceinline__ uint32_t bits4_to_bytes(uint32_t b4) { return (b4 * 0x00204081u) & 0x01010101u; }

// Membership row of one token: R bytes, 1 where the rank is in the mask
// (16-byte stores when R % 16 == 0 and the rows are 16-byte aligned).
template <int MW>
__device__ __forceinline__ void store_member_row(uint8_t* out, int R, const RankMask<MW>& m, bool vec16) {
  if (vec16) {
    for (int r0 = 0; r0 < R; r0 += 16) {
      const int q = r0 >> 6;
      uint64_t w = m.w[0];
#pragma unroll
      for (int i = 1; i < MW; ++i) w = (q == i) ? m.w[i] : w;
      const uint32_t b16 = static_cast<uint32_t>(w >> (r0 & 63)) & 0xFFFFu;
      *reinterpret_cast<uint4*>(out + r0) = make_uint4(bits4_to_bytes(b16 & 15u), bits4_to_bytes((b16 >> 4) & 15u),
                                                       bits4_to_bytes((b16 >> 8) & 15u), bits4_to_bytes(b16 >> 12));
    }
  } else if ((R & 3) == 0) {
    for (int r0 = 0; r0 < R; r0 += 4) {
      const uint32_t b = m.get(r0) | (m.get(r0 + 1) << 8) | (m.get(r0 + 2) << 16) | (m.get(r0 + 3) << 24);
      *reinterpret_cast<uint32_t*>(out + r0) = b;
    }
  } else {
    for (int r = 0; r < R; ++r) out[r] = static_cast<uint8_t>(m.get(r));
  }
}

template <int MW>
__global__ __launch_bounds__(1024) void layout_kernel(LayoutArgs a) {
  extern __shared__ int32_t lds[];
  const int G = a.R > 8 ? a.R / 8 : 0;
  int32_t* hist = lds;            // [E]
  int32_t* rcnt = hist + a.E;     // [R]
  int32_t* gcnt = rcnt + a.R;     // [G]
  const int s = blockIdx.x;
  const int lane = lane_id();
  const bool vec = (a.K & 1) == 0 && (reinterpret_cast<uintptr_t>(a.topk_idx) & 15u) == 0;   // 16-byte rows pairs
  const bool vec16 = (a.R & 15) == 0 && (reinterpret_cast<uintptr_t>(a.in_rank) & 15u) == 0;
  // the first 8 top-k entries of this thread's first token: loaded before
  // the LDS clear and its barrier, so that their latency covers both
  const bool pre_ok = vec && a.K >= 8 && static_cast<int>(threadIdx.x) < a.T;
  int64_t pre8[8];
  if (pre_ok) {
    const int64_t* row = a.topk_idx + (static_cast<int64_t>(s) * a.T + threadIdx.x) * a.K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4u v = ld16(row + 2 * j);
      pre8[2 * j] = static_cast<int64_t>((static_cast<uint64_t>(v.y) << 32) | v.x);
      pre8[2 * j + 1] = static_cast<int64_t>((static_cast<uint64_t>(v.w) << 32) | v.z);
    }
  }
  for (int i = threadIdx.x; i < a.E + a.R + G; i += blockDim.x) lds[i] = 0;
  __syncthreads();

  // whole wavefronts walk the tokens (the rank counts below are wavefront
  // ballots, so every lane of a wavefront takes part in each iteration)
  const int tpad = (a.T + kWave - 1) / kWave * kWave;
  RankMask<MW> m_last;                 // this thread's token of the last tile
  m_last.clear();
  int t_last = -1;
  for (int t = threadIdx.x; t < tpad; t += blockDim.x) {
    t_last = t;
    const bool valid = t < a.T;
    const int64_t n = static_cast<int64_t>(s) * a.T + t;
    const int64_t* row = a.topk_idx + n * a.K;
    RankMask<MW> m;
    m.clear();
    if (valid) {
      for (int k0 = 0; k0 < a.K; k0 += 8) {         // 8 entries in flight (16-byte loads when aligned)
        int64_t e8[8];
        if (k0 == 0 && pre_ok && t == static_cast<int>(threadIdx.x)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) e8[j] = pre8[j];
        } else if (k0 + 8 <= a.K && vec) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v4u v = ld16(row + k0 + 2 * j);
            e8[2 * j] = static_cast<int64_t>((static_cast<uint64_t>(v.y) << 32) | v.x);
            e8[2 * j + 1] = static_cast<int64_t>((static_cast<uint64_t>(v.w) << 32) | v.z);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) e8[j] = k0 + j < a.K ? row[k0 + j] : -1;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t e = e8[j];
          if (e < 0 || e >= a.E) continue;            // masked (or out of range)
          atomicAdd(&hist[e], 1);
          m.set(fdiv(static_cast<int>(e), a.Ldiv));
        }
      }
      // the last tile's rows are written after the final barrier, which
      // would otherwise wait for these stores to land
      if (t + static_cast<int>(blockDim.x) < tpad) store_member_row(a.in_rank + n * a.R, a.R, m, vec16);
    }
    m_last = m;
    if (a.R > 8) {
      // rank and RDMA-group counts of wide rows: one LDS add per set bit of
      // the token's rank mask and of its group mask (about rho adds per
      // token instead of one ballot per rank per wavefront)
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        for (uint64_t mm = m.w[i]; mm != 0; mm &= mm - 1) atomicAdd(&rcnt[kWave * i + __builtin_ctzll(mm)], 1);
        // group g (ranks 8g..8g+7) of this word is hit when its byte is nonzero
        uint64_t f = m.w[i];
        f |= f >> 4;
        f |= f >> 2;
        f |= f >> 1;
        uint32_t gm = static_cast<uint32_t>(((f & 0x0101010101010101ull) * 0x0102040810204080ull) >> 56);
        for (; gm != 0; gm &= gm - 1) atomicAdd(&gcnt[8 * i + __builtin_ctz(gm)], 1);
      }
      continue;
    }
    // rank counts of rows of <= 8 ranks: one ballot per rank over the
    // wavefront; lane j adds the wavefront's count for rank j
    for (int r0 = 0; r0 < a.R; r0 += kWave) {
      const int rend = a.R - r0 < kWave ? a.R - r0 : kWave;
      int mine = 0;
      for (int j = 0; j < rend; ++j) {
        const int c = __popcll(ballot(m.get(r0 + j) != 0));
        mine = lane == j ? c : mine;
      }
      if (lane < rend && mine) atomicAdd(&rcnt[r0 + lane], mine);
    }
    if (G) {
      int mine = 0;
      for (int g = 0; g < G; ++g) {
        bool hit = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) hit |= m.get(8 * g + j) != 0;
        const int c = __popcll(ballot(hit));
        mine = lane == (g & (kWave - 1)) ? mine + c : mine;
      }
      if (lane < G && mine) atomicAdd(&gcnt[lane], mine);
    }
  }
  __syncthreads();
  if (t_last >= 0 && t_last < a.T)
    store_member_row(a.in_rank + (static_cast<int64_t>(s) * a.T + t_last) * a.R, a.R, m_last, vec16);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.ntpe[static_cast<int64_t>(s) * a.E + e] = hist[e];
  for (int r = threadIdx.x; r < a.R; r += blockDim.x) a.ntpr[static_cast<int64_t>(s) * a.R + r] = rcnt[r];
  if (a.ntp_rdma)
    for (int g = threadIdx.x; g < G; g += blockDim.x) a.ntp_rdma[static_cast<int64_t>(s) * G + g] = gcnt[g];
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t st) {
  if (a.S == 0) return hipSuccess;
  int threads = ((a.T + kWave - 1) / kWave) * kWave;
  threads = threads < kWave ? kWave : (threads > 1024 ? 1024 : threads);
  const int G = a.R > 8 ? a.R / 8 : 0;
  const size_t lds = sizeof(int32_t) * static_cast<size_t>(a.E + a.R + G);
  if (a.R <= 64)
    hipLaunchKernelGGL(layout_kernel<1>, dim3(a.S), dim3(threads), lds, st, a);
  else
    hipLaunchKernelGGL(layout_kernel<4>, dim3(a.S), dim3(threads), lds, st, a);
  return hipGetLastError();
}

}  // namespace miep
