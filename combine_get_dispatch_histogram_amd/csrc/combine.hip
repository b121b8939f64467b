// combine.hip -- normal-mode combine on gfx950.
//
// "Chapter 4  V1: layout, dispatch and combine", section 4.2: combine uses
// the dispatch handle to send expert outputs back without re-deriving the
// routing; section 4.4: combine only adds the tokens (no gate weights are
// applied in it), and the top-k weights are reduced separately.
// Accumulation is fp32, the result is rounded once to bf16.
//
// Pull design: one wavefront per (token, row slice) gathers the rows that
// the token's receiving ranks hold (send_head names them), adds them in
// ascending rank order in fp32 registers, and writes the bf16 row once.
// Every HBM byte is touched once: rho row reads + 1 row write per token.
// No atomics: a token's sum lives in one wavefront's registers.  Row
// traffic uses buffer instructions on the wave-uniform row base; by default
// the expert outputs stream in non-temporal and the combined rows are
// written at device scope.
//
// Row element types (IO): kBf16 reads bf16 rows and writes bf16 rows;
// kToF32 writes the fp32 sums unrounded (the two-level combine's first
// level with fp32 partials); kFromF32 reads fp32 rows (its second level).
// A lane owns 8 channels: one 16-byte vector of bf16 rows, or with an fp32
// side two 4-channel quads 64 lanes apart (see the kernel).
#include "device.h"
#include "kernels.h"

namespace miep {

enum CombineIO { kBf16 = 0, kToF32 = 1, kFromF32 = 2 };

// 8 channels of an expert-output row -> fp32 (one bf16 vector, or two fp32 vectors)
template <bool IN32>
__device__ __forceinline__ void widen8(const v4u (&d)[2], float (&f)[8]) {
  if constexpr (IN32) {
    f[0] = __uint_as_float(d[0].x); f[1] = __uint_as_float(d[0].y);
    f[2] = __uint_as_float(d[0].z); f[3] = __uint_as_float(d[0].w);
    f[4] = __uint_as_float(d[1].x); f[5] = __uint_as_float(d[1].y);
    f[6] = __uint_as_float(d[1].z); f[7] = __uint_as_float(d[1].w);
  } else {
    f[0] = bf16_lo(d[0].x); f[1] = bf16_hi(d[0].x); f[2] = bf16_lo(d[0].y); f[3] = bf16_hi(d[0].y);
    f[4] = bf16_lo(d[0].z); f[5] = bf16_hi(d[0].z); f[6] = bf16_lo(d[0].w); f[7] = bf16_hi(d[0].w);
  }
}

template <int VPL, int MAXR, int MW, int NT, int IO = kBf16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int nslices) {
  constexpr bool kIn32 = IO == kFromF32;
  constexpr bool kOut32 = IO == kToF32;
  // With an fp32 side the lane's 8 channels are two 4-channel quads 64
  // lanes apart (quads 2*v0 + lane and 2*v0 + 64 + lane), so that every load
  // and store instruction covers one contiguous run (512 B of bf16 or 1 KiB
  // of fp32) instead of half of each 32-byte fp32 piece; the channels a
  // wavefront covers, and each channel's order of additions, are the same.
  constexpr bool kQuads = IO != kBf16;
  const int lane = lane_id();
  const int64_t gw = wave_index();
  const int64_t n = gw / nslices;
  const int slice = static_cast<int>(gw - n * nslices);
  if (n >= a.N) return;
  if (a.count != nullptr && n >= *a.count) return;   // past the group rows
  const int R = a.R;
  // group-level reduction: lane j of row n's group g reads rank g*group_w + j
  int rbase = 0;
  if (a.group_off != nullptr) {
    const bool le = lane <= a.groups && a.group_off[lane] <= n;
    rbase = (__popcll(ballot(le)) - 1) * a.group_w;
  }

  int src[MW];
  uint64_t smask[MW];
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
    src[i] = row;
    smask[i] = ballot(ok);
  }

  const int nv = a.H / 8;  // groups of 8 channels
  const int nq = a.H / 4;  // quads of 4 channels
  const uint8_t* y = reinterpret_cast<const uint8_t*>(a.y);
  const int64_t bf_row_bytes = 2 * static_cast<int64_t>(a.H);
  const int64_t in_row_bytes = (kIn32 ? 4 : 2) * static_cast<int64_t>(a.H);
  uint8_t* orow = reinterpret_cast<uint8_t*>(a.out) + n * (kOut32 ? 4 : 2) * static_cast<int64_t>(a.H);
  const int span = kWave * VPL;
  for (int v0 = slice * span; v0 < nv; v0 += nslices * span) {
    float acc[VPL][8];
    bool have = false;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      uint64_t m = smask[i];
      while (m) {
        // a batch of up to MAXR source rows: every load issued, then the adds
        // in ascending rank order (the order the oracle fixes)
        int64_t rows[MAXR];
        int nb = 0;
#pragma unroll
        for (int q = 0; q < MAXR; ++q) {
          rows[q] = 0;
          if (m) {
            const int b = __builtin_ctzll(m);
            m &= m - 1;
            rows[q] = readlane(src[i], b);
            nb = q + 1;
          }
        }
        v4u d[MAXR][VPL][2];
#pragma unroll
        for (int q = 0; q < MAXR; ++q) {
          if (q < nb) {
            const uint8_t* yrow = y + rows[q] * in_row_bytes;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
              if constexpr (kQuads) {
                const int qa = 2 * (v0 + j * kWave) + lane, qb = qa + kWave;   // this lane's two 4-channel quads
                if constexpr (kIn32) {
                  if (qa < nq) d[q][j][0] = ldb16<load_cpol(NT)>(yrow, static_cast<uint32_t>(qa) * 16);
                  if (qb < nq) d[q][j][1] = ldb16<load_cpol(NT)>(yrow, static_cast<uint32_t>(qb) * 16);
                } else {
                  v2u ha{0u, 0u}, hb{0u, 0u};
                  if (qa < nq) ha = ldb8<load_cpol(NT)>(yrow, static_cast<uint32_t>(qa) * 8);
                  if (qb < nq) hb = ldb8<load_cpol(NT)>(yrow, static_cast<uint32_t>(qb) * 8);
                  d[q][j][0] = v4u{ha.x, ha.y, hb.x, hb.y};
                }
              } else {
                const int v = v0 + j * kWave + lane;
                if (v < nv) d[q][j][0] = ldb16<load_cpol(NT)>(yrow, static_cast<uint32_t>(v) * 16);
              }
            }
          }
        }
#pragma unroll
        for (int q = 0; q < MAXR; ++q) {
          if (q < nb) {
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
              float f[8];
              widen8<kIn32>(d[q][j], f);
#pragma unroll
              for (int k = 0; k < 8; ++k) acc[j][k] = have ? acc[j][k] + f[k] : f[k];
            }
            have = true;
          }
        }
      }
    }
    // bias rows: added after the received contributions, bias_0 then bias_1
    const bool biased = a.bias0 != nullptr || a.bias1 != nullptr;
    if (biased) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int v = v0 + j * kWave + lane;
        const int qa = 2 * (v0 + j * kWave) + lane, qb = qa + kWave;
        if (kQuads ? qa >= nq : v >= nv) continue;
        if (!have) {
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[j][k] = 0.0f;
        }
        for (int b = 0; b < 2; ++b) {
          const uint16_t* bias = b == 0 ? a.bias0 : a.bias1;
          if (bias == nullptr) continue;
          const uint8_t* brow = reinterpret_cast<const uint8_t*>(bias) + n * bf_row_bytes;
          v4u t;
          if constexpr (kQuads) {
            const uint32_t oa = static_cast<uint32_t>(qa) * 8, ob = static_cast<uint32_t>(qb < nq ? qb : qa) * 8;
            const v2u ha = a.bias_nt ? ldb8<kCpolNt>(brow, oa) : ldb8<0>(brow, oa);   // uniform choice
            const v2u hb = a.bias_nt ? ldb8<kCpolNt>(brow, ob) : ldb8<0>(brow, ob);
            t = v4u{ha.x, ha.y, hb.x, hb.y};
          } else {
            const uint32_t ov = static_cast<uint32_t>(v) * 16;
            t = a.bias_nt ? ldb16<kCpolNt>(brow, ov) : ldb16<0>(brow, ov);
          }
          const float f[8] = {bf16_lo(t.x), bf16_hi(t.x), bf16_lo(t.y), bf16_hi(t.y),
                              bf16_lo(t.z), bf16_hi(t.z), bf16_lo(t.w), bf16_hi(t.w)};
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[j][k] += f[k];
        }
      }
      have = true;
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int v = v0 + j * kWave + lane;
      if constexpr (kQuads) {
        const int qa = 2 * (v0 + j * kWave) + lane, qb = qa + kWave;
        if constexpr (kOut32) {
          const v4u o0 = have ? v4u{__float_as_uint(acc[j][0]), __float_as_uint(acc[j][1]), __float_as_uint(acc[j][2]),
                                    __float_as_uint(acc[j][3])}
                              : v4u{0u, 0u, 0u, 0u};
          const v4u o1 = have ? v4u{__float_as_uint(acc[j][4]), __float_as_uint(acc[j][5]), __float_as_uint(acc[j][6]),
                                    __float_as_uint(acc[j][7])}
                              : v4u{0u, 0u, 0u, 0u};
          if (qa < nq) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(qa) * 16, o0);
          if (qb < nq) stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(qb) * 16, o1);
        } else {
          const v2u o0 = have ? v2u{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])} : v2u{0u, 0u};
          const v2u o1 = have ? v2u{pack_bf16x2(acc[j][4], acc[j][5]), pack_bf16x2(acc[j][6], acc[j][7])} : v2u{0u, 0u};
          if (qa < nq) stb8<store_cpol(NT)>(orow, static_cast<uint32_t>(qa) * 8, o0);
          if (qb < nq) stb8<store_cpol(NT)>(orow, static_cast<uint32_t>(qb) * 8, o1);
        }
      } else if (v < nv) {
        {
          v4u o;
          if (have) {
            o.x = pack_bf16x2(acc[j][0], acc[j][1]);
            o.y = pack_bf16x2(acc[j][2], acc[j][3]);
            o.z = pack_bf16x2(acc[j][4], acc[j][5]);
            o.w = pack_bf16x2(acc[j][6], acc[j][7]);
          } else {
            o = v4u{0u, 0u, 0u, 0u};
          }
          stb16<store_cpol(NT)>(orow, static_cast<uint32_t>(v) * 16, o);
        }
      }
    }
  }
  // top-k weights (slice 0): lane k sums its column over the receiving
  // ranks, after the rows, so that these small dependent loads trail the
  // wavefront's row traffic instead of holding it back (measured: normal
  // combine 61.2 -> 60.0 us, 64-rank combine 338 -> 330 us)
  if (slice == 0 && a.out_w != nullptr) {
    float acc = 0.0f;
    bool have = false;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      uint64_t m = smask[i];
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        const int64_t row = readlane(src[i], b);
        if (lane < a.K) {
          const float v = a.w ? a.w[row * a.K + lane] : 0.0f;
          acc = have ? acc + v : v;
        }
        have = true;
      }
    }
    if (lane < a.K) a.out_w[n * a.K + lane] = have ? acc : 0.0f;
  }
}

template <int VPL, int MAXR, int NT, int IO = kBf16>
static hipError_t launch_combine_cfg(const CombineArgs& a, int nslices, hipStream_t st) {
  const int64_t waves = a.N * nslices;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > max_blocks(256)) return hipErrorInvalidConfiguration;
  if (a.R <= 64)
    hipLaunchKernelGGL((combine_kernel<VPL, MAXR, 1, NT, IO>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       a, nslices);
  else
    hipLaunchKernelGGL((combine_kernel<VPL, MAXR, 4, NT, IO>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       a, nslices);
  return hipGetLastError();
}

// The two-level combine with fp32 partials: the relay's cache-policy code
// (non-temporal loads and stores at device scope).  Geometry per level,
// measured on the 64-rank relay (two-level combine 1,217 -> 1,171 us
// against 4 groups per lane with 2 rows in flight for both): the group
// level (bf16 in, fp32 out) 2 channel groups per lane with 4 rows in
// flight, the token level (fp32 in) 1 with 8 rows; ragged rows 8 with 2.
template <int VPL, int MAXR, int IO>
static hipError_t launch_combine_f32_cfg(const CombineArgs& a, int nslices, int nt, hipStream_t st) {
  switch (nt) {
    case 0: return launch_combine_cfg<VPL, MAXR, 0, IO>(a, nslices, st);
    case 1: return launch_combine_cfg<VPL, MAXR, 1, IO>(a, nslices, st);
    case 4: return launch_combine_cfg<VPL, MAXR, 4, IO>(a, nslices, st);
    case 5: return launch_combine_cfg<VPL, MAXR, 5, IO>(a, nslices, st);
    default: return launch_combine_cfg<VPL, MAXR, 7, IO>(a, nslices, st);
  }
}

template <int IO>
static hipError_t launch_combine_f32(const CombineArgs& a, hipStream_t st) {
  const int nv = a.H / 8;
  const bool ragged = nv % kWave != 0;
  const int vpl = ragged ? 8 : (IO == kToF32 ? 2 : 1);
  const int span = vpl * kWave;
  const int nslices = (nv + span - 1) / span;
  const int nt = tuning().combine_nt >= 0 ? tuning().combine_nt & 7 : 7;
  if (ragged) return launch_combine_f32_cfg<8, 2, IO>(a, nslices, nt, st);
  if constexpr (IO == kToF32) return launch_combine_f32_cfg<2, 4, IO>(a, nslices, nt, st);
  else return launch_combine_f32_cfg<1, 8, IO>(a, nslices, nt, st);
}

// (vectors per lane, rows loaded per batch) pairs compiled in; register use
// grows with their product, so large rows-per-batch go with short slices.
template <int NT>
static hipError_t launch_combine_nt(const CombineArgs& a, int vpl, int maxr, int nslices, hipStream_t st) {
  if (vpl == 1) return maxr <= 4 ? launch_combine_cfg<1, 4, NT>(a, nslices, st)
                                 : maxr <= 8 ? launch_combine_cfg<1, 8, NT>(a, nslices, st)
                                             : launch_combine_cfg<1, 16, NT>(a, nslices, st);
  if (vpl == 2) return maxr <= 4 ? launch_combine_cfg<2, 4, NT>(a, nslices, st)
                                 : launch_combine_cfg<2, 8, NT>(a, nslices, st);
  if (vpl == 4) return maxr <= 2 ? launch_combine_cfg<4, 2, NT>(a, nslices, st)
                                 : launch_combine_cfg<4, 4, NT>(a, nslices, st);
  if (vpl == 7) return maxr <= 1 ? launch_combine_cfg<7, 1, NT>(a, nslices, st)
                                 : launch_combine_cfg<7, 2, NT>(a, nslices, st);
  return maxr <= 1 ? launch_combine_cfg<8, 1, NT>(a, nslices, st) : launch_combine_cfg<8, 2, NT>(a, nslices, st);
}

constexpr int64_t kBiasStreamBytes = int64_t(128) << 20;   // half the last-level cache

hipError_t launch_combine(const CombineArgs& a_in, hipStream_t st) {
  if (a_in.N == 0) return hipSuccess;
  CombineArgs a = a_in;
  // bias rows that the last-level cache cannot hold stream in non-temporally
  // (measured on the 16384-token workload, a 235 MB bias: combine with bias
  // 411 -> 376 us, the combine alone 337 us); smaller ones, likely still
  // cached from their producer, keep the default policy (the 59 MB bias of
  // the normal workload: 66 -> 70 us when streamed)
  const int bnt = tuning().bias_nt;
  a.bias_nt = bnt >= 0 ? (bnt != 0) : (a.N * 2 * static_cast<int64_t>(a.H) > kBiasStreamBytes ? 1 : 0);
  if (a.out_f32) return launch_combine_f32<kToF32>(a, st);
  if (a.in_f32) return launch_combine_f32<kFromF32>(a, st);
  const Tuning& tu = tuning();
  const int nv = a.H / 8;
  // default: one 16-byte vector per lane per row and 8 rows' loads in flight
  // (hidden 7168 -> 14 waves per token); ragged rows keep 8 vectors x 2 rows
  // the group-level reduction of the relay (longer per-wavefront prologue:
  // row count and group lookup) moves 4 vectors per lane (measured on the
  // 64-rank relay: two-level combine 909 -> 805 us)
  const int base_vpl = a.group_off != nullptr ? 4 : 1;
  int vpl = tu.combine_vpl > 0 ? tu.combine_vpl : (nv % kWave == 0 ? base_vpl : 8);
  int maxr = tu.combine_maxr > 0 ? tu.combine_maxr : (vpl <= 2 ? 8 : 2);
  const int span = vpl * kWave;
  int nslices = tu.combine_slices > 0 ? tu.combine_slices : (nv + span - 1) / span;
  if (nslices < 1) nslices = 1;
  const int nt = tu.combine_nt >= 0 ? tu.combine_nt & 7 : (a.cpol >= 0 ? a.cpol & 7 : 5);
  switch (nt) {
    case 0: return launch_combine_nt<0>(a, vpl, maxr, nslices, st);
    case 1: return launch_combine_nt<1>(a, vpl, maxr, nslices, st);
    case 2: return launch_combine_nt<2>(a, vpl, maxr, nslices, st);
    case 3: return launch_combine_nt<3>(a, vpl, maxr, nslices, st);
    case 4: return launch_combine_nt<4>(a, vpl, maxr, nslices, st);
    case 6: return launch_combine_nt<6>(a, vpl, maxr, nslices, st);
    case 7: return launch_combine_nt<7>(a, vpl, maxr, nslices, st);
    default: return launch_combine_nt<5>(a, vpl, maxr, nslices, st);
  }
}

}  // namespace miep
