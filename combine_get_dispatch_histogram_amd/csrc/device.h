// device.h -- gfx950 (CDNA4) device helpers shared by the miep kernels:
// 64-lane wavefront primitives, 16-byte vector memory access, bf16 and
// OCP E4M3 conversion, and the per-128-channel FP8 scale rule.
//
// The FP8 rule follows the low-latency dispatch of "DeepEP Normal vs
// Low-Latency dual-mode analysis" (send-loop listing: per-group amax ->
// scale / inverse scale, optionally rounded to a power of two, UE8M0).
// The pages give only the call, so the exact steps are a reading:
//   amax floored at 1e-4; plain: scale = 448/amax, scale_inv = amax/448
//   (IEEE-rounded fp32 divisions); round_scale: scale_inv = 2^e with
//   e = ceil(log2(amax/448)) taken from the bits of the quotient.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace miep {

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Uniform broadcast of lane `src` (src must be wave-uniform).
__device__ __forceinline__ int readlane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// floor(n / f.d) for 0 <= n with n * f.d < 2^40 (see FastDiv).
__host__ __device__ __forceinline__ int fdiv(int n, const FastDiv& f) {
  return static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(n)) * f.m) >> 40);
}

// Inclusive scan across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  // every lane active: DPP row shifts by 1, 2, 4 and 8 (lanes shifted in
  // from outside the row read 0) scan each row of 16 lanes, then the row
  // broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and
  // 3) carry the lower rows' totals up; no LDS round trips
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// ---------------------------------------------------------------- memory
// 16-byte vector types and a plain 16-byte load (bias rows, top-k rows).
struct alignas(16) v4u { uint32_t x, y, z, w; };
struct alignas(8) v2u { uint32_t x, y; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }

// Row traffic of the pack, combine and low-latency kernels goes through buffer
// instructions on a wave-uniform row base (the resource lives in scalar
// registers, the lane's byte offset in one VGPR), which also carries the
// cache-policy field of gfx950 vector memory instructions: sc0 and sc1 pick
// the coherence scope, nt marks data that streams through.  Offsets are 32
// bits, so a row holds at most 2^31 bytes.
constexpr int kCpolSc0 = 1, kCpolNt = 2, kCpolSc1 = 16;

// Policy codes of the pack / combine kernels: bit 0 = non-temporal loads,
// bit 1 = non-temporal stores, bit 2 = device-scope (sc1) stores.
__host__ __device__ constexpr int load_cpol(int code) { return (code & 1) ? kCpolNt : 0; }
__host__ __device__ constexpr int store_cpol(int code) {
  return ((code & 2) ? kCpolNt : 0) | ((code & 4) ? kCpolSc1 : 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base) {
  // raw (untyped) access: stride 0, 2^31 - 1 bytes in range, dword 3 as
  // every gfx9-family raw buffer access takes it
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

template <int CPOL>
__device__ __forceinline__ v4u ldb16(const void* base, uint32_t off) {
  const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(base), off, 0, CPOL);
  return v4u{t.x, t.y, t.z, t.w};
}

template <int CPOL>
__device__ __forceinline__ void stb16(void* base, uint32_t off, const v4u& v) {
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(t, row_rsrc(base), off, 0, CPOL);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CPOL>
__device__ __forceinline__ v2u ldb8(const void* base, uint32_t off) {
  const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(row_rsrc(base), off, 0, CPOL);
  return v2u{t.x, t.y};
}

template <int CPOL>
__device__ __forceinline__ void stb8(void* base, uint32_t off, const v2u& v) {
  const u32x2 t = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(t, row_rsrc(base), off, 0, CPOL);
}

// Wavefront index of the calling lane over the grid, computed from
// wave-uniform values only (so the compiler keeps it in scalar registers).
__device__ __forceinline__ int64_t wave_index() {
  return static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) +
         __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 round-to-nearest-even: gfx950 converts natively.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------- E4M3
// Per-group scales.  Returns scale (multiplier) and writes scale_inv.
__device__ __forceinline__ float fp8_scales(float amax, bool round_scale, float* scale_inv) {
  amax = fmaxf(amax, 1e-4f);
  if (round_scale) {
    const uint32_t b = __float_as_uint(amax / 448.0f);
    const int e = static_cast<int>((b >> 23) & 0xFFu) - 127 + ((b & 0x7FFFFFu) != 0u ? 1 : 0);
    *scale_inv = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
  }
  *scale_inv = amax / 448.0f;
  return 448.0f / amax;
}

// Exponent byte (UE8M0) of a power-of-two scale 2^e from fp8_scales with
// round_scale: its biased fp32 exponent field, e + 127 (the sign is 0 and the
// mantissa 0, and e + 127 stays in [1, 254] for every floored amax).
__device__ __forceinline__ uint8_t ue8m0_byte(float pow2_scale) {
  return static_cast<uint8_t>(__float_as_uint(pow2_scale) >> 23);
}

// Max over the 8 lanes that hold one 128-channel group (16 channels each),
// every lane active: DPP quad permutes [1,0,3,2] and [2,3,0,1], then the
// half-row mirror (lane i of each 8 reads lane 7 - i), no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
  return v;
}

// 8 bf16 channels (one 16-byte vector) -> amax of their magnitudes.
__device__ __forceinline__ float absmax8(const v4u& v) {
  float m = fabsf(bf16_lo(v.x));
  m = fmaxf(m, fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fabsf(bf16_lo(v.y)));
  m = fmaxf(m, fabsf(bf16_hi(v.y)));
  m = fmaxf(m, fabsf(bf16_lo(v.z)));
  m = fmaxf(m, fabsf(bf16_hi(v.z)));
  m = fmaxf(m, fabsf(bf16_lo(v.w)));
  m = fmaxf(m, fabsf(bf16_hi(v.w)));
  return m;
}

// Four fp32 -> four E4M3 codes (byte i = value i).  gfx950 converts two
// values per v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even).  Every
// caller feeds finite |v| <= 448 (amax * (448 / amax) rounds to at most
// 448 in fp32), a range where no saturation rule is involved; the parity
// tests compare the codes with the oracle over every bf16 value and over
// millions of scaled products.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

// 8 bf16 channels times `scale` -> 8 E4M3 codes (one fp32 multiply each).
__device__ __forceinline__ v2u cast8(const v4u& v, float scale) {
  v2u r;
  r.x = e4m3x4(bf16_lo(v.x) * scale, bf16_hi(v.x) * scale, bf16_lo(v.y) * scale, bf16_hi(v.y) * scale);
  r.y = e4m3x4(bf16_lo(v.z) * scale, bf16_hi(v.z) * scale, bf16_lo(v.w) * scale, bf16_hi(v.w) * scale);
  return r;
}

// 16 bf16 channels (two adjacent 16-byte vectors) -> 16 E4M3 codes, one
// 16-byte store.
__device__ __forceinline__ v4u cast16(const v4u& a, const v4u& b, float scale) {
  const v2u lo = cast8(a, scale), hi = cast8(b, scale);
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// Rank set of one token (up to 64*MW ranks) held in registers; selects
// instead of dynamic indexing keep it out of scratch memory.
template <int MW>
struct RankMask {
  uint64_t w[MW];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < MW; ++i) w[i] = 0;
  }
  __device__ __forceinline__ void set(int r) {
    const int q = r >> 6;
    const uint64_t b = 1ull << (r & 63);
#pragma unroll
    for (int i = 0; i < MW; ++i) w[i] |= (q == i) ? b : 0ull;
  }
  __device__ __forceinline__ uint32_t get(int r) const {
    const int q = r >> 6;
    uint64_t v = w[0];
#pragma unroll
    for (int i = 1; i < MW; ++i) v = (q == i) ? w[i] : v;
    return static_cast<uint32_t>((v >> (r & 63)) & 1ull);
  }
};

// Membership row (R bytes, nonzero = member) -> RankMask.  All loads of a
// 64-rank chunk are issued before any is consumed (4-byte loads when
// R % 4 == 0 and the row is 4-byte aligned, else bytes for R < 8).
template <int MW>
__device__ __forceinline__ RankMask<MW> load_rank_row(const uint8_t* row, int R) {
  RankMask<MW> m;
  m.clear();
  if ((R & 3) == 0) {
    for (int c0 = 0; c0 < R; c0 += 64) {
      uint32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = c0 + 4 * i < R ? *reinterpret_cast<const uint32_t*>(row + c0 + 4 * i) : 0u;
      uint64_t w = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w |= static_cast<uint64_t>(((v[i] >> (8 * j)) & 0xFFu) != 0u) << (4 * i + j);
      const int q = c0 >> 6;
#pragma unroll
      for (int k = 0; k < MW; ++k) m.w[k] = (k == q) ? w : m.w[k];
    }
  } else {
    uint8_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < R ? row[i] : 0;
    uint64_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= static_cast<uint64_t>(v[i] != 0) << i;
    m.w[0] = w;
  }
  return m;
}

}  // namespace miep
