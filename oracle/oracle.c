/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the MoE
 * expert-parallel layout / dispatch / combine core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library: it includes only the C standard library.
 *
 * Every function writes out the plain definition of the result it computes,
 * in the order and notation of the pages it cites:
 *   [Ch4]  "Chapter 4  V1: layout, dispatch and combine"
 *          (bowenzhou.top, repos/deepep/04-v1-dispatch-combine), sections 4.1-4.5
 *   [NvLL] "DeepEP Normal vs Low-Latency dual-mode analysis"
 *          (backyes.github.io, deepepv2 chapter 07_deep_ep_03)
 *   [Phil] "Normal vs Low-Latency: two communication philosophies in
 *          DeepEP V1 / V2 / DeepGEMM" (backyes.github.io, deepepv2 chapter 06_07)
 *
 * Floating point: the pages fix fp32 accumulation for combine and an fp32
 * FP8 scale, so those steps are fp32 here; reference sums for accuracy
 * checks are additionally returned in fp64.
 *
 * Parity pins: every exported function is pinned by the CPU tests against
 * an independent pure-Python brute force on tiny inputs, against invariants
 * the pages fix, and (for the encoders) against exhaustive nearest-value
 * search and library casts.  Readings where the pages are silent are listed
 * beside the function that takes them.
 *
 * Build:  gcc -O2 -std=c11 -shared -fPIC -o liboracle.so oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* ------------------------------------------------------------------------ */
/* Scalar formats                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: a bf16 is the top half of an fp32. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even (plain definition): take the
 * two bf16 neighbours of f (truncation toward zero and the next one away
 * from zero), compare the exact distances in double, and on a tie keep the
 * one whose last mantissa bit is 0.  NaN maps to the canonical quiet NaN
 * with the input's sign; infinities are bf16 values already. */
uint16_t oracle_bf16_round(float f) {
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint16_t lo = (uint16_t)(u >> 16);            /* toward zero          */
    if ((u & 0xFFFFu) == 0) return lo;              /* already a bf16 value */
    uint16_t hi = (uint16_t)(lo + 1);               /* away from zero       */
    double d_lo = fabs((double)f - (double)oracle_bf16_to_f32(lo));
    double d_hi = fabs((double)oracle_bf16_to_f32(hi) - (double)f);
    if (isinf(oracle_bf16_to_f32(hi))) {
        /* hi is the infinity just past the largest finite bf16: the IEEE
         * rule treats it as the value 2^128 for the rounding decision. */
        double two128 = ldexp(1.0, 128);
        d_hi = two128 - fabs((double)f);
    }
    if (d_lo < d_hi) return lo;
    if (d_hi < d_lo) return hi;
    return (lo & 1u) ? hi : lo;                     /* tie: even wins       */
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; the largest finite magnitude is 448 (code 0x7E).
 * Decoding is the format's definition. */
float oracle_e4m3_decode(uint8_t c) {
    int sign = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    float v;
    if (e == 0xF && m == 7) return sign ? -NAN : NAN;
    if (e == 0) v = ldexpf((float)m, -9);                 /* m/8 * 2^-6 */
    else        v = ldexpf((float)(8 + m), e - 7 - 3);    /* (1+m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* fp32 -> E4M3FN with round-to-nearest-even and saturation (the cast the
 * low-latency dispatch applies before sending, [NvLL] low-latency dispatch
 * send loop; the pages name the cast but not its format or rounding, so
 * both are a reading: OCP E4M3FN, the FP8 format of the pages' hardware).
 * Plain definition: the nearest finite E4M3 value to |a| (all 127
 * non-negative finite codes are candidates, so anything beyond 448 lands
 * on 448), ties to the even code, sign copied (so -0 -> 0x80).  Codes of
 * non-negative values are ordered like their values, so a binary search
 * over the code range finds the neighbours. */
uint8_t oracle_e4m3_encode(float a) {
    if (isnan(a)) return 0x7F;
    uint8_t sign = signbit(a) ? 0x80 : 0x00;
    double m = fabs((double)a);
    /* largest code c in [0, 0x7E] with value(c) <= m */
    int lo = 0, hi = 0x7E;
    if (m >= (double)oracle_e4m3_decode(0x7E)) return sign | 0x7E;
    while (lo < hi) {                     /* invariant: value(lo) <= m */
        int mid = (lo + hi + 1) / 2;
        if ((double)oracle_e4m3_decode((uint8_t)mid) <= m) lo = mid; else hi = mid - 1;
    }
    int c0 = lo, c1 = lo + 1;             /* value(c0) <= m < value(c1) */
    double d0 = m - (double)oracle_e4m3_decode((uint8_t)c0);
    double d1 = (double)oracle_e4m3_decode((uint8_t)c1) - m;
    int c;
    if (d0 < d1) c = c0;
    else if (d1 < d0) c = c1;
    else c = (c0 % 2 == 0) ? c0 : c1;
    return sign | (uint8_t)c;
}

/* ------------------------------------------------------------------------ */
/* O6: per-128-channel FP8 quantisation of one bf16 row                      */
/* ------------------------------------------------------------------------ */
/* [NvLL] low-latency dispatch send loop: each token is cast to FP8 with a
 * per-group amax, a scale and an inverse scale, optionally rounded to a
 * power of two ("round_scale"; "UE8M0" stores only the exponent).
 * Readings (pages give only the call, not the formula):
 *   - group = 128 consecutive channels; amax floored at 1e-4;
 *   - plain scales: scale = 448/amax, scale_inv = amax/448 (fp32, correctly
 *     rounded divisions);
 *   - round_scale: scale_inv = 2^e with e = ceil(log2(amax/448)), the
 *     smallest power of two not below amax/448, so |x*scale| <= 448;
 *     scale = 2^-e; the UE8M0 byte is e + 127;
 *   - code = e4m3(x * scale), one fp32 multiply.                          */
#define ORC_FP8_GROUP 128
#define ORC_FP8_MAX 448.0f

static void oracle_fp8_group_scales(float amax, int round_scale, float* scale, float* scale_inv, int* exp_out) {
    if (amax < 1e-4f) amax = 1e-4f;
    if (round_scale) {
        float v = amax / ORC_FP8_MAX;
        int ex;
        double f = frexp((double)v, &ex);     /* v = f * 2^ex, f in [0.5, 1) */
        int e = (f == 0.5) ? ex - 1 : ex;     /* ceil(log2 v)               */
        *scale_inv = ldexpf(1.0f, e);
        *scale = ldexpf(1.0f, -e);
        if (exp_out) *exp_out = e;
    } else {
        *scale = ORC_FP8_MAX / amax;
        *scale_inv = amax / ORC_FP8_MAX;
        if (exp_out) *exp_out = 0;
    }
}

/* Quantise `rows` bf16 rows of H channels (H % 128 == 0).
 * codes [rows][H] u8, scale_inv [rows][H/128] f32, ue8m0 [rows][H/128] u8
 * (ue8m0 only when round_scale; nullable). */
int oracle_fp8_quantize(int64_t rows, int H, const uint16_t* x, int round_scale,
                        uint8_t* codes, float* scale_inv, uint8_t* ue8m0) {
    if (H <= 0 || H % ORC_FP8_GROUP != 0 || rows < 0) return ORC_EINVAL;
    int G = H / ORC_FP8_GROUP;
    for (int64_t i = 0; i < rows; ++i) {
        for (int g = 0; g < G; ++g) {
            const uint16_t* xs = x + i * H + g * ORC_FP8_GROUP;
            float amax = 0.0f;
            for (int h = 0; h < ORC_FP8_GROUP; ++h) {
                float a = fabsf(oracle_bf16_to_f32(xs[h]));
                if (a > amax) amax = a;
            }
            float sc, sci; int e;
            oracle_fp8_group_scales(amax, round_scale, &sc, &sci, &e);
            for (int h = 0; h < ORC_FP8_GROUP; ++h) {
                volatile float p = oracle_bf16_to_f32(xs[h]) * sc;   /* one fp32 multiply */
                codes[i * H + g * ORC_FP8_GROUP + h] = oracle_e4m3_encode(p);
            }
            scale_inv[i * G + g] = sci;
            if (ue8m0 && round_scale) ue8m0[i * G + g] = (uint8_t)(e + 127);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* O1: get_dispatch_layout                                                   */
/* ------------------------------------------------------------------------ */
/* [Ch4] 4.1: from topk_idx compute the tokens per rank, per RDMA rank, per
 * expert and the token-in-rank matrix.  Expert e lives on rank e / (E/R)
 * ([NvLL] low-latency send loop: dst_rank = expert / num_local_experts);
 * a negative entry is skipped (same loop: only dst_expert_idx >= 0 sends);
 * ranks form RDMA groups of 8 GPUs ([NvLL] translate_dst_rdma_rank and the
 * 8-peer NVLink constant).
 * Readings: S source partitions of T tokens each; entries outside [0, E)
 * are ignored like masked ones; a duplicated expert counts once per entry
 * in num_tokens_per_expert but once per token for the rank membership;
 * num_tokens_per_rdma_rank is produced only when R > 8.
 *   topk_idx [S*T][K] i64 -> ntpr [S][R], ntp_rdma [S][R/8] (or NULL),
 *   ntpe [S][E], in_rank [S*T][R] u8 (0/1).                                */
int oracle_layout(int S, int T, int K, int E, int R, const int64_t* topk_idx,
                  int32_t* ntpr, int32_t* ntp_rdma, int32_t* ntpe, uint8_t* in_rank) {
    if (S < 0 || T < 0 || K <= 0 || E <= 0 || R <= 0 || E % R != 0) return ORC_EINVAL;
    if (R > 8 && R % 8 != 0) return ORC_EINVAL;
    const int L = E / R;
    const int G = R > 8 ? R / 8 : 0;
    uint8_t* hit = (uint8_t*)malloc((size_t)R);
    if (!hit) return ORC_EINVAL;
    for (int s = 0; s < S; ++s) {
        for (int r = 0; r < R; ++r) ntpr[s * R + r] = 0;
        for (int e = 0; e < E; ++e) ntpe[s * E + e] = 0;
        for (int g = 0; g < G; ++g) if (ntp_rdma) ntp_rdma[s * G + g] = 0;
        for (int t = 0; t < T; ++t) {
            int64_t n = (int64_t)s * T + t;
            memset(hit, 0, (size_t)R);
            for (int k = 0; k < K; ++k) {
                int64_t e = topk_idx[n * K + k];
                if (e < 0 || e >= E) continue;
                ntpe[s * E + e] += 1;
                hit[e / L] = 1;
            }
            for (int r = 0; r < R; ++r) {
                in_rank[n * R + r] = hit[r];
                ntpr[s * R + r] += hit[r];
            }
            if (ntp_rdma) {
                for (int g = 0; g < G; ++g) {
                    int any = 0;
                    for (int j = 0; j < 8; ++j) any |= hit[g * 8 + j];
                    ntp_rdma[s * G + g] += any;
                }
            }
        }
    }
    free(hit);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Payload of one source row as it travels                                    */
/* ------------------------------------------------------------------------ */
/* x kinds: 0 = bf16 row (2H bytes); 1 = pre-quantised FP8 codes (H bytes)
 * with their fp32 scales; 2 = bf16 input cast to FP8 on the way (O6).   */
#define ORC_X_BF16 0
#define ORC_X_FP8 1
#define ORC_X_BF16_CAST_FP8 2

static int64_t orc_row_bytes(int kind, int H) { return kind == ORC_X_BF16 ? 2LL * H : (int64_t)H; }

/* dst_ue8m0 (nullable, cast kind with round_scale only) receives the
 * exponent byte e + 127 of every power-of-two scale 2^e of the row.        */
static void orc_write_payload(int kind, int H, const void* x, const float* x_scales, int round_scale,
                              int64_t src_row, uint8_t* dst_row, float* dst_scales, uint8_t* dst_ue8m0) {
    const int G = H / ORC_FP8_GROUP;
    if (kind == ORC_X_BF16) {
        memcpy(dst_row, (const uint8_t*)x + src_row * 2LL * H, 2ULL * H);
    } else if (kind == ORC_X_FP8) {
        memcpy(dst_row, (const uint8_t*)x + src_row * (int64_t)H, (size_t)H);
        if (dst_scales) memcpy(dst_scales, x_scales + src_row * G, sizeof(float) * G);
    } else {
        float tmp_scales[1024];
        uint8_t tmp_ue[1024];
        oracle_fp8_quantize(1, H, (const uint16_t*)x + src_row * H, round_scale, dst_row, tmp_scales,
                            round_scale ? tmp_ue : NULL);
        if (dst_scales) memcpy(dst_scales, tmp_scales, sizeof(float) * G);
        if (dst_ue8m0 && round_scale) memcpy(dst_ue8m0, tmp_ue, (size_t)G);
    }
}

/* ------------------------------------------------------------------------ */
/* O2 + O3: notify (prefix matrices) and normal-mode dispatch                 */
/* ------------------------------------------------------------------------ */
/* [Ch4] 4.1: a fresh dispatch takes x, the optional scales, topk_idx,
 * topk_weights and the layout, and returns recv_x, recv_x_scales,
 * recv_topk_idx, recv_topk_weights, the per-expert receive counts, the
 * rank / channel / receive-channel prefix matrices, recv_src_idx and
 * send_head; 4.2: those last ones form the handle, a reverse-routing
 * record.  Channels split a source's tokens into ceil(T/C)-token runs
 * ([NvLL] V2 channel constants: max tokens per channel = ceil_div).
 * Readings (the pages name these arrays but not their conventions):
 *   cnt[s][r][c]  = tokens of source s, channel c, that go to rank r;
 *   cpm[s][r][c]  = sum_{c'<=c} cnt[s][r][c']          (inclusive);
 *   rpm[s][r]     = sum_{s'<=s} sum_c cnt[s'][r][c]      (inclusive);
 *   rcpm[r][s][c] = (s > 0 ? rpm[s-1][r] : 0) + cpm[s][r][c];
 *   rank r receives n_r = rpm[S-1][r] rows, at recv rows
 *     [off[r], off[r] + n_r) with off[r] = sum_{r'<r} n_r' (off[R] = total);
 *   rows are in (source, token) order; send_head[s,t,r] is the row within
 *     rank r's block, or -1; recv_src_idx[row] = t;
 *   recv_topk_idx[row][k] = e - r*L if expert e lives on r, else -1;
 *   recv_topk_weights[row][k] = w if so, else 0;
 *   num_recv_tokens_per_expert[r][l] = ceil(sum_s ntpe[s][r*L+l] / a) * a.
 * With the cast kind and round_scale, recv_x_scales_ue8m0 (nullable)
 * receives each scale's exponent byte e + 127 ([Ch4] 4.3 use_ue8m0: the
 * power-of-two scale kept as its exponent).
 * Rows at or beyond `capacity` are not written (the call reports the
 * total in off[R] so that the caller can detect the overflow).            */
int oracle_dispatch(int S, int T, int H, int K, int E, int R, int C, int align,
                    int x_kind, const void* x, const float* x_scales, int round_scale,
                    const int64_t* topk_idx, const float* topk_weights,
                    const uint8_t* in_rank, const int32_t* ntpe, int64_t capacity,
                    void* recv_x, float* recv_x_scales, uint8_t* recv_x_scales_ue8m0, int32_t* recv_src_idx,
                    int64_t* recv_topk_idx, float* recv_topk_weights,
                    int32_t* num_recv_tokens_per_expert,
                    int32_t* rpm, int32_t* cpm, int32_t* rcpm, int32_t* recv_rank_offset,
                    int32_t* send_head) {
    if (S < 0 || T < 0 || H <= 0 || E <= 0 || R <= 0 || C <= 0 || E % R != 0 || align <= 0) return ORC_EINVAL;
    if (x_kind != ORC_X_BF16 && (H % ORC_FP8_GROUP != 0 || H / ORC_FP8_GROUP > 1024)) return ORC_EINVAL;
    if (recv_x_scales_ue8m0 && !(x_kind == ORC_X_BF16_CAST_FP8 && round_scale)) return ORC_EINVAL;
    const int L = E / R;
    const int tc = (T + C - 1) / C;                   /* tokens per channel */
    const int G = H / ORC_FP8_GROUP;
    const int64_t rb = orc_row_bytes(x_kind, H);

    /* cnt and cpm */
    for (int s = 0; s < S; ++s)
        for (int r = 0; r < R; ++r) {
            int run = 0;
            for (int c = 0; c < C; ++c) {
                int t0 = c * tc, t1 = (c + 1) * tc < T ? (c + 1) * tc : T;
                for (int t = t0; t < t1; ++t) run += in_rank[((int64_t)s * T + t) * R + r];
                cpm[((int64_t)s * R + r) * C + c] = run;
            }
        }
    /* rpm, rcpm */
    for (int r = 0; r < R; ++r) {
        int run = 0;
        for (int s = 0; s < S; ++s) {
            int before = run;
            run += cpm[((int64_t)s * R + r) * C + (C - 1)];
            rpm[s * R + r] = run;
            for (int c = 0; c < C; ++c)
                rcpm[((int64_t)r * S + s) * C + c] = before + cpm[((int64_t)s * R + r) * C + c];
        }
    }
    /* receive offsets */
    recv_rank_offset[0] = 0;
    for (int r = 0; r < R; ++r)
        recv_rank_offset[r + 1] = recv_rank_offset[r] + (S > 0 ? rpm[(S - 1) * R + r] : 0);
    /* per-expert receive counts */
    if (num_recv_tokens_per_expert && ntpe) {
        for (int r = 0; r < R; ++r)
            for (int l = 0; l < L; ++l) {
                int64_t sum = 0;
                for (int s = 0; s < S; ++s) sum += ntpe[(int64_t)s * E + r * L + l];
                num_recv_tokens_per_expert[r * L + l] = (int32_t)((sum + align - 1) / align * align);
            }
    }
    /* placement: rank-major, then source, then token */
    for (int r = 0; r < R; ++r) {
        int row = 0;
        for (int s = 0; s < S; ++s)
            for (int t = 0; t < T; ++t) {
                int64_t n = (int64_t)s * T + t;
                if (!in_rank[n * R + r]) { send_head[n * R + r] = -1; continue; }
                send_head[n * R + r] = row;
                int64_t g = (int64_t)recv_rank_offset[r] + row;
                row++;
                if (g >= capacity) continue;
                orc_write_payload(x_kind, H, x, x_scales, round_scale, n,
                                  (uint8_t*)recv_x + g * rb,
                                  recv_x_scales && x_kind != ORC_X_BF16 ? recv_x_scales + g * G : NULL,
                                  recv_x_scales_ue8m0 ? recv_x_scales_ue8m0 + g * G : NULL);
                recv_src_idx[g] = t;
                if (topk_idx && recv_topk_idx) {
                    for (int k = 0; k < K; ++k) {
                        int64_t e = topk_idx[n * K + k];
                        int mine = e >= 0 && e < E && e / L == r;
                        recv_topk_idx[g * K + k] = mine ? e - (int64_t)r * L : -1;
                        if (topk_weights && recv_topk_weights)
                            recv_topk_weights[g * K + k] = mine ? topk_weights[n * K + k] : 0.0f;
                    }
                }
            }
    }
    return ORC_OK;
}

/* O5: cached dispatch ([Ch4] 4.1, cached branch): with a handle, only x
 * (and its scales) move; the placement is the handle's send_head.         */
int oracle_cached_dispatch(int S, int T, int H, int R, int x_kind, const void* x, const float* x_scales,
                           int round_scale, const int32_t* send_head, const int32_t* recv_rank_offset,
                           int64_t capacity, void* recv_x, float* recv_x_scales, uint8_t* recv_x_scales_ue8m0) {
    if (S < 0 || T < 0 || H <= 0 || R <= 0) return ORC_EINVAL;
    if (x_kind != ORC_X_BF16 && (H % ORC_FP8_GROUP != 0 || H / ORC_FP8_GROUP > 1024)) return ORC_EINVAL;
    if (recv_x_scales_ue8m0 && !(x_kind == ORC_X_BF16_CAST_FP8 && round_scale)) return ORC_EINVAL;
    const int G = H / ORC_FP8_GROUP;
    const int64_t rb = orc_row_bytes(x_kind, H);
    for (int64_t n = 0; n < (int64_t)S * T; ++n)
        for (int r = 0; r < R; ++r) {
            int32_t j = send_head[n * R + r];
            if (j < 0) continue;
            int64_t g = (int64_t)recv_rank_offset[r] + j;
            if (g >= capacity) continue;
            orc_write_payload(x_kind, H, x, x_scales, round_scale, n, (uint8_t*)recv_x + g * rb,
                              recv_x_scales && x_kind != ORC_X_BF16 ? recv_x_scales + g * G : NULL,
                              recv_x_scales_ue8m0 ? recv_x_scales_ue8m0 + g * G : NULL);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* O4: combine                                                               */
/* ------------------------------------------------------------------------ */
/* [Ch4] 4.2: combine reuses the handle to send expert outputs back without
 * re-deriving the routing; 4.4: combine only adds tokens, it does not
 * multiply by the gate weights, which are reduced separately through
 * topk_weights.  Accumulation is fp32, output bf16 (RNE).
 * Reading: contributions are added in ascending rank order, the sum is
 * started from the first contribution (so a lone -0.0 stays -0.0), and a
 * token that no rank received combines to +0.0.
 * [Ch4] 4.2 also unpacks a bias into bias_0 and bias_1 for the combine; the
 * pages give no formula.  Reading: each bias is a [S*T][H] bf16 row per
 * source token added after the received contributions, bias_0 then bias_1,
 * in fp32 (an empty contribution sum counts as +0.0 then).
 *   y [capacity][H] bf16 in the receive layout, w [capacity][K] f32
 *   (nullable), bias0/bias1 [S*T][H] bf16 (nullable)
 *   -> out [S*T][H] bf16, out_w [S*T][K] f32 (nullable),
 *   out_f32 [S*T][H] (nullable): the fp32 sums before the bf16 rounding;
 *   out_f64 [S*T][H] (nullable): the same sums in fp64, for accuracy checks. */
int oracle_combine(int S, int T, int H, int K, int R, const uint16_t* y, const float* w,
                   const uint16_t* bias0, const uint16_t* bias1,
                   const int32_t* send_head, const int32_t* recv_rank_offset, int64_t capacity,
                   uint16_t* out, float* out_w, float* out_f32, double* out_f64) {
    if (S < 0 || T < 0 || H <= 0 || R <= 0 || K < 0) return ORC_EINVAL;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    double* acc64 = (double*)malloc(sizeof(double) * (size_t)H);
    float* wacc = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    if (!acc || !acc64 || !wacc) { free(acc); free(acc64); free(wacc); return ORC_EINVAL; }
    for (int64_t n = 0; n < (int64_t)S * T; ++n) {
        int have = 0;
        for (int r = 0; r < R; ++r) {
            int32_t j = send_head[n * R + r];
            if (j < 0) continue;
            int64_t g = (int64_t)recv_rank_offset[r] + j;
            if (g >= capacity) continue;
            for (int h = 0; h < H; ++h) {
                float v = oracle_bf16_to_f32(y[g * H + h]);
                if (!have) { acc[h] = v; acc64[h] = v; } else { acc[h] += v; acc64[h] += v; }
            }
            for (int k = 0; k < K; ++k) {
                float v = w ? w[g * K + k] : 0.0f;
                if (!have) wacc[k] = v; else wacc[k] += v;
            }
            have = 1;
        }
        const int biased = bias0 != NULL || bias1 != NULL;
        for (int h = 0; h < H; ++h) {
            if (biased) {
                if (!have) { acc[h] = 0.0f; acc64[h] = 0.0; }
                if (bias0) { acc[h] += oracle_bf16_to_f32(bias0[n * H + h]); acc64[h] += oracle_bf16_to_f32(bias0[n * H + h]); }
                if (bias1) { acc[h] += oracle_bf16_to_f32(bias1[n * H + h]); acc64[h] += oracle_bf16_to_f32(bias1[n * H + h]); }
            }
            const int any = have || biased;
            out[n * H + h] = any ? oracle_bf16_round(acc[h]) : 0;
            if (out_f32) out_f32[n * H + h] = any ? acc[h] : 0.0f;
            if (out_f64) out_f64[n * H + h] = any ? acc64[h] : 0.0;
        }
        if (out_w)
            for (int k = 0; k < K; ++k) out_w[n * K + k] = have ? wacc[k] : 0.0f;
    }
    free(acc); free(acc64); free(wacc);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* O7 + O8: low-latency dispatch, send side (messages) and receive side      */
/* ------------------------------------------------------------------------ */
/* [NvLL] low-latency dispatch: each token is cast once (FP8 optional) and
 * one message is sent per top-k expert entry that is >= 0; the receiver
 * keeps messages expert-major: slot (local_expert, src_rank, i) at
 * ((local_expert * R + src_rank) * M + i) messages; the packed output of
 * local expert l starts at row l * R * M.  [Phil] low-latency message
 * format: one int4 header (source token index + 3 reserved ints) then the
 * payload, either H FP8 bytes followed by H/128 fp32 scales, or 2H bf16
 * bytes.  [Ch4] 4.3: the call returns packed_recv_x, its scales, the
 * per-expert counts, the source info and the layout range.
 * Readings: this models the receive side of rank d; S = R source ranks of
 * T <= M tokens; slots within (l, s) go in ascending (token, k) order
 * instead of the atomic arrival order; reserved header ints are 0; the
 * (l, s) blocks are packed in ascending s; layout_range[l][s] =
 * (begin << 32) | count; slots past M are dropped (count capped at M);
 * with use_ue8m0 the scales also come out as exponent bytes (e + 127).
 * Rank masking ([NvLL] low-latency send loop and receive wait: a masked
 * destination is not sent to, a masked source is not waited for): with a
 * mask array [R] (nonzero = masked), nothing travels to rank d if d is
 * masked, and nothing from a masked source s -- its (l, s) blocks hold 0
 * messages.  */
/* The message stride is the header plus payload rounded up to 16 bytes
 * (messages are written in 16-byte pieces); the padding bytes carry no
 * value.  At H % 512 == 0 (FP8) and any H % 8 == 0 (bf16) there is none. */
int64_t oracle_ll_msg_bytes(int H, int use_fp8) {
    const int64_t used = 16 + (use_fp8 ? (int64_t)H + 4LL * (H / ORC_FP8_GROUP) : 2LL * H);
    return (used + 15) / 16 * 16;
}

int oracle_ll_dispatch(int S, int T, int M, int H, int K, int E, int R, int d,
                       const uint16_t* x, const int64_t* topk_idx,
                       int use_fp8, int round_scale, int use_ue8m0,
                       uint8_t* msg_buf, int32_t* msg_count,
                       void* packed_recv_x, float* packed_recv_x_scales, uint8_t* packed_recv_ue8m0,
                       int32_t* packed_recv_src_info, int64_t* packed_recv_layout_range,
                       int32_t* packed_recv_count, int32_t* cumulative_stats, const int32_t* mask) {
    if (S <= 0 || T < 0 || M <= 0 || T > M || H <= 0 || K <= 0 || E <= 0 || R <= 0 || E % R != 0) return ORC_EINVAL;
    if (S != R || d < 0 || d >= R) return ORC_EINVAL;
    if (use_fp8 && H % ORC_FP8_GROUP != 0) return ORC_EINVAL;
    if (use_ue8m0 && !round_scale) return ORC_EINVAL;
    const int L = E / R;
    const int G = H / ORC_FP8_GROUP;
    const int64_t mb = oracle_ll_msg_bytes(H, use_fp8);
    const int64_t pb = use_fp8 ? (int64_t)H : 2LL * H;     /* payload row bytes */
    uint8_t* codes = (uint8_t*)malloc((size_t)H);
    float* sci = (float*)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    uint8_t* ue = (uint8_t*)malloc((size_t)(G > 0 ? G : 1));
    if (!codes || !sci || !ue) { free(codes); free(sci); free(ue); return ORC_EINVAL; }

    /* send side (O7) */
    for (int l = 0; l < L; ++l)
        for (int s = 0; s < S; ++s) {
            int j = 0;
            const int masked = mask != NULL && (mask[d] != 0 || mask[s] != 0);
            for (int t = 0; t < (masked ? 0 : T); ++t)
                for (int k = 0; k < K; ++k) {
                    if (topk_idx[((int64_t)s * T + t) * K + k] != (int64_t)d * L + l) continue;
                    if (j < M) {
                        uint8_t* msg = msg_buf + (((int64_t)l * S + s) * M + j) * mb;
                        int32_t hdr[4] = {t, 0, 0, 0};
                        memcpy(msg, hdr, 16);
                        const uint16_t* xr = x + ((int64_t)s * T + t) * H;
                        if (use_fp8) {
                            oracle_fp8_quantize(1, H, xr, round_scale, codes, sci, ue);
                            memcpy(msg + 16, codes, (size_t)H);
                            memcpy(msg + 16 + H, sci, sizeof(float) * G);
                        } else {
                            memcpy(msg + 16, xr, 2ULL * H);
                        }
                    }
                    j++;
                }
            msg_count[l * S + s] = j < M ? j : M;
        }

    /* receive side (O8) */
    for (int l = 0; l < L; ++l) {
        int begin = 0;
        for (int s = 0; s < S; ++s) {
            int n = msg_count[l * S + s];
            packed_recv_layout_range[l * S + s] = ((int64_t)begin << 32) | (int64_t)(uint32_t)n;
            for (int i = 0; i < n; ++i) {
                const uint8_t* msg = msg_buf + (((int64_t)l * S + s) * M + i) * mb;
                int64_t row = (int64_t)l * S * M + begin + i;
                int32_t hdr[4];
                memcpy(hdr, msg, 16);
                packed_recv_src_info[row] = hdr[0];
                memcpy((uint8_t*)packed_recv_x + row * pb, msg + 16, (size_t)pb);
                if (use_fp8) {
                    memcpy(packed_recv_x_scales + row * G, msg + 16 + H, sizeof(float) * G);
                    if (use_ue8m0 && packed_recv_ue8m0) {
                        for (int g = 0; g < G; ++g) {
                            float v;
                            memcpy(&v, msg + 16 + H + 4 * g, 4);
                            int ex;
                            frexp((double)v, &ex);          /* v = 2^e exactly: frexp gives e+1 */
                            packed_recv_ue8m0[row * G + g] = (uint8_t)(ex - 1 + 127);
                        }
                    }
                }
            }
            begin += n;
        }
        packed_recv_count[l] = begin;
        if (cumulative_stats) cumulative_stats[l] += begin;
    }
    free(codes); free(sci); free(ue);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Low-latency combine                                                        */
/* ------------------------------------------------------------------------ */
/* [Ch4] 4.3 names a low-latency combine beside the low-latency dispatch
 * (with a deferred-receive hook and a zero-copy option) and [NvLL] lists it
 * among the low-latency kernels; neither gives its arithmetic.
 * Reading: it is the reverse of the low-latency dispatch seen from rank d.
 * Every packed row of local expert l that came from source token (s, t)
 * returns to that token.  For each source token, its top-k entries that name
 * one of d's local experts are visited in ascending k; the entry's row is
 * the dispatch's slot rule (the j-th such entry of source s in (token, k)
 * order is row l*S*M + begin(l, s) + j); the row is multiplied by the
 * entry's gate weight when weights are given (one fp32 multiply), else taken
 * as is like the normal combine; contributions are summed in fp32 from the
 * first one and rounded once to bf16; a token with no entry on rank d (or
 * only dropped ones) combines to +0.0.  A row whose src_info does not name
 * the token means the handle does not belong to this routing: error.
 *   y [L][S*M][H] bf16, src_info [L][S*M], layout_range [L][S], topk_idx
 *   [S*T][K], w [S*T][K] (nullable) -> out [S*T][H] bf16, out_f64 (nullable). */
int oracle_ll_combine(int S, int T, int M, int H, int K, int E, int R, int d,
                      const uint16_t* y, const int32_t* src_info, const int64_t* layout_range,
                      const int64_t* topk_idx, const float* w, uint16_t* out, double* out_f64) {
    if (S <= 0 || T < 0 || M <= 0 || T > M || H <= 0 || K <= 0 || E <= 0 || R <= 0 || E % R != 0) return ORC_EINVAL;
    if (S != R || d < 0 || d >= R) return ORC_EINVAL;
    const int L = E / R;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    double* acc64 = (double*)malloc(sizeof(double) * (size_t)H);
    if (!acc || !acc64) { free(acc); free(acc64); return ORC_EINVAL; }
    int rc = ORC_OK;
    for (int s = 0; s < S && rc == ORC_OK; ++s)
        for (int t = 0; t < T && rc == ORC_OK; ++t) {
            const int64_t n = (int64_t)s * T + t;
            int have = 0;
            for (int k = 0; k < K; ++k) {
                const int64_t e = topk_idx[n * K + k];
                if (e < (int64_t)d * L || e >= (int64_t)(d + 1) * L) continue;
                const int l = (int)(e - (int64_t)d * L);
                int64_t j = 0;                                   /* slot of entry (t, k) */
                for (int t2 = 0; t2 < t; ++t2)
                    for (int k2 = 0; k2 < K; ++k2) j += topk_idx[((int64_t)s * T + t2) * K + k2] == e;
                for (int k2 = 0; k2 < k; ++k2) j += topk_idx[n * K + k2] == e;
                const int64_t lr = layout_range[l * S + s];
                const int64_t begin = lr >> 32, cnt = lr & 0xFFFFFFFFLL;
                if (j >= cnt) continue;                          /* dropped at the slot cap, or masked */
                const int64_t row = (int64_t)l * S * M + begin + j;
                if (src_info[row] != t) { rc = ORC_EINVAL; break; }
                const float wk = w ? w[n * K + k] : 1.0f;
                for (int h = 0; h < H; ++h) {
                    const float yv = oracle_bf16_to_f32(y[row * H + h]);
                    const float v = w ? yv * wk : yv;
                    const double v64 = (double)yv * (double)wk;     /* exact product, fp64 reference */
                    if (!have) { acc[h] = v; acc64[h] = v64; } else { acc[h] += v; acc64[h] += v64; }
                }
                have = 1;
            }
            for (int h = 0; h < H; ++h) {
                out[n * H + h] = have ? oracle_bf16_round(acc[h]) : 0;
                if (out_f64) out_f64[n * H + h] = have ? acc64[h] : 0.0;
            }
        }
    free(acc); free(acc64);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Two-level relay: dispatch through one buffer per RDMA group, and the     */
/* two-level combine                                                        */
/* ------------------------------------------------------------------------ */
/* [NvLL] normal-mode internode dispatch: a token crosses the RDMA network
 * once per destination node (RDMA rank = rank / 8, the RDMA rank
 * translation), lands in that node's RDMA receive buffer together with its
 * source metadata (which of the node's 8 NVLink ranks want it), and a
 * forwarder copies it from the RDMA buffer into the NVLink buffer of each
 * of those ranks, from which the receivers fill recv_x.  [Ch4] 4.2: the
 * internode handle adds RDMA / global channel prefixes, rank prefixes and
 * the source metadata.  On one GPU both hops are HBM copies.
 * Readings (the pages give the pipeline, not the layouts):
 *   - group g = ranks 8g..8g+7 (G = R/8 groups); token n goes to group g
 *     when it goes to any of those ranks;
 *   - the RDMA buffer of group g holds one row per such token, in (source,
 *     token) order, at rows [roff[g], roff[g+1]) of one [rdma_capacity]
 *     array; a row carries the payload as it travels (bf16, or E4M3 codes +
 *     fp32 scales: the FP8 cast happens once, before the first hop);
 *     rdma_src_idx[row] = n (source token s*T + t);
 *   - send_rdma_head[n][g] = the row of n within group g's block, or -1;
 *     rdma prefix matrices as O2 with groups in place of ranks:
 *     rdma_cpm[s][g][c], rdma_rpm[s][g], rdma_rcpm[g][s][c];
 *   - the forwarder walks group g's rows in order and appends each to the
 *     receive block of every rank g*8+j whose bit is set, so rank r's rows
 *     are again in (source, token) order (the same recv side as O3);
 *     send_nvl_head[row][j] = the row within rank g*8+j's block, or -1;
 *     recv_src_idx and recv_topk_* as O3.
 * Rows at or past a capacity are not written.                              */
int oracle_relay_dispatch(int S, int T, int H, int K, int E, int R, int C,
                          int x_kind, const void* x, const float* x_scales, int round_scale,
                          const int64_t* topk_idx, const float* topk_weights, const uint8_t* in_rank,
                          int64_t rdma_capacity, void* rdma_x, float* rdma_x_scales, int32_t* rdma_src_idx,
                          int32_t* rdma_rpm, int32_t* rdma_cpm, int32_t* rdma_rcpm, int32_t* recv_rdma_offset,
                          int32_t* send_rdma_head, int32_t* send_nvl_head,
                          int64_t capacity, void* recv_x, float* recv_x_scales, int32_t* recv_src_idx,
                          int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* recv_rank_offset) {
    if (S < 0 || T < 0 || H <= 0 || E <= 0 || R <= 0 || C <= 0 || E % R != 0 || R % 8 != 0) return ORC_EINVAL;
    if (x_kind != ORC_X_BF16 && (H % ORC_FP8_GROUP != 0 || H / ORC_FP8_GROUP > 1024)) return ORC_EINVAL;
    const int L = E / R, NG = R / 8;
    const int tc = (T + C - 1) / C;
    const int G = H / ORC_FP8_GROUP;
    const int64_t rb = orc_row_bytes(x_kind, H);
    const int fp8 = x_kind != ORC_X_BF16;

    /* group membership, counted per (source, group, channel) */
    for (int s = 0; s < S; ++s)
        for (int g = 0; g < NG; ++g) {
            int run = 0;
            for (int c = 0; c < C; ++c) {
                int t0 = c * tc, t1 = (c + 1) * tc < T ? (c + 1) * tc : T;
                for (int t = t0; t < t1; ++t) {
                    int hit = 0;
                    for (int j = 0; j < 8; ++j) hit |= in_rank[((int64_t)s * T + t) * R + g * 8 + j] != 0;
                    run += hit;
                }
                rdma_cpm[((int64_t)s * NG + g) * C + c] = run;
            }
        }
    for (int g = 0; g < NG; ++g) {
        int run = 0;
        for (int s = 0; s < S; ++s) {
            int before = run;
            run += rdma_cpm[((int64_t)s * NG + g) * C + (C - 1)];
            rdma_rpm[s * NG + g] = run;
            for (int c = 0; c < C; ++c)
                rdma_rcpm[((int64_t)g * S + s) * C + c] = before + rdma_cpm[((int64_t)s * NG + g) * C + c];
        }
    }
    recv_rdma_offset[0] = 0;
    for (int g = 0; g < NG; ++g)
        recv_rdma_offset[g + 1] = recv_rdma_offset[g] + (S > 0 ? rdma_rpm[(S - 1) * NG + g] : 0);

    /* first hop: each token once per destination group, cast once */
    for (int g = 0; g < NG; ++g) {
        int row = 0;
        for (int s = 0; s < S; ++s)
            for (int t = 0; t < T; ++t) {
                int64_t n = (int64_t)s * T + t;
                int hit = 0;
                for (int j = 0; j < 8; ++j) hit |= in_rank[n * R + g * 8 + j] != 0;
                if (!hit) { send_rdma_head[n * NG + g] = -1; continue; }
                send_rdma_head[n * NG + g] = row;
                int64_t i = (int64_t)recv_rdma_offset[g] + row;
                row++;
                if (i >= rdma_capacity) continue;
                orc_write_payload(x_kind, H, x, x_scales, round_scale, n, (uint8_t*)rdma_x + i * rb,
                                  fp8 ? rdma_x_scales + i * G : NULL, NULL);
                rdma_src_idx[i] = (int32_t)n;
            }
    }

    /* receive blocks of the final ranks */
    recv_rank_offset[0] = 0;
    for (int r = 0; r < R; ++r) {
        int n_r = 0;
        for (int64_t n = 0; n < (int64_t)S * T; ++n) n_r += in_rank[n * R + r] != 0;
        recv_rank_offset[r + 1] = recv_rank_offset[r] + n_r;
    }

    /* second hop: the forwarder of group g walks its rows in order */
    for (int g = 0; g < NG; ++g) {
        int row_of[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int64_t total = (int64_t)recv_rdma_offset[g + 1] - recv_rdma_offset[g];
        for (int64_t q = 0; q < total; ++q) {
            int64_t i = (int64_t)recv_rdma_offset[g] + q;
            if (i >= rdma_capacity) break;
            int64_t n = rdma_src_idx[i];
            for (int j = 0; j < 8; ++j) {
                int r = g * 8 + j;
                if (!in_rank[n * R + r]) { send_nvl_head[i * 8 + j] = -1; continue; }
                send_nvl_head[i * 8 + j] = row_of[j];
                int64_t dst = (int64_t)recv_rank_offset[r] + row_of[j];
                row_of[j]++;
                if (dst >= capacity) continue;
                memcpy((uint8_t*)recv_x + dst * rb, (const uint8_t*)rdma_x + i * rb, (size_t)rb);
                if (fp8 && recv_x_scales) memcpy(recv_x_scales + dst * G, rdma_x_scales + i * G, sizeof(float) * G);
                recv_src_idx[dst] = (int32_t)(n % T);
                if (topk_idx && recv_topk_idx) {
                    for (int k = 0; k < K; ++k) {
                        int64_t e = topk_idx[n * K + k];
                        int mine = e >= 0 && e < E && e / L == r;
                        recv_topk_idx[dst * K + k] = mine ? e - (int64_t)r * L : -1;
                        if (topk_weights && recv_topk_weights)
                            recv_topk_weights[dst * K + k] = mine ? topk_weights[n * K + k] : 0.0f;
                    }
                }
            }
        }
    }
    return ORC_OK;
}

/* Two-level combine, the reverse of the relay ([NvLL] normal mode: the
 * combine reduces inside the node over NVLink first, then sends one row
 * per node back over RDMA; [Ch4] 4.4: only additions, weights reduced
 * separately).  Readings:
 *   - first level: every RDMA row of group g sums, in fp32 from its first
 *     term, the expert outputs of the group's ranks j ascending with
 *     send_nvl_head[row][j] >= 0, and is rounded to bf16 -- the type a
 *     partial travels in; the top-k weights are summed the same way in fp32;
 *     a row no rank holds is +0.0;
 *   - with partial_f32 the partial rows stay fp32 (no rounding between the
 *     levels): twice the partial bytes, and the result is then one fp32
 *     sum rounded once, like O4's;
 *   - second level: every source token sums, in fp32 from its first term,
 *     its groups' partial rows g ascending (send_rdma_head >= 0), then the
 *     bias rows as in O4, and is rounded once more to bf16; weights as fp32.
 *   y [capacity][H] bf16, w [capacity][K] (nullable) -> rdma_y
 *   [rdma_capacity][H] partials (bf16, or fp32 with partial_f32), rdma_w
 *   (nullable), out [S*T][H] bf16, out_w [S*T][K] (nullable), out_f32
 *   (nullable): the second level's fp32 sums before the last rounding;
 *   out_f64 (nullable): every contribution and bias summed in fp64 without
 *   any intermediate rounding (accuracy reference).                        */
int oracle_relay_combine(int S, int T, int H, int K, int R,
                         const uint16_t* y, const float* w, const uint16_t* bias0, const uint16_t* bias1,
                         int64_t capacity, const int32_t* recv_rank_offset,
                         int64_t rdma_capacity, const int32_t* recv_rdma_offset, const int32_t* send_nvl_head,
                         const int32_t* send_rdma_head, int partial_f32,
                         void* rdma_y, float* rdma_w, uint16_t* out, float* out_w, float* out_f32,
                         double* out_f64) {
    if (S < 0 || T < 0 || H <= 0 || R <= 0 || R % 8 != 0 || K < 0) return ORC_EINVAL;
    uint16_t* py16 = partial_f32 ? NULL : (uint16_t*)rdma_y;
    float* py32 = partial_f32 ? (float*)rdma_y : NULL;
    const int NG = R / 8;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    double* acc64 = (double*)malloc(sizeof(double) * (size_t)H);
    if (!acc || !acc64) { free(acc); free(acc64); return ORC_EINVAL; }
    float wacc[64];
    if (K > 64) { free(acc); free(acc64); return ORC_EINVAL; }

    /* first level: inside each group */
    for (int g = 0; g < NG; ++g)
        for (int64_t i = recv_rdma_offset[g]; i < recv_rdma_offset[g + 1] && i < rdma_capacity; ++i) {
            int have = 0;
            for (int j = 0; j < 8; ++j) {
                int32_t h = send_nvl_head[i * 8 + j];
                if (h < 0) continue;
                int64_t row = (int64_t)recv_rank_offset[g * 8 + j] + h;
                if (row >= capacity) continue;
                for (int c = 0; c < H; ++c) {
                    float v = oracle_bf16_to_f32(y[row * H + c]);
                    acc[c] = have ? acc[c] + v : v;
                }
                if (w) for (int k = 0; k < K; ++k) wacc[k] = have ? wacc[k] + w[row * K + k] : w[row * K + k];
                have = 1;
            }
            for (int c = 0; c < H; ++c) {
                if (py32) py32[i * H + c] = have ? acc[c] : 0.0f;
                else py16[i * H + c] = have ? oracle_bf16_round(acc[c]) : 0;
            }
            if (w && rdma_w) for (int k = 0; k < K; ++k) rdma_w[i * K + k] = have ? wacc[k] : 0.0f;
        }

    /* second level: across groups, per source token */
    for (int64_t n = 0; n < (int64_t)S * T; ++n) {
        int have = 0;
        for (int c = 0; c < H; ++c) acc64[c] = 0.0;
        for (int g = 0; g < NG; ++g) {
            int32_t h = send_rdma_head[n * NG + g];
            if (h < 0) continue;
            int64_t i = (int64_t)recv_rdma_offset[g] + h;
            if (i >= rdma_capacity) continue;
            for (int c = 0; c < H; ++c) {
                float v = py32 ? py32[i * H + c] : oracle_bf16_to_f32(py16[i * H + c]);
                acc[c] = have ? acc[c] + v : v;
            }
            if (w && rdma_w) for (int k = 0; k < K; ++k) wacc[k] = have ? wacc[k] + rdma_w[i * K + k] : rdma_w[i * K + k];
            have = 1;
            if (out_f64) {
                for (int j = 0; j < 8; ++j) {
                    int32_t hh = send_nvl_head[i * 8 + j];
                    if (hh < 0) continue;
                    int64_t row = (int64_t)recv_rank_offset[g * 8 + j] + hh;
                    if (row >= capacity) continue;
                    for (int c = 0; c < H; ++c) acc64[c] += oracle_bf16_to_f32(y[row * H + c]);
                }
            }
        }
        const int biased = bias0 != NULL || bias1 != NULL;
        for (int c = 0; c < H; ++c) {
            if (biased) {
                if (!have) acc[c] = 0.0f;
                if (bias0) { acc[c] += oracle_bf16_to_f32(bias0[n * H + c]); acc64[c] += oracle_bf16_to_f32(bias0[n * H + c]); }
                if (bias1) { acc[c] += oracle_bf16_to_f32(bias1[n * H + c]); acc64[c] += oracle_bf16_to_f32(bias1[n * H + c]); }
            }
            out[n * H + c] = (have || biased) ? oracle_bf16_round(acc[c]) : 0;
            if (out_f32) out_f32[n * H + c] = (have || biased) ? acc[c] : 0.0f;
            if (out_f64) out_f64[n * H + c] = acc64[c];
        }
        if (out_w) for (int k = 0; k < K; ++k) out_w[n * K + k] = (have && w && rdma_w) ? wacc[k] : 0.0f;
    }
    free(acc); free(acc64);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Batch forms of the scalar encoders (for exhaustive tests)                 */
/* ------------------------------------------------------------------------ */
void oracle_e4m3_encode_n(int64_t n, const float* a, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(a[i]);
}
void oracle_e4m3_decode_n(int64_t n, const uint8_t* c, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_bf16_round_n(int64_t n, const float* a, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(a[i]);
}
