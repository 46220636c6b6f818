// Device helpers shared by the gfx950 kernels: the hardware-cosine SnakeBeta,
// the anti-aliased activation staged through LDS (act_from_xs, stage_act),
// the bf16 piece split, and the LDS sizes of the conv kernel.
//
// Method: FastVideo API docs "minimax_h3_audio_vae" (MLXMiniMaxH3AudioVAE.decode,
// module overview), diffusers docs "AutoencoderKLMiniMaxH3Audio" (decode).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "mh3a_internal.h"

namespace mh3a {

typedef float v16f __attribute__((ext_vector_type(16)));


__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// SnakeBeta at the 2x rate: u + sin^2(alpha u) / beta, written as
// u + hb (1 - cos(2 alpha u)) with hb = 0.5 / beta. The cosine runs on the
// hardware unit, whose argument is in revolutions: 2 alpha u / (2 pi) =
// u * (alpha / pi), reduced to [-0.5, 0.5] first (exact for |r| < 2^23).
__device__ __forceinline__ float snake_beta(float u, float a_over_pi, float hb) {
    float r = u * a_over_pi;
    r = r - __builtin_rintf(r);
    const float c = __builtin_amdgcn_cosf(r);
    return u + hb * (1.0f - c);
}

// The same SnakeBeta from U = u + hb (the up-sampling FIR's sum started at
// hb instead of 0): the argument is U (alpha / pi) - hb (alpha / pi), its
// fractional part (exact) gives the same cosine, and the result is
// U - hb cos(2 alpha u). Four instructions: fma, fract, cos, fma. `hba` is
// hb * (alpha / pi).
__device__ __forceinline__ float snake_beta_biased(float U, float a_over_pi, float hb, float hba) {
    const float r = __builtin_fmaf(U, a_over_pi, -hba);
    const float c = __builtin_amdgcn_cosf(__builtin_amdgcn_fractf(r));
    return __builtin_fmaf(-hb, c, U);
}

// Make this wave's earlier LDS writes visible to its later LDS reads (the
// producer steps exchange data only within a wave: 32 lanes own a channel).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS row lengths of the activation staging for window width W. The x row
// holds X[n_lo - 6 ...] with room for the two-pair reads. The 2x-rate
// signal is kept as two planes of act_ss_half(W): even slots and odd slots
// (the latter shifted by one), so that both the up pass's pair stores and
// the down pass's tap reads are 8-byte accesses at an 8-byte lane stride
// (no LDS bank conflicts).
__host__ __device__ constexpr int act_xs_len(int W) { return (W + 14 + 3) & ~3; }
__host__ __device__ constexpr int act_ss_half(int W) { return (W + 8 + 3) & ~3; }
__host__ __device__ constexpr int act_ss_len(int W) { return 2 * act_ss_half(W); }

// The resampler taps in registers: even / odd parity up taps (gain folded)
// and the down taps. Loaded once per kernel: they are the same for every
// channel, and loading them next to the input rows would make the first
// use wait for those rows too (vector memory counters retire in order).
struct ActTaps {
    float fe[6], fo[6], fd[12];
};
__device__ __forceinline__ ActTaps load_act_taps(const float* tp) {
    ActTaps t;
#pragma unroll
    for (int e = 0; e < 6; ++e) {
        t.fe[e] = tp[e];
        t.fo[e] = tp[6 + e];
    }
#pragma unroll
    for (int q = 0; q < 12; ++q) t.fd[q] = tp[12 + q];
    return t;
}

// Stage CI channels [ch0, ch0 + CI) of act(x) over input positions
// [n_lo, n_lo + W) into as[CI][W] (zero outside [0, l_in): the conv's zero
// padding). act is the anti-aliased SnakeBeta:
//   X[t] = x[clamp(t, 0, L-1)]                        (replicate edge)
//   u[2t]   = sum_{e=0..5} 2 f[1+2e] X[t+2-e]          (zero-insert, 12-tap FIR,
//   u[2t+1] = sum_{e=0..5} 2 f[2e]   X[t+3-e]           gain 2, crop 15/15)
//   s[m] = SnakeBeta(u[m]),   m in [0, 2L)
//   a[n] = sum_{q=0..11} f[q] s[clamp(2n + q - 5, 0, 2L-1)]   (pad 5 / 6, stride 2)
// `lane32` in [0, 32) and `ci` identify the calling thread: 32 threads of
// one wave own one channel, so the steps synchronize only within the wave.
// `ab` is this thread's channel's (alpha / pi, 0.5 / beta).
// LDS: xs[CI][act_xs_len(W)] holds X[n_lo - 6 ...]; ss[CI][act_ss_len(W)]
// holds slot mm = s[clamp(2 n_lo - 5 + mm)] at index mm + 1; as[CI][W] is
// the result (W even).
//
// Tiles whose window lies inside the sequence (no clamping, no zeroing)
// take the fast path: each thread computes two adjacent pairs from eight X
// values and stores their four s values at once, then two adjacent outputs
// from sixteen s values. Edge tiles take the general path.
//
// PAIRED writes the result in the conv kernel's operand layout instead of
// rows: as[hi][w][p] holds channel 2p + hi, so that one 16-byte LDS read
// gives a matrix-core lane its four K-steps (channels hi, 2 + hi, 4 + hi,
// 6 + hi) at one position.
template <int CI, bool PAIRED = false>
__device__ __forceinline__ void act_from_xs(float* as, float* xs, float* __restrict__ ss, int ch0, int c_in, int l_in,
                                            int n_lo, int W, const ActTaps& f, float2 ab, int ci, int lane32,
                                            int as_stride, int xs_stride) {
    const int ch = ch0 + ci;
    const bool live = ch < c_in;
    const int XS = xs_stride, SH = act_ss_half(W);
    const float hba = ab.x * ab.y;
    float* xrow = xs + ci * XS;
    // slot m of the 2x-rate signal, s[2 n_lo - 5 + m]: even m = 2k at ev[k],
    // odd m = 2k + 1 at od[k + 1]
    float* ev = ss + ci * 2 * SH;
    float* od = ev + SH;
    static_assert(!PAIRED || CI == 8, "paired layout holds 8 channels");
    constexpr int OS = PAIRED ? 4 : 1;  // float stride between positions
    float* arow = PAIRED ? as + (ci & 1) * W * 4 + (ci >> 1) : as + ci * as_stride;
    const float(&fe)[6] = f.fe;
    const float(&fo)[6] = f.fo;
    const float(&fd)[12] = f.fd;
    const bool interior = n_lo - 6 >= 0 && n_lo + W + 8 <= l_in && ch0 + CI <= c_in;

    (void)XS;
    if (interior) {
        // pairs idx, idx + 1 (t' = n_lo - 3 + idx): X[t' - 3 ...] = xrow[idx ...]
        for (int idx = 2 * lane32; idx < W + 6; idx += 64) {
            const float2 x01 = *reinterpret_cast<const float2*>(xrow + idx);
            const float2 x23 = *reinterpret_cast<const float2*>(xrow + idx + 2);
            const float2 x45 = *reinterpret_cast<const float2*>(xrow + idx + 4);
            const float2 x67 = *reinterpret_cast<const float2*>(xrow + idx + 6);
            const float X[8] = {x01.x, x01.y, x23.x, x23.y, x45.x, x45.y, x67.x, x67.y};
            // the sums start at hb (see snake_beta_biased)
            float ue0 = ab.y, uo0 = ab.y, ue1 = ab.y, uo1 = ab.y;
#pragma unroll
            for (int e = 0; e < 6; ++e) {
                ue0 = fmaf(fe[e], X[5 - e], ue0);
                uo0 = fmaf(fo[e], X[6 - e], uo0);
                ue1 = fmaf(fe[e], X[6 - e], ue1);
                uo1 = fmaf(fo[e], X[7 - e], uo1);
            }
            // s[2t'] is slot 2 idx - 1 (od[idx]), s[2t' + 1] slot 2 idx (ev[idx])
            *reinterpret_cast<float2*>(od + idx) = make_float2(snake_beta_biased(ue0, ab.x, ab.y, hba),
                                                               snake_beta_biased(ue1, ab.x, ab.y, hba));
            *reinterpret_cast<float2*>(ev + idx) = make_float2(snake_beta_biased(uo0, ab.x, ab.y, hba),
                                                               snake_beta_biased(uo1, ab.x, ab.y, hba));
        }
        wave_lds_sync();
        // outputs w, w + 1: a[w] = sum_q f[q] slot[2w + q], i.e. f[2j] ev[w + j]
        // and f[2j + 1] od[w + j + 1]; w even, so the reads are 8-byte aligned
        const float2* ev2 = reinterpret_cast<const float2*>(__builtin_assume_aligned(ev, 8));
        const float2* od2 = reinterpret_cast<const float2*>(__builtin_assume_aligned(od, 8));
        for (int w = 2 * lane32; w < W; w += 64) {
            float E[8], O[8];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float2 e2 = ev2[w / 2 + v], o2 = od2[w / 2 + v];
                E[2 * v] = e2.x;
                E[2 * v + 1] = e2.y;
                O[2 * v] = o2.x;
                O[2 * v + 1] = o2.y;
            }
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int q = 0; q < 12; ++q) {
                if (q % 2 == 0) {
                    a0 = fmaf(fd[q], E[q / 2], a0);
                    a1 = fmaf(fd[q], E[q / 2 + 1], a1);
                } else {
                    a0 = fmaf(fd[q], O[(q + 1) / 2], a0);
                    a1 = fmaf(fd[q], O[(q + 1) / 2 + 1], a1);
                }
            }
            if constexpr (PAIRED) {
                arow[w * OS] = a0;
                arow[(w + 1) * OS] = a1;
            } else {
                *reinterpret_cast<float2*>(arow + w) = make_float2(a0, a1);
            }
        }
        return;
    }

    // pairs t' = n_lo - 3 + idx, idx in [0, W + 6): slot 2 idx - 1 (od[idx]) <- s[2t'],
    // slot 2 idx (ev[idx]) <- s[2t' + 1]
    for (int idx = lane32; idx < W + 6; idx += 32) {
        const int tq = n_lo - 3 + idx;
        const int tc = clampi(tq, 0, l_in - 1);
        const float* xv = xrow + (tc - n_lo + 3);  // xv[e] = X[tc - 3 + e]
        float ue = ab.y, uo = ab.y;
#pragma unroll
        for (int e = 0; e < 6; ++e) {
            ue = fmaf(fe[e], xv[5 - e], ue);
            uo = fmaf(fo[e], xv[6 - e], uo);
        }
        float se = snake_beta_biased(ue, ab.x, ab.y, hba);
        float so = snake_beta_biased(uo, ab.x, ab.y, hba);
        if (tq < 0) so = se;
        if (tq >= l_in) se = so;
        od[idx] = se;
        ev[idx] = so;
    }
    wave_lds_sync();
    for (int w = lane32; w < W; w += 32) {
        const int n = n_lo + w;
        float v = 0.0f;
        if (live && n >= 0 && n < l_in) {
#pragma unroll
            for (int q = 0; q < 12; ++q) v = fmaf(fd[q], (q % 2 == 0) ? ev[w + q / 2] : od[w + (q + 1) / 2], v);
        }
        arow[w * OS] = v;
    }
}

// The interior case of act_from_xs (window inside the sequence, every
// channel live) with four up-sampling pairs and four outputs per lane
// instead of two: per sample the lane's LDS traffic drops from about 68 to
// 48 bytes (each x value and each 2x-rate slot is read by fewer lanes) at
// the same multiply-add count. W is a compile-time width with W % 4 == 2,
// so the last pass's extra pairs and outputs stay inside the rows:
// pairs up to W + 5 from x values up to W + 11 (the 2x-rate planes hold
// act_ss_half(W) = W + 10 slots, the x rows act_xs_len(W) = W + 14 loaded
// values), reads of slots up to W + 7, and outputs up to W + 1 (the result
// row aliases the x row). Outputs at W and W + 1 are garbage that no caller
// reads.
template <int W>
__device__ __forceinline__ void act_interior4(float* arow, const float* xrow, float* __restrict__ ev,
                                              float* __restrict__ od, const ActTaps& f, float2 ab, int lane32) {
    static_assert(W % 4 == 2, "W = 2 mod 4");
    static_assert(act_ss_half(W) >= W + 10 && act_xs_len(W) >= W + 12, "rows hold the last pass");
    const float hba = ab.x * ab.y;
    const float(&fe)[6] = f.fe;
    const float(&fo)[6] = f.fo;
    const float(&fd)[12] = f.fd;
    // pairs idx .. idx + 3 (t' = n_lo - 3 + idx): X[t' - 3 ...] = xrow[idx ...]
    for (int idx = 4 * lane32; idx < W + 6; idx += 128) {
        const float4 x0 = *reinterpret_cast<const float4*>(xrow + idx);
        const float4 x1 = *reinterpret_cast<const float4*>(xrow + idx + 4);
        const float2 x2 = *reinterpret_cast<const float2*>(xrow + idx + 8);
        const float X[10] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w, x2.x, x2.y};
        float ue[4], uo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            ue[k] = ab.y;
            uo[k] = ab.y;  // the sums start at hb (see snake_beta_biased)
        }
#pragma unroll
        for (int e = 0; e < 6; ++e)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ue[k] = fmaf(fe[e], X[k + 5 - e], ue[k]);
                uo[k] = fmaf(fo[e], X[k + 6 - e], uo[k]);
            }
        // pair idx + k: s[2t'] at od[idx + k], s[2t' + 1] at ev[idx + k]
        *reinterpret_cast<float4*>(od + idx) =
            make_float4(snake_beta_biased(ue[0], ab.x, ab.y, hba), snake_beta_biased(ue[1], ab.x, ab.y, hba),
                        snake_beta_biased(ue[2], ab.x, ab.y, hba), snake_beta_biased(ue[3], ab.x, ab.y, hba));
        *reinterpret_cast<float4*>(ev + idx) =
            make_float4(snake_beta_biased(uo[0], ab.x, ab.y, hba), snake_beta_biased(uo[1], ab.x, ab.y, hba),
                        snake_beta_biased(uo[2], ab.x, ab.y, hba), snake_beta_biased(uo[3], ab.x, ab.y, hba));
    }
    wave_lds_sync();
    // outputs w .. w + 3: a[w] = sum_j f[2j] ev[w + j] + f[2j + 1] od[w + j + 1]
    for (int w = 4 * lane32; w < W; w += 128) {
        const float4 e0 = *reinterpret_cast<const float4*>(ev + w);
        const float4 e1 = *reinterpret_cast<const float4*>(ev + w + 4);
        const float e2 = ev[w + 8];
        const float4 o0 = *reinterpret_cast<const float4*>(od + w);
        const float4 o1 = *reinterpret_cast<const float4*>(od + w + 4);
        const float2 o2 = *reinterpret_cast<const float2*>(od + w + 8);
        const float E[9] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w, e2};
        const float O[10] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w, o2.x, o2.y};
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 6; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[k] = fmaf(fd[2 * j], E[k + j], acc[k]);
                acc[k] = fmaf(fd[2 * j + 1], O[k + j + 1], acc[k]);
            }
        *reinterpret_cast<float4*>(arow + w) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// Load X[n_lo - 6 ...] (replicate-clamped) for channel ch0 + ci into xs and
// run act_from_xs into rows of `as` (stride as_stride; `as` may be xs itself
// with stride act_xs_len(W): a channel's x row is dead once its up pass is
// done, and each channel's rows belong to one wave).
// The row is loaded into registers with every load in flight at once (a
// loop of load-then-store would wait one memory latency per element).
template <int CI, int W, int P = 2>
__device__ __forceinline__ void stage_act(float* as, float* xs, float* __restrict__ ss, const float* __restrict__ xb,
                                          int ch0, int c_in, int l_in, int n_lo, const ActTaps& f,
                                          const float2* abp, int ci, int lane32, int as_stride) {
    constexpr int XL = act_xs_len(W);
    constexpr int NR = (XL + 31) / 32;
    const int ch = ch0 + ci;
    const bool live = ch < c_in;
    const float* xc = xb + (int64_t)(live ? ch : 0) * l_in;
    const float2 ab = live ? abp[ch] : make_float2(0.0f, 0.0f);
    float* xrow = xs + ci * XL;
    float v[NR];
    if (n_lo - 6 >= 0 && n_lo - 6 + 32 * NR <= l_in) {
        // every load inside the row: one address, the loads at immediate offsets
        const float* p = xc + (n_lo - 6 + lane32);
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = p[32 * r];
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = xc[clampi(n_lo - 6 + lane32 + 32 * r, 0, l_in - 1)];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int w = lane32 + 32 * r;
        if (w < XL) xrow[w] = live ? v[r] : 0.0f;
    }
    wave_lds_sync();
    if constexpr (P == 4) {
        // (the interior test of act_from_xs)
        if (n_lo - 6 >= 0 && n_lo + W + 8 <= l_in && ch0 + CI <= c_in) {
            float* ev = ss + ci * 2 * act_ss_half(W);
            act_interior4<W>(as + ci * as_stride, xrow, ev, ev + act_ss_half(W), f, ab, lane32);
            return;
        }
    }
    act_from_xs<CI>(as, xs, ss, ch0, c_in, l_in, n_lo, W, f, ab, ci, lane32, as_stride, XL);
}

__device__ __forceinline__ float round_bf16(float v) {
    // round to nearest even at bfloat16 precision, kept in an fp32 register
    unsigned u = __float_as_uint(v);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return __uint_as_float(u);
}

// bf16(v) rounded to nearest even, as raw bits: one v_cvt_pk_bf16_f32 on
// gfx950 (the same bits as (u + 0x7fff + ((u >> 16) & 1)) >> 16 for finite v).
__device__ __forceinline__ unsigned bf16_bits(float v) {
    return __builtin_bit_cast(unsigned short, (__bf16)v);
}
// bf16(a) | bf16(b) << 16, both rounded to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned bf16x2_bits(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf2));
}
// The three bf16 pieces of 8 values (see split3_bf16) as three 16-byte
// groups, g[p] = piece p of v[0..7]; channel pairs share each conversion.
__device__ __forceinline__ void split3_pack8(const float (&v)[8], uint4 (&g)[3]) {
    unsigned w[3][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float a = v[2 * k], b = v[2 * k + 1];
        unsigned p = bf16x2_bits(a, b);
        w[0][k] = p;
        a -= __uint_as_float(p << 16);
        b -= __uint_as_float(p & 0xffff0000u);
        p = bf16x2_bits(a, b);
        w[1][k] = p;
        a -= __uint_as_float(p << 16);
        b -= __uint_as_float(p & 0xffff0000u);
        w[2][k] = bf16x2_bits(a, b);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) g[p] = make_uint4(w[p][0], w[p][1], w[p][2], w[p][3]);
}
// The two fp16 pieces of 8 values as two 16-byte groups: g[0] = fp16(v),
// g[1] = fp16(v - fp16(v)) (round to nearest even; the difference is exact
// in fp32). v0 + v1 equals v to about 2^-22 relative for |v| >= 2^-3 and to
// 2^-25 absolute below (the second piece is then subnormal); |v| must stay
// below the fp16 range, 65504.
__device__ __forceinline__ void split2h_pack8(const float (&v)[8], uint4 (&g)[2]) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    unsigned w[2][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f2 x = {v[2 * k], v[2 * k + 1]};
        const h2 p0 = __builtin_convertvector(x, h2);
        const f2 back = __builtin_convertvector(p0, f2);
        const f2 r = {x.x - back.x, x.y - back.y};
        const h2 p1 = __builtin_convertvector(r, h2);
        w[0][k] = __builtin_bit_cast(unsigned, p0);
        w[1][k] = __builtin_bit_cast(unsigned, p1);
    }
    g[0] = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
    g[1] = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
}
// Pieces of 8 values in form PC (kPieces: bf16 x 3; kPiecesH: fp16 x 2).
template <int PC>
__device__ __forceinline__ void split_pack8(const float (&v)[8], uint4 (&g)[PC]) {
    if constexpr (PC == kPieces) {
        split3_pack8(v, g);
    } else {
        static_assert(PC == kPiecesH, "piece forms: bf16 x 3 or fp16 x 2");
        split2h_pack8(v, g);
    }
}
// The three bf16 pieces of v (raw bits): v0 = bf16(v), v1 = bf16(v - v0),
// v2 = bf16(v - v0 - v1); both differences are exact in fp32.
__device__ __forceinline__ void split3_bf16(float v, unsigned& p0, unsigned& p1, unsigned& p2) {
    p0 = bf16_bits(v);
    const float r1 = v - __uint_as_float(p0 << 16);
    p1 = bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(p1 << 16);
    p2 = bf16_bits(r2);
}

// Word 3 of a buffer resource for raw dword access on gfx9-family chips
// (data format 32, no swizzle), and the largest batch-item slice (floats)
// whose byte offsets a buffer instruction takes without overflow.
constexpr int kBufferWord3 = 0x00020000;
// Slots of the split-product conv's weight register ring (weights load
// kWeightRing - 1 slot pairs ahead of their products).
#ifndef MH3A_WEIGHT_RING
#define MH3A_WEIGHT_RING 4
#endif
constexpr int kWeightRing = MH3A_WEIGHT_RING;
constexpr int64_t kEpiMaxSlice = (int64_t)1 << 29;

// LDS floats of the conv kernel for window width W: the double-buffered
// operand window, the activation staging (act only) and 64 floats per
// producer wave that the epilogue line touches write into (never read).
constexpr int kTouchFloats = 4 * 64;
__host__ __device__ constexpr int conv_lds_floats(int W, bool act) {
    return 2 * kChunk * W + (act ? kChunk * act_xs_len(W) + kChunk * act_ss_len(W) : 0) + kTouchFloats;
}
// Split-product convs: per item kPieces planes of PS positions (16 bytes
// each), PS sized for the largest dilation so that plane offsets are
// compile-time constants.
__host__ __device__ constexpr int bx6_plane(int nwg, int taps, int dmax = kBx6MaxDil) { return nwg + (taps - 1) * dmax; }
__host__ __device__ constexpr int conv_lds_floats6(int nwg, int taps, int dmax = kBx6MaxDil, int planes = kPieces) {
    return 2 * bx6_cpi(nwg, taps, dmax, planes) * planes * bx6_plane(nwg, taps, dmax) * 4 + kTouchFloats;  // two items
}

}  // namespace mh3a
