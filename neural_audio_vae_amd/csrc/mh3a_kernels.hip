// gfx950 kernels of the BigVGAN decode path.
//
// conv_kernel: implicit-GEMM 1-D convolution on the fp32 matrix cores
//   (v_mfma_f32_32x32x2f32, fp32 accumulation). The GEMM is
//   M = output channels, N = output positions, K = (input channel, tap).
//   K is walked in chunks of kChunk input channels; each chunk's input
//   window (tile width + dilated kernel span) is staged in LDS, optionally
//   through the anti-aliased SnakeBeta (2x up-sample, SnakeBeta, 2x
//   low-pass down-sample), so the 2x-rate signal lives only in LDS. The
//   weights stream from L2 in an order packed at create time so that every
//   lane reads 16 contiguous bytes per 4 K-steps. The epilogue fuses bias,
//   residual add, the running AMP-block sum and the 1/num_blocks scale.
//   The same kernel runs the transposed convolutions as polyphase convs
//   (one weight set per output phase, output stride = rate).
//
// act_kernel: the anti-aliased SnakeBeta alone, (B, C, L) rows -> the packed
//   operand layout, for AMP convs that take their activated input from
//   memory (their producer waves then copy it to LDS with no arithmetic).
//
// final_kernel: activation_post + conv_post (C -> 1, k = 7, pad 3) + clamp.
//
// Method: FastVideo API docs "minimax_h3_audio_vae" (MLXMiniMaxH3AudioVAE.decode,
// module overview), diffusers docs "AutoencoderKLMiniMaxH3Audio" (decode).

#include <hip/hip_runtime.h>

#include <algorithm>

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
                                            int as_stride) {
    const int ch = ch0 + ci;
    const bool live = ch < c_in;
    const int XS = act_xs_len(W), SH = act_ss_half(W);
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
            float ue0 = 0.f, uo0 = 0.f, ue1 = 0.f, uo1 = 0.f;
#pragma unroll
            for (int e = 0; e < 6; ++e) {
                ue0 = fmaf(fe[e], X[5 - e], ue0);
                uo0 = fmaf(fo[e], X[6 - e], uo0);
                ue1 = fmaf(fe[e], X[6 - e], ue1);
                uo1 = fmaf(fo[e], X[7 - e], uo1);
            }
            // s[2t'] is slot 2 idx - 1 (od[idx]), s[2t' + 1] slot 2 idx (ev[idx])
            *reinterpret_cast<float2*>(od + idx) = make_float2(snake_beta(ue0, ab.x, ab.y), snake_beta(ue1, ab.x, ab.y));
            *reinterpret_cast<float2*>(ev + idx) = make_float2(snake_beta(uo0, ab.x, ab.y), snake_beta(uo1, ab.x, ab.y));
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
        float ue = 0.0f, uo = 0.0f;
#pragma unroll
        for (int e = 0; e < 6; ++e) {
            ue = fmaf(fe[e], xv[5 - e], ue);
            uo = fmaf(fo[e], xv[6 - e], uo);
        }
        float se = snake_beta(ue, ab.x, ab.y);
        float so = snake_beta(uo, ab.x, ab.y);
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

// Load X[n_lo - 6 ...] (replicate-clamped) for channel ch0 + ci into xs and
// run act_from_xs into rows of `as` (stride as_stride; `as` may be xs itself
// with stride act_xs_len(W): a channel's x row is dead once its up pass is
// done, and each channel's rows belong to one wave).
// The row is loaded into registers with every load in flight at once (a
// loop of load-then-store would wait one memory latency per element).
template <int CI, int W>
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
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = xc[clampi(n_lo - 6 + lane32 + 32 * r, 0, l_in - 1)];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int w = lane32 + 32 * r;
        if (w < XL) xrow[w] = live ? v[r] : 0.0f;
    }
    wave_lds_sync();
    act_from_xs<CI>(as, xs, ss, ch0, c_in, l_in, n_lo, W, f, ab, ci, lane32, as_stride);
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
// The three bf16 pieces of v (raw bits): v0 = bf16(v), v1 = bf16(v - v0),
// v2 = bf16(v - v0 - v1); both differences are exact in fp32.
__device__ __forceinline__ void split3_bf16(float v, unsigned& p0, unsigned& p1, unsigned& p2) {
    p0 = bf16_bits(v);
    const float r1 = v - __uint_as_float(p0 << 16);
    p1 = bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(p1 << 16);
    p2 = bf16_bits(r2);
}

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
__host__ __device__ constexpr int conv_lds_floats6(int nwg, int taps, int dmax = kBx6MaxDil) {
    return 2 * bx6_cpi(nwg, taps, dmax) * kPieces * bx6_plane(nwg, taps, dmax) * 4 + kTouchFloats;  // two item buffers
}

// Wave-specialized, persistent implicit-GEMM conv. 512 threads: waves 0-3
// are the consumers (matrix-core loop, WM x WN of them, each MBW x NBW
// blocks of 32 x 32 outputs); waves 4-7 are the producers. A workgroup owns
// a contiguous range of output tiles and walks the (tile, K-chunk) items of
// that range as one pipeline: while the consumers multiply item i, the
// producers stage item i + 1 (the next chunk, or the first chunk of the next
// tile) into the other half of a double-buffered LDS window, so the
// epilogue of one tile overlaps the staging of the next. One workgroup
// barrier per item hands the buffers over.
//
// RB = 16 selects 16 x 16 blocks on v_mfma_f32_16x16x4f32 (MBW = WM = 1):
// for AMP convs of at most 16 output channels a 32-row block would be half
// or three quarters padding.
//
// PREC selects the products: 0 fp32 matrix cores; 1 the bf16 operand
// variant (three-term split on fp32 matrix cores); 2 split products on bf16
// matrix cores (packed input in the split-product form, see kPieces); 3 the
// bf16 operand variant on bf16 matrix cores (pieces 0 and 1 only, the three
// products w0 x0, w0 x1, w1 x0: the numerics of PREC 1).
//
// DMAX bounds the dilation of a split-product conv (its LDS planes hold
// NWG + (TAPS - 1) DMAX positions).
template <int MBW, int NBW, int WM, int WN, bool ACT, int PREC, int TAPS, int RB = 32, int DMAX = kBx6MaxDil>
// (fp32 tiles of at most 2 x 2 blocks per wave keep two workgroups per CU: <= 128 VGPRs)
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu((MBW * NBW <= 4 && PREC < 2) ? 4 : 1)))
conv_kernel(ConvArgs a) {
    constexpr bool BF16 = PREC == 1;
    constexpr bool BX6 = PREC >= 2;            // bf16 matrix cores on the pieces
    constexpr int NPROD = PREC == 3 ? 3 : 6;   // piece products per pair
    constexpr int NPA = PREC == 3 ? 2 : kPieces;  // weight / activation pieces used
    static_assert(WM * WN == 4, "four consumer waves");
    static_assert(RB == 32 || (RB == 16 && MBW == 1 && WM == 1 && TAPS > 0 && !BF16), "16-row tiles");
    constexpr int CI = kChunk;
    // AMP convs without the fused activation (compile-time taps) read the
    // packed activated input; other plain convs read rows.
    constexpr bool PK = !ACT && TAPS > 0;
    static_assert(!BX6 || (PK && RB == 32), "split products read the packed input");
    constexpr int NWG = WN * NBW * RB;
    constexpr int MWG = WM * MBW * RB;
    constexpr int PS6 = bx6_plane(NWG, TAPS > 0 ? TAPS : 1, DMAX);  // split-product plane stride (positions)
    // an item is CPI chunks (split products: two, so that each barrier hands
    // over as much matrix-core work as an fp32 item)
    constexpr int CPI = BX6 ? bx6_cpi(NWG, TAPS, DMAX) : 1;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool producer = wave >= 4;
    const int W = NWG + (a.taps - 1) * a.dil;
    // one item's operand window: [CI][W] floats, or kPieces planes of PS6 16-byte groups
    const int ABUF = BX6 ? CPI * kPieces * PS6 * 4 : CI * W;
    float* abuf = lds;                       // [2][ABUF]
    float* xs = lds + 2 * CI * W;            // [CI][act_xs_len(W)]   (act only)
    float* ss = xs + CI * act_xs_len(W);     // [CI][act_ss_len(W)]   (act only)
    float* touch = lds + (BX6 ? 2 * ABUF : conv_lds_floats(W, ACT) - kTouchFloats);  // [4][64], write-only
    const int nch = (a.c_in + CI - 1) / CI;
    const int G = nch * a.taps;
    // With a K split the chunks are cut into ksplit equal ranges; each
    // (range, tile) pair is a virtual tile whose raw sums go to `partial`.
    const int nchs = nch / a.ksplit;
    const int ipt = nchs / CPI;  // items per tile
    const int n_nt = (a.positions + NWG - 1) / NWG;
    const int n_mt = (a.c_out + MWG - 1) / MWG;
    const int base_tiles = n_nt * n_mt * a.groups;
    const int total = base_tiles * a.ksplit;
    const int t_begin = (int)((int64_t)total * blockIdx.x / gridDim.x);
    const int t_end = (int)((int64_t)total * (blockIdx.x + 1) / gridDim.x);
    const int n_items = (t_end - t_begin) * ipt;
    if (n_items == 0) return;

    // virtual tile id -> (K range, batch item, phase, M tile, N tile); N tiles
    // vary fastest, K ranges slowest
    struct Tile {
        int b, ph, mt, p0, c0, vid, n_lo;  // n_lo: first input position of the window
    };
    auto tile_at = [&](int id) {
        const int split = a.ksplit > 1 ? id / base_tiles : 0;
        const int bid = id - split * base_tiles;
        const int nt = bid % n_nt;
        const int rest = bid / n_nt;
        const int mt = rest % n_mt;
        const int g = rest / n_mt;
        const int ph = g % a.phases;
        return Tile{g / a.phases, ph, mt, nt * NWG, split * nchs, id, nt * NWG + a.in_off[ph]};
    };

    // producer identity: 256 threads, 32 per channel
    const int ptid = tid - 256;
    const int pci = ptid >> 5, plane = ptid & 31;
    // An item's input row for this thread's channel: with the activation
    // X[n_lo - 6 ...] over act_xs_len(W) (replicate-clamped), without it
    // x[n_lo ...] over W (zero outside). Rows of up to 32 * XR values are
    // prefetched into registers one item ahead; longer rows load directly.
    constexpr int XR = (NWG + 64 + 16 + 31) / 32;
    const int row_len = ACT ? act_xs_len(W) : W;
    const bool prefetchable = row_len <= 32 * XR;
    float xr[XR];
    float2 ab_pf = make_float2(0.0f, 0.0f);  // prefetched (alpha / pi, 0.5 / beta) of the row's channel
    float2 ab_st = ab_pf;                    // that of the staged row
    auto row_value = [&](const Tile& t, int c, int w) {
        const int ch = (t.c0 + c) * CI + pci;
        if (ch >= a.c_in) return 0.0f;
        const float* xc = a.x + (int64_t)t.b * a.x_bstride + (int64_t)ch * a.l_in;
        if constexpr (ACT) {
            return xc[clampi(t.n_lo - 6 + w, 0, a.l_in - 1)];
        } else {
            const int n = t.n_lo + w;
            return (n >= 0 && n < a.l_in) ? xc[n] : 0.0f;
        }
    };
    // Branch-free row prefetch: every load is issued, from a clamped (in
    // bounds) address, and masked after it lands.
    auto prefetch = [&](const Tile& t, int c) {
        const int ch = (t.c0 + c) * CI + pci;
        const bool live = ch < a.c_in;
        const int chc = min(ch, a.c_in - 1);
        const float* xc = a.x + (int64_t)t.b * a.x_bstride + (int64_t)chc * a.l_in;
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int w = plane + 32 * r;
            if constexpr (ACT) {
                const float v = xc[clampi(t.n_lo - 6 + w, 0, a.l_in - 1)];
                xr[r] = live ? v : 0.0f;
            } else {
                const int n = t.n_lo + w;
                const float v = xc[clampi(n, 0, a.l_in - 1)];
                xr[r] = (live && n >= 0 && n < a.l_in) ? v : 0.0f;
            }
        }
        if constexpr (ACT) {
            const float2 v = a.act.ab[chc];
            ab_pf = live ? v : make_float2(0.0f, 0.0f);
        }
    };
    // write item (t, c)'s row to LDS (from the prefetch registers when it
    // fits) and, with the activation, compute it into dst
    auto stage = [&](const Tile& t, int c, float* dst) {
        // with the activation the x row goes to its staging row; without, the
        // values go straight to the operand layout (position stride 4)
        constexpr int RS = ACT ? 1 : 4;
        float* row = ACT ? xs + pci * act_xs_len(W) : dst + (pci & 1) * W * 4 + (pci >> 1);
        if (prefetchable) {
#pragma unroll
            for (int r = 0; r < XR; ++r) {
                const int w = plane + 32 * r;
                if (w < row_len) row[w * RS] = xr[r];
            }
            ab_st = ab_pf;
        } else {
            for (int w = plane; w < row_len; w += 32) row[w * RS] = row_value(t, c, w);
            if constexpr (ACT) {
                const int ch = (t.c0 + c) * CI + pci;
                ab_st = ch < a.c_in ? a.act.ab[ch] : make_float2(0.0f, 0.0f);
            }
        }
    };
    ActTaps ftaps;
    if constexpr (ACT) {
        if (producer) ftaps = load_act_taps(a.act.taps);
    }
    auto compute = [&](const Tile& t, int c, float* dst) {
        if constexpr (ACT) {
            wave_lds_sync();
            act_from_xs<CI, true>(dst, xs, ss, (t.c0 + c) * CI, a.c_in, a.l_in, t.n_lo, W, ftaps, ab_st, pci, plane,
                                  0);
        }
    };

    // consumer identity
    const int wm = wave % WM, wn = wave / WM;
    const int mb_tot = (a.c_out + 31) >> 5;
    const int hi = lane >> 5, lo = lane & 31;
    const int colbase = wn * NBW * 32 + lo;

    v16f acc[MBW][NBW];
    // Accumulators start at the bias: one MFMA of the bias column (lanes
    // 0-31 hold bias[row], K index 0) against a ones row (K index 0).
    float bias_frag[MBW];
    auto load_bias = [&](int mb_base, int c0) {
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            bias_frag[mb] = (hi == 0 && c0 == 0) ? a.bias[min((mb_base + mb) * 32 + lo, a.c_out - 1)] : 0.0f;
    };
    auto init_acc = [&]() {
        const float ones = hi == 0 ? 1.0f : 0.0f;
        v16f z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
            for (int j = 0; j < NBW; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bias_frag[i], ones, z, 0, 0, 0);
    };
    // A operand of K-group g for the M blocks starting at mb_base, phase ph
    auto load_a = [&](float4 (&dst)[MBW], int mb_base, int ph, int g) {
        const float4* wp = reinterpret_cast<const float4*>(a.w + (int64_t)ph * a.w_phase_stride) +
                           ((int64_t)mb_base * G + g) * 64 + lane;
        if (mb_base + MBW <= mb_tot) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) dst[mb] = wp[(int64_t)mb * G * 64];
        } else {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                dst[mb] = mb_base + mb < mb_tot ? wp[(int64_t)mb * G * 64] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    // Branch-free variant: blocks past c_out read the last valid block (their
    // rows are discarded in the epilogue), so no exec-mask branch breaks the
    // counter waits of the unrolled tap loop.
    auto load_a_nb = [&](float4 (&dst)[MBW], int mb_base, int ph, int g) {
        const float4* wp = reinterpret_cast<const float4*>(a.w + (int64_t)ph * a.w_phase_stride) + g * 64 + lane;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) dst[mb] = wp[(int64_t)min(mb_base + mb, mb_tot - 1) * G * 64];
    };
    // B operand of one tap: the 4 channel pairs x NBW blocks of 32 positions
    // (operand layout [hi][position][p]: one 16-byte read per block)
    auto load_b = [&](float (&dst)[4][NBW], const float* buf, int j) {
        const float* bp = buf + (hi * W + colbase + j * a.dil) * 4;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const float4 v = *reinterpret_cast<const float4*>(bp + nb * 128);
            dst[0][nb] = v.x;
            dst[1][nb] = v.y;
            dst[2][nb] = v.z;
            dst[3][nb] = v.w;
        }
    };
    auto mfma_tap = [&](const float4 (&A)[MBW], const float (&Bv)[4][NBW]) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                const float av = p == 0 ? A[mb].x : (p == 1 ? A[mb].y : (p == 2 ? A[mb].z : A[mb].w));
                if constexpr (BF16) {
                    // three-term bfloat16 split: ah*bh + al*bh + ah*bl
                    const float ah = round_bf16(av), al = round_bf16(av - ah);
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const float bh = round_bf16(Bv[p][nb]), bl = round_bf16(Bv[p][nb] - bh);
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ah, bh, acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(al, bh, acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ah, bl, acc[mb][nb], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, Bv[p][nb], acc[mb][nb], 0, 0, 0);
                }
            }
        }
    };
    float4 An[MBW];

    // Split products (PREC 2): v_mfma_f32_32x32x16_bf16 with K = 16 = two
    // (chunk, tap) slots x 8 channels. The slots of a K range run chunk-major,
    // s = chunk * TAPS + tap, and instruction u of an item takes slots 2u and
    // 2u + 1: lane l holds, for piece p, the A values W[m = l % 32][channel i
    // of the chunk of slot 2u + l / 32][its tap] and the B values of that
    // chunk's 8 channels at position n + tap dil: one 16-byte read per piece
    // and block. With an odd tap count a pair may span two chunks, so no slot
    // is padding. Weights ride a three-slot ring two pairs ahead.
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
    const int G6 = nch * (TAPS > 0 ? TAPS : 1) / 2;  // weight groups (slot pairs) per 32-row block
    v4u A6a[BX6 ? kPieces : 1][MBW], A6b[BX6 ? kPieces : 1][MBW], A6c[BX6 ? kPieces : 1][MBW];
    auto load_a6 = [&](v4u (&dst)[BX6 ? kPieces : 1][MBW], int mb_base, int ph, int g) {
        const v4u* wp = reinterpret_cast<const v4u*>(a.w6 + (int64_t)ph * a.w6_phase_stride) + (int64_t)g * kPieces * 64 + lane;
#pragma unroll
        for (int p = 0; p < (BX6 ? NPA : 1); ++p)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                dst[p][mb] = wp[((int64_t)min(mb_base + mb, mb_tot - 1) * G6 * kPieces + p) * 64];
    };
    // the six products of order <= 2 (the first three for PREC 3): (A piece, B piece),
    // measured 1-2% faster in this order
    auto mfma6 = [&](const v4u (&A)[BX6 ? kPieces : 1][MBW], const v4u (&B)[BX6 ? kPieces : 1][NBW]) {
        // by activation piece, so that only piece 0's LDS reads gate the first
        // products (PREC 3: the first three entries are its products too)
        constexpr int TA[6] = {0, 1, 0, 2, 1, 0}, TB[6] = {0, 0, 1, 0, 1, 2};
#pragma unroll
        for (int t = 0; t < NPROD; ++t)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(v8bf, A[BX6 ? TA[t] : 0][mb]), __builtin_bit_cast(v8bf, B[BX6 ? TB[t] : 0][nb]),
                        acc[mb][nb], 0, 0, 0);
    };

    // The pipeline walks items (tile, chunk) with chunk fastest. Producers
    // and consumers run separate loops with one barrier per item each, so
    // the compiler allocates registers for the larger role only.
    // Epilogue line touches: when the producers stage the last K-chunk of a
    // tile, one lane per 128-byte line of the tile's residual and running-sum
    // rows loads it (into a write-only LDS scratch), so that the consumers'
    // epilogue reads, one item later, hit L2 instead of waiting on HBM.
    auto touch_epilogue = [&](const Tile& t) {
        // (not for pointwise split products: with two items per tile the
        // touch has little lead and its loads slow the copies; measured 1.3%
        // faster on the encoder without them)
        if (a.ksplit > 1 || a.out_mul != 1 || (!a.res && !a.sum_in) || (BX6 && TAPS == 1)) return;
        const int row0 = t.mt * MWG;
        const int nrows = min(MWG, a.c_out - row0);
        const int npos = min(NWG, a.positions - t.p0);
        if (nrows <= 0 || npos <= 0) return;
        const int lpr = ((npos + 31) >> 5) + 1;  // lines per row segment (+1: unaligned start)
        const int64_t base = (int64_t)t.b * a.y_bstride + (int64_t)row0 * a.positions + t.p0 + a.out_add[t.ph];
        auto* tl = (__attribute__((address_space(3))) void*)(touch + (wave - 4) * 64);
        for (int i = tid - 256; i < nrows * lpr; i += 256) {
            const int row = i / lpr;
            const int off = min((i - row * lpr) * 32, npos - 1);
            const int64_t idx = base + (int64_t)row * a.positions + off;
            if (a.res) __builtin_amdgcn_global_load_lds((const void*)(a.res + idx), tl, 4, 0, 0);
            if (a.sum_in) __builtin_amdgcn_global_load_lds((const void*)(a.sum_in + idx), tl, 4, 0, 0);
        }
    };

    if (producer) {
        if constexpr (PK) {
            // Packed input: the window of each channel parity is a contiguous
            // run of W 16-byte groups, already in the operand layout; the
            // memory unit copies it to LDS 1 KB per wave instruction, so the
            // producers issue no vector ALU work next to the matrix cores.
            // (split products: kPieces planes per chunk instead of two parities)
            constexpr int NPL = BX6 ? kPieces : 2;
            const int DS = BX6 ? PS6 : W;    // LDS plane stride (positions)
            const int pw = wave - 4;
            const int segs = (W + 63) >> 6;  // 64-position segments per plane
            // item c of tile t: chunks t.c0 + CPI c + cc, planes one after another
            auto dma = [&](const Tile& t, int c, float* dst) {
                const float* src = a.x + (int64_t)t.b * a.x_bstride +
                                   ((int64_t)(t.c0 + CPI * c) * NPL * a.pk_lp + kPkPadL + t.n_lo) * 4;
                for (int q = pw; q < CPI * NPL * segs; q += 4) {
                    const int hp = q / segs;  // plane within the item (chunk cc = hp / NPL)
                    const int pos0 = (q - hp * segs) * 64;
                    const int pos = pos0 + lane;
                    auto* ldst = (__attribute__((address_space(3))) void*)(dst + (hp * DS + pos0) * 4);
                    if (pos < W)
                        __builtin_amdgcn_global_load_lds((const void*)(src + ((int64_t)hp * a.pk_lp + pos) * 4), ldst, 16,
                                                         0, 0);
                }
            };
            Tile nt = tile_at(t_begin);
            int nc = 0;
            dma(nt, 0, abuf);
            if (ipt == 1) touch_epilogue(nt);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            for (int it = 0; it < n_items; ++it) {
                if (it + 1 < n_items) {
                    if (++nc == ipt) {
                        nc = 0;
                        nt = tile_at(t_begin + (it + 1) / ipt);
                    }
                    dma(nt, nc, abuf + ((it + 1) & 1) * ABUF);
                    if (nc == ipt - 1) touch_epilogue(nt);
                }
                // the copies land in LDS before the buffer is handed over
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            return;
        }
        Tile cur = tile_at(t_begin);
        int cur_c = 0;
        if (prefetchable) prefetch(cur, 0);
        // look-ahead item (the one after `cur`)
        Tile la = cur;
        int la_c = 0;
        auto advance = [&](Tile& t, int& c, int item) {
            if (++c == ipt) {
                c = 0;
                t = tile_at(t_begin + item / ipt);
            }
        };
        stage(cur, 0, abuf);
        if (ipt == 1) touch_epilogue(cur);
        if (n_items > 1) {
            advance(la, la_c, 1);
            if (prefetchable) prefetch(la, la_c);
        }
        compute(cur, 0, abuf);
        __syncthreads();
        for (int it = 0; it < n_items; ++it) {
            if (it + 1 < n_items) {
                // la is item it + 1: commit its row, start fetching it + 2, compute it + 1
                float* dst = abuf + ((it + 1) & 1) * ABUF;
                const Tile t1 = la;
                const int c1 = la_c;
                stage(t1, c1, dst);
                if (c1 == ipt - 1) touch_epilogue(t1);
                if (it + 2 < n_items) {
                    advance(la, la_c, it + 2);
                    if (prefetchable) prefetch(la, la_c);
                }
                compute(t1, c1, dst);
            }
            __syncthreads();
        }
        return;
    }

    if constexpr (RB == 16) {
        // 16 x 16 x 4 roles: lane l is row / column l % 16 and K-step l / 16.
        // K-step k of half s is channel 4s + k of the chunk, in LDS at
        // [hi = k & 1][position][p = 2s + (k >> 1)]: one 16-byte read gives
        // a lane both halves.
        typedef float v4f __attribute__((ext_vector_type(4)));
        const int l16 = lane & 15, k4 = lane >> 4;
        const int kp = k4 >> 1, khi = k4 & 1;
        const int colbase16 = wave * NBW * 16 + l16;  // (WM == 1: consumer wave = column)
        const float2* w16 = reinterpret_cast<const float2*>(a.w16);
        auto ld16 = [&](int mt, int g) { return w16[((int64_t)mt * G + g) * 64 + lane]; };
        v4f acc16[NBW];
        // accumulators start at the bias: bias column (K-step 0) x ones row
        auto init16 = [&](int mt) {
            const int m = mt * 16 + l16;
            const float bz = (k4 == 0 && m < a.c_out) ? a.bias[m] : 0.0f;
            const float one = k4 == 0 ? 1.0f : 0.0f;
            const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) acc16[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bz, one, z, 0, 0, 0);
        };
        Tile cur = tile_at(t_begin);
        int cur_c = 0;
        init16(cur.mt);
        // weights of taps j, j + 1, j + 2 in a three-slot ring (as the 32-row path)
        float2 R0 = ld16(cur.mt, cur.c0 * TAPS), R1 = ld16(cur.mt, cur.c0 * TAPS + 1), R2;
        __syncthreads();
        for (int it = 0; it < n_items; ++it) {
            const bool has_next = it + 1 < n_items;
            Tile nxt = cur;
            int nxt_c = cur_c + 1;
            if (nxt_c == ipt) {
                nxt_c = 0;
                if (has_next) nxt = tile_at(t_begin + (it + 1) / ipt);
            }
            const float* cur_buf = abuf + (it & 1) * ABUF;
            const int g0 = (cur.c0 + cur_c) * TAPS;
            const int ng0 = has_next ? (nxt.c0 + nxt_c) * TAPS : g0;
            const int nmt = has_next ? nxt.mt : cur.mt;
#pragma unroll
            for (int j = 0; j < TAPS; ++j) {
                float2& use = (j % 3 == 0) ? R0 : ((j % 3 == 1) ? R1 : R2);
                float2& fill = ((j + 2) % 3 == 0) ? R0 : (((j + 2) % 3 == 1) ? R1 : R2);
                fill = (j + 2 < TAPS) ? ld16(cur.mt, g0 + j + 2) : ld16(nmt, ng0 + (j + 2 - TAPS));
                __builtin_amdgcn_sched_barrier(0);
                float4 bv[NBW];
                const float* bp = cur_buf + (khi * W + colbase16 + j * a.dil) * 4;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) bv[nb] = *reinterpret_cast<const float4*>(bp + nb * 64);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const float b0 = kp ? bv[nb].y : bv[nb].x;
                    const float b1 = kp ? bv[nb].w : bv[nb].z;
                    acc16[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(use.x, b0, acc16[nb], 0, 0, 0);
                    acc16[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(use.y, b1, acc16[nb], 0, 0, 0);
                }
            }
            // the next item's taps 0 and 1 sit in slots TAPS % 3, (TAPS + 1) % 3
            if constexpr (TAPS % 3 == 1) {
                R0 = R1;
                R1 = R2;
            } else if constexpr (TAPS % 3 == 2) {
                const float2 t0 = R2;
                R1 = R0;
                R0 = t0;
            }
            if (cur_c == ipt - 1) {
                // row 4 (l / 16) + i, column l % 16 of each 16 x 16 block
                const int64_t ostride = (int64_t)a.out_mul * a.positions;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const int pos = cur.p0 + colbase16 + nb * 16;
                    if (pos >= a.positions) continue;
                    const int tt = a.out_mul * pos + a.out_add[cur.ph];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int o = cur.mt * 16 + 4 * k4 + i;
                        if (o >= a.c_out) continue;
                        const int64_t idx = (int64_t)cur.b * a.y_bstride + (int64_t)o * ostride + tt;
                        float v = acc16[nb][i];
                        if (a.res) v += a.res[idx];
                        if (a.sum_in) v += a.sum_in[idx];
                        a.y[idx] = v * a.scale;
                    }
                }
                init16(nmt);
            }
            cur = nxt;
            cur_c = nxt_c;
            __syncthreads();
        }
        return;
    }

    Tile cur = tile_at(t_begin);
    int cur_c = 0;
    load_bias(__builtin_amdgcn_readfirstlane(cur.mt * (MWG / 32) + wm * MBW), cur.c0);
    init_acc();
    float4 Ar0[MBW], Ar1[MBW], Ar2[MBW];
    if constexpr (BX6) {
        const int mb0 = __builtin_amdgcn_readfirstlane(cur.mt * (MWG / 32) + wm * MBW);
        const int g0 = cur.c0 * TAPS / 2;
        load_a6(A6a, mb0, cur.ph, g0);
        load_a6(A6b, mb0, cur.ph, g0 + 1);
    } else if constexpr (TAPS > 0) {
        const int mb0 = __builtin_amdgcn_readfirstlane(cur.mt * (MWG / 32) + wm * MBW);
        load_a_nb(Ar0, mb0, cur.ph, cur.c0 * a.taps);
        load_a_nb(Ar1, mb0, cur.ph, cur.c0 * a.taps + 1);
    } else {
        load_a(An, __builtin_amdgcn_readfirstlane(cur.mt * (MWG / 32) + wm * MBW), cur.ph, cur.c0 * a.taps);
    }
    (void)Ar2;
    __syncthreads();
    for (int it = 0; it < n_items; ++it) {
        // the item after this one
        const bool has_next = it + 1 < n_items;
        Tile nxt = cur;
        int nxt_c = cur_c + 1;
        if (nxt_c == ipt) {
            nxt_c = 0;
            if (has_next) nxt = tile_at(t_begin + (it + 1) / ipt);
        }
        // wave-uniform M-block base (the compiler cannot see it is uniform)
        const int mb_base = __builtin_amdgcn_readfirstlane(cur.mt * (MWG / 32) + wm * MBW);
        // the next tile's bias, in flight during this item
        if (nxt_c == 0 && has_next)
            load_bias(__builtin_amdgcn_readfirstlane(nxt.mt * (MWG / 32) + wm * MBW), nxt.c0);
        const bool live = mb_base < mb_tot;
        const float* cur_buf = abuf + (it & 1) * ABUF;
        const int g0 = (cur.c0 + cur_c) * a.taps;
        if constexpr (BX6) {
            const int nmb_base = __builtin_amdgcn_readfirstlane(nxt.mt * (MWG / 32) + wm * MBW);
            // the item's CPI chunks hold CPI * TAPS slots: pair u is weight group q0 + u
            constexpr int NPI = CPI * TAPS / 2;
            static_assert((CPI * TAPS) % 2 == 0 && NPI >= 2, "whole slot pairs; the ring holds two ahead");
            const int q0 = (cur.c0 + CPI * cur_c) * TAPS / 2;
            const int nq0 = has_next ? (nxt.c0 + CPI * nxt_c) * TAPS / 2 : q0;
            const int nmb = has_next ? nmb_base : mb_base;
            const int nph6 = has_next ? nxt.ph : cur.ph;
            const float* bb_0 = cur_buf + colbase * 4;
            // slots 0 and 1 hold pairs 0 and 1 on entry; pair u + 2 (or the next
            // item's pair u + 2 - NPI) loads while pair u multiplies
#pragma unroll
            for (int u = 0; u < NPI; ++u) {
                v4u(&use)[kPieces][MBW] = (u % 3 == 0) ? A6a : ((u % 3 == 1) ? A6b : A6c);
                v4u(&fill)[kPieces][MBW] = ((u + 2) % 3 == 0) ? A6a : (((u + 2) % 3 == 1) ? A6b : A6c);
                if (u + 2 < NPI) {
                    load_a6(fill, mb_base, cur.ph, q0 + u + 2);
                } else {
                    load_a6(fill, nmb, nph6, nq0 + (u + 2 - NPI));
                }
                __builtin_amdgcn_sched_barrier(0);
                const int s0 = 2 * u, s1 = 2 * u + 1;
                const int off0 = (s0 / TAPS) * kPieces * PS6 + (s0 % TAPS) * a.dil;
                const int off1 = (s1 / TAPS) * kPieces * PS6 + (s1 % TAPS) * a.dil;
                const float* bq = bb_0 + (hi ? off1 : off0) * 4;
                v4u Bv[kPieces][NBW];
#pragma unroll
                for (int p = 0; p < NPA; ++p)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        Bv[p][nb] = *reinterpret_cast<const v4u*>(bq + (p * PS6 + nb * 32) * 4);
                __builtin_amdgcn_sched_barrier(0);
                mfma6(use, Bv);
            }
            // the next item's pairs 0 and 1 sit in slots NPI % 3, (NPI + 1) % 3
            if constexpr (NPI % 3 == 1) {
#pragma unroll
                for (int p = 0; p < kPieces; ++p)
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
                        A6a[p][mb] = A6b[p][mb];
                        A6b[p][mb] = A6c[p][mb];
                    }
            } else if constexpr (NPI % 3 == 2) {
#pragma unroll
                for (int p = 0; p < kPieces; ++p)
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
                        const v4u t0 = A6c[p][mb];
                        A6b[p][mb] = A6a[p][mb];
                        A6a[p][mb] = t0;
                    }
            }
        } else if constexpr (TAPS > 0) {
            // Compile-time tap count: the tap loop is fully unrolled and
            // branch-free. The weights ride a three-slot register ring loaded
            // two taps ahead (one tap of MFMAs does not cover the L2
            // latency); the last two taps prefetch the next item's first two.
            // Slots 0 and 1 hold taps 0 and 1 of the current item on entry.
            const int nmb_base = __builtin_amdgcn_readfirstlane(nxt.mt * (MWG / 32) + wm * MBW);
            const int nph = has_next ? nxt.ph : cur.ph;
            const int ng0 = has_next ? (nxt.c0 + nxt_c) * TAPS : g0;
            const int nmb = has_next ? nmb_base : mb_base;
            // Large wave tiles (more than 2 x 2 blocks) double-buffer the LDS
            // operands across taps: tap j + 1's reads go out before tap j's
            // MFMAs, so only tap 0 waits on LDS latency. (Smaller tiles would
            // pay for the registers with resident workgroups.)
            constexpr bool BDB = MBW * NBW > 4;
            float Bb[BDB ? 2 : 1][4][NBW];
            if constexpr (BDB) load_b(Bb[0], cur_buf, 0);
#pragma unroll
            for (int j = 0; j < TAPS; ++j) {
                float4(&use)[MBW] = (j % 3 == 0) ? Ar0 : ((j % 3 == 1) ? Ar1 : Ar2);
                float4(&fill)[MBW] = ((j + 2) % 3 == 0) ? Ar0 : (((j + 2) % 3 == 1) ? Ar1 : Ar2);
                if (j + 2 < TAPS) {
                    load_a_nb(fill, mb_base, cur.ph, g0 + j + 2);
                } else {
                    load_a_nb(fill, nmb, nph, ng0 + (j + 2 - TAPS));
                }
                // keep the prefetch at the top of the tap: the scheduler would
                // otherwise sink it next to its use two taps later
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (BDB) {
                    if (j + 1 < TAPS) load_b(Bb[(j + 1) & 1], cur_buf, j + 1);
                } else {
                    load_b(Bb[0], cur_buf, j);
                }
                // issue the LDS reads before the tap's MFMAs
                __builtin_amdgcn_sched_barrier(0);
                mfma_tap(use, Bb[BDB ? (j & 1) : 0]);
            }
            // the next item's taps 0 and 1 sit in slots TAPS % 3, (TAPS + 1) % 3
            if constexpr (TAPS % 3 == 1) {
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) {
                    Ar0[mb] = Ar1[mb];
                    Ar1[mb] = Ar2[mb];
                }
            } else if constexpr (TAPS % 3 == 2) {
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) {
                    const float4 t0 = Ar2[mb];
                    Ar1[mb] = Ar0[mb];
                    Ar0[mb] = t0;
                }
            }
        } else {
            // Runtime tap count: the weights of tap j + 1 load while tap j
            // multiplies; the LDS operands are read per tap and the second
            // resident workgroup covers their latency.
            for (int j = 0; j < a.taps; ++j) {
                float4 Ac[MBW];
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) Ac[mb] = An[mb];
                if (j + 1 < a.taps) {
                    load_a(An, mb_base, cur.ph, g0 + j + 1);
                } else if (has_next) {
                    load_a(An, __builtin_amdgcn_readfirstlane(nxt.mt * (MWG / 32) + wm * MBW), nxt.ph,
                           (nxt.c0 + nxt_c) * a.taps);
                }
                if (!live) continue;
                float Bv[4][NBW];
                load_b(Bv, cur_buf, j);
                mfma_tap(Ac, Bv);
            }
        }
        if (cur_c == ipt - 1) {
            if (a.ksplit > 1) {
                // raw partial sums of this K range in MFMA fragment order:
                // [wave][mb][nb][r][lane], so each register is one 256-byte
                // row of the wave and the 16 of a block share one address
                float* pt = a.partial + (int64_t)cur.vid * (MWG * NWG) + wave * (MBW * NBW * 1024) + lane;
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) pt[(mb * NBW + nb) * 1024 + r * 64] = acc[mb][nb][r];
            } else if (live) {
                const int64_t ostride = (int64_t)a.out_mul * a.positions;
                if constexpr (BX6 && MBW == 1) {
                    // Split-product tiles of one row block per wave: by 32 x 32
                    // block, the block's 16 residual and running-sum loads per
                    // lane all go out before its adds and stores (exact for
                    // in-place updates: no output is read after another one
                    // has been written; per-workgroup time measured 4% lower).
                    const int64_t ybase = (int64_t)cur.b * a.y_bstride;
                    if (!a.sum_in) {
                        // no running sum (the encoder's convs, conv_pre, the
                        // transposed convs): the residual loads of three
                        // blocks at a time go out together (all NBW would
                        // spill registers), so a tile pays ceil(NBW / 3)
                        // memory round trips
                        constexpr int EG = 3;
#pragma unroll
                        for (int g0 = 0; g0 < NBW; g0 += EG) {
                            float rv[EG][16];
#pragma unroll
                            for (int k = 0; k < EG; ++k) {
                                if (g0 + k >= NBW) break;
                                const int pos = cur.p0 + wn * NBW * 32 + (g0 + k) * 32 + lo;
                                const bool pos_ok = pos < a.positions;
                                const int tt = a.out_mul * pos + a.out_add[cur.ph];
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int o = mb_base * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                    const int64_t idx =
                                        (pos_ok && o < a.c_out) ? ybase + (int64_t)o * ostride + tt : ybase;
                                    rv[k][r] = a.res ? a.res[idx] : 0.0f;
                                }
                            }
#pragma unroll
                            for (int k = 0; k < EG; ++k) {
                                if (g0 + k >= NBW) break;
                                const int pos = cur.p0 + wn * NBW * 32 + (g0 + k) * 32 + lo;
                                const bool pos_ok = pos < a.positions;
                                const int tt = a.out_mul * pos + a.out_add[cur.ph];
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int o = mb_base * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                    if (!(pos_ok && o < a.c_out)) continue;
                                    a.y[ybase + (int64_t)o * ostride + tt] = (acc[0][g0 + k][r] + rv[k][r]) * a.scale;
                                }
                            }
                        }
                    } else
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) {
                            const int pos = cur.p0 + wn * NBW * 32 + nb * 32 + lo;
                            const bool pos_ok = pos < a.positions;
                            const int tt = a.out_mul * pos + a.out_add[cur.ph];
                            float rv[16], sv[16];
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int o = (mb_base + mb) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                const int64_t idx = (pos_ok && o < a.c_out) ? ybase + (int64_t)o * ostride + tt : ybase;
                                rv[r] = a.res ? a.res[idx] : 0.0f;
                                sv[r] = a.sum_in ? a.sum_in[idx] : 0.0f;
                            }
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int o = (mb_base + mb) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                if (!(pos_ok && o < a.c_out)) continue;
                                a.y[ybase + (int64_t)o * ostride + tt] = (acc[mb][nb][r] + rv[r] + sv[r]) * a.scale;
                            }
                        }
                    }
                } else if constexpr (MBW * NBW > 4) {
                    // Large tiles (one workgroup per CU, registers to spare):
                    // by row group of 4 outputs per lane, the group's residual
                    // and running-sum loads all go out before its adds and
                    // stores. y may alias both (in-place updates), so the
                    // compiler keeps every load behind the stores before it;
                    // grouping is still exact, since no output is read after
                    // another output has been written. Groups past c_out are
                    // skipped.
                    const int64_t ybase = (int64_t)cur.b * a.y_bstride;
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
                        const int row0 = (mb_base + mb) * 32;
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) {
                            const int pos = cur.p0 + wn * NBW * 32 + nb * 32 + lo;
                            const bool pos_ok = pos < a.positions;
                            const int tt = a.out_mul * pos + a.out_add[cur.ph];
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                if (row0 + 8 * g >= a.c_out) break;
                                const int o0 = row0 + 8 * g + 4 * hi;
                                float rv[4], sv[4];
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const bool ok = pos_ok && o0 + i < a.c_out;
                                    const int64_t idx = ok ? ybase + (int64_t)(o0 + i) * ostride + tt : 0;
                                    rv[i] = a.res ? a.res[idx] : 0.0f;
                                    sv[i] = a.sum_in ? a.sum_in[idx] : 0.0f;
                                }
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    if (!(pos_ok && o0 + i < a.c_out)) continue;
                                    float v = acc[mb][nb][4 * g + i];
                                    if (a.res) v += rv[i];
                                    if (a.sum_in) v += sv[i];
                                    a.y[ybase + (int64_t)(o0 + i) * ostride + tt] = v * a.scale;
                                }
                            }
                        }
                    }
                } else {
                    // Per element (smaller tiles: batching costs a resident
                    // workgroup per CU, measured slower).
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) {
                            const int pos = cur.p0 + wn * NBW * 32 + nb * 32 + lo;
                            if (pos >= a.positions) continue;
                            const int tt = a.out_mul * pos + a.out_add[cur.ph];
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int o = (mb_base + mb) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                if (o >= a.c_out) continue;
                                const int64_t idx = (int64_t)cur.b * a.y_bstride + (int64_t)o * ostride + tt;
                                float v = acc[mb][nb][r];
                                if (a.res) v += a.res[idx];
                                if (a.sum_in) v += a.sum_in[idx];
                                a.y[idx] = v * a.scale;
                            }
                        }
                    }
                }
            }
            init_acc();
        }
        cur = nxt;
        cur_c = nxt_c;
        __syncthreads();
    }
}

// Sum the ksplit partial tiles of a split conv in a fixed order and apply
// residual, running sum and scale (the bias is in the first range's sums).
// One thread per (base tile, row, column); the partial tiles are in the
// conv kernel's fragment order for consumer waves arranged wm + WM * wn.
struct SplitGeom {
    int mbw, nbw, wm, wn;
};
__global__ void __launch_bounds__(256) split_reduce_kernel(ConvArgs a, SplitGeom g) {
    const int tile_m = g.wm * g.mbw * 32, tile_n = g.wn * g.nbw * 32;
    const int n_nt = (a.positions + tile_n - 1) / tile_n;
    const int n_mt = (a.c_out + tile_m - 1) / tile_m;
    const int64_t base_tiles = (int64_t)n_nt * n_mt * a.groups;
    const int64_t per_tile = (int64_t)tile_m * tile_n;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= base_tiles * per_tile) return;
    const int64_t id = e / per_tile;
    const int local = (int)(e - id * per_tile);
    const int row = local / tile_n, col = local - row * tile_n;
    const int nt = (int)(id % n_nt);
    const int64_t rest = id / n_nt;
    const int mt = (int)(rest % n_mt);
    const int grp = (int)(rest / n_mt);
    const int b = grp / a.phases, ph = grp % a.phases;
    const int o = mt * tile_m + row, pos = nt * tile_n + col;
    if (o >= a.c_out || pos >= a.positions) return;
    // (row, col) -> fragment slot
    const int wm = row / (g.mbw * 32), mb = (row / 32) % g.mbw, rr = row % 32;
    const int wn = col / (g.nbw * 32), nb = (col / 32) % g.nbw, lo = col % 32;
    const int r = 4 * (rr / 8) + rr % 4, hi = (rr / 4) % 2;
    const int slot = ((((wn * g.wm + wm) * g.mbw + mb) * g.nbw + nb) * 16 + r) * 64 + hi * 32 + lo;
    float v = 0.0f;
    for (int sp = 0; sp < a.ksplit; ++sp) v += a.partial[(sp * base_tiles + id) * per_tile + slot];
    const int64_t idx = (int64_t)b * a.y_bstride + (int64_t)o * a.out_mul * a.positions + a.out_mul * pos + a.out_add[ph];
    if (a.res) v += a.res[idx];
    if (a.sum_in) v += a.sum_in[idx];
    a.y[idx] = v * a.scale;
}

TileShape tile_shape(TileId t) {
    if (t == TILE_16x256) return {16, 256};
    switch (t) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: return {wm * mbw * 32, wn * nbw * 32};
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return {0, 0};
    }
}

template <typename K>
static hipError_t launch_persistent(K kernel, const ConvArgs& a, int64_t tiles, size_t lds, hipStream_t stream) {
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    // One slot per resident workgroup; cached per (kernel, LDS size).
    static thread_local const void* last_k = nullptr;
    static thread_local size_t last_lds = 0;
    static thread_local int last_slots = 0;
    int slots;
    if (last_k == (const void*)kernel && last_lds == lds) {
        slots = last_slots;
    } else {
        int per_cu = 0, dev = 0, cus = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 512, lds);
        if (e != hipSuccess) return e;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        slots = std::max(1, per_cu) * std::max(1, cus);
        last_k = (const void*)kernel;
        last_lds = lds;
        last_slots = slots;
    }
    const int64_t grid = std::min<int64_t>(tiles, slots);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(512), lds, stream, a);
    return hipGetLastError();
}

template <int MBW, int NBW, int WM, int WN, bool TAPS_TILE>
static hipError_t launch_tile(const ConvArgs& a, hipStream_t stream) {
    constexpr int NWG = WN * NBW * 32;
    constexpr int MWG = WM * MBW * 32;
    const int W = NWG + (a.taps - 1) * a.dil;
    const int64_t tiles =
        (int64_t)((a.positions + NWG - 1) / NWG) * ((a.c_out + MWG - 1) / MWG) * a.groups * a.ksplit;
    const bool act = a.act.taps != nullptr;
    if (a.bx6 && (act || a.pk_lp <= 0)) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * (size_t)conv_lds_floats(W, act);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    // instances with the AMP tap counts compiled in (3, 7, 11)
#define MH3A_TAPS(ACTV, T)                                                                                          \
    if (a.taps == T)                                                                                               \
        return a.bf16 ? launch_persistent(conv_kernel<MBW, NBW, WM, WN, ACTV, 1, T>, a, tiles, lds, stream)        \
                      : launch_persistent(conv_kernel<MBW, NBW, WM, WN, ACTV, 0, T>, a, tiles, lds, stream);
    if (act) {
        if constexpr (TAPS_TILE) {
            MH3A_TAPS(true, 3)
            MH3A_TAPS(true, 7)
            MH3A_TAPS(true, 11)
        }
        return a.bf16 ? launch_persistent(conv_kernel<MBW, NBW, WM, WN, true, 1, 0>, a, tiles, lds, stream)
                      : launch_persistent(conv_kernel<MBW, NBW, WM, WN, true, 0, 0>, a, tiles, lds, stream);
    }
    if (a.pk_lp > 0) {
        // packed input: compile-time taps only
        if constexpr (TAPS_TILE) {
            if (NWG > 256) return hipErrorInvalidValue;
            if (a.bx6) {
                // split products: bf16 pieces, one phase, planes sized for kBx6MaxDil
                if (!a.w6 || a.dil < 1) return hipErrorInvalidValue;
                // whole items per K range
                if ((((a.c_in + kChunk - 1) / kChunk) / a.ksplit) % bx6_cpi(NWG, a.taps)) return hipErrorInvalidValue;
                if (a.dil > kBx6MaxDil) {
                    // wider planes: 7 taps up to dilation kBx6WideDil (encoder units), fp32-level products only
                    if (a.taps != 7 || a.dil > kBx6WideDil || a.bf16) return hipErrorInvalidValue;
                    return launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 2, 7, 32, kBx6WideDil>, a, tiles,
                                             sizeof(float) * (size_t)conv_lds_floats6(NWG, 7, kBx6WideDil), stream);
                }
                if (a.taps == 1 && !a.bf16)  // pointwise convs (encoder units): one zero-padded tap pair
                    return launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 2, 1>, a, tiles,
                                             sizeof(float) * (size_t)conv_lds_floats6(NWG, 1), stream);
#define MH3A_TAPS6(T)                                                                                           \
    if (a.taps == T)                                                                                           \
        return a.bf16 ? launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 3, T>, a, tiles,                \
                                          sizeof(float) * (size_t)conv_lds_floats6(NWG, T), stream)            \
                      : launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 2, T>, a, tiles,                \
                                          sizeof(float) * (size_t)conv_lds_floats6(NWG, T), stream);
                MH3A_TAPS6(2)
                MH3A_TAPS6(3)
                MH3A_TAPS6(7)
                MH3A_TAPS6(11)
#undef MH3A_TAPS6
                return hipErrorInvalidValue;
            }
            MH3A_TAPS(false, 3)
            MH3A_TAPS(false, 7)
            MH3A_TAPS(false, 11)
        }
        return hipErrorInvalidValue;
    }
#undef MH3A_TAPS
    // (in_proj, conv_pre and the upsamplers: fp32 operands, runtime taps)
    return (a.bf16 || a.bx6) ? hipErrorInvalidValue
                             : launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 0, 0>, a, tiles, lds, stream);
}

// 16 x 256 tiles: AMP convs (compile-time taps, fp32), fused activation or
// packed input, no K split.
static hipError_t launch_tile16(const ConvArgs& a, hipStream_t stream) {
    constexpr int NWG = 256;
    if (!a.w16 || a.bf16 || a.bx6 || a.ksplit != 1 || a.phases != 1) return hipErrorInvalidValue;
    const int W = NWG + (a.taps - 1) * a.dil;
    const int64_t tiles = (int64_t)((a.positions + NWG - 1) / NWG) * ((a.c_out + 15) / 16) * a.groups;
    const bool act = a.act.taps != nullptr;
    if (!act && a.pk_lp <= 0) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * (size_t)conv_lds_floats(W, act);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
#define MH3A_TAPS16(T)                                                                                            \
    if (a.taps == T)                                                                                             \
        return act ? launch_persistent(conv_kernel<1, 4, 1, 4, true, 0, T, 16>, a, tiles, lds, stream)            \
                   : launch_persistent(conv_kernel<1, 4, 1, 4, false, 0, T, 16>, a, tiles, lds, stream);
    MH3A_TAPS16(3)
    MH3A_TAPS16(7)
    MH3A_TAPS16(11)
#undef MH3A_TAPS16
    return hipErrorInvalidValue;
}

hipError_t launch_conv(const ConvArgs& a, TileId tile, hipStream_t stream) {
    // the kernel cuts the chunks into ksplit equal ranges
    const int nch = (a.c_in + kChunk - 1) / kChunk;
    if (a.ksplit < 1 || nch % a.ksplit != 0 || (a.ksplit > 1 && !a.partial)) return hipErrorInvalidValue;
    if (tile == TILE_16x256) return launch_tile16(a, stream);
    hipError_t e = hipSuccess;
    switch (tile) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: e = launch_tile<mbw, nbw, wm, wn, tile_has_act_taps(id)>(a, stream); break;
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || a.ksplit <= 1) return e;
    SplitGeom g{};
    switch (tile) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: g = {mbw, nbw, wm, wn}; break;
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return hipErrorInvalidValue;
    }
    const int tm = g.wm * g.mbw * 32, tn = g.wn * g.nbw * 32;
    const int64_t n = (int64_t)((a.positions + tn - 1) / tn) * ((a.c_out + tm - 1) / tm) * a.groups * tm * tn;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// activation_post + conv_post + clamp. A workgroup owns kFinalT outputs;
// the act window is [t0 - 3, t0 + kFinalT + 3).
// ---------------------------------------------------------------------------
constexpr int kFinalT = 256;

__global__ void __launch_bounds__(256) final_kernel(FinalArgs a) {
    constexpr int CI = kChunk;
    constexpr int W = kFinalT + 6;
    __shared__ __attribute__((aligned(16))) float as[CI * W];
    __shared__ __attribute__((aligned(16))) float xs[CI * act_xs_len(W)];
    __shared__ __attribute__((aligned(16))) float ss[CI * act_ss_len(W)];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kFinalT;
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    const int t = t0 + threadIdx.x;
    float acc = 0.0f;
    const ActTaps f = load_act_taps(a.act.taps);
    for (int c0 = 0; c0 < a.c; c0 += CI) {
        __syncthreads();
        stage_act<CI, W>(as, xs, ss, xb, c0, a.c, a.l, t0 - 3, f, a.act.ab, threadIdx.x >> 5, threadIdx.x & 31, W);
        __syncthreads();
        for (int ci = 0; ci < CI && c0 + ci < a.c; ++ci) {
            const float* wr = a.w + (c0 + ci) * 7;
            const float* ar = as + ci * W + threadIdx.x;
#pragma unroll
            for (int j = 0; j < 7; ++j) acc = fmaf(wr[j], ar[j], acc);
        }
    }
    if (t < a.l) {
        float v = acc + a.bias;
        if (a.clamp) v = fminf(fmaxf(v, -1.0f), 1.0f);
        a.y[(int64_t)b * a.l + t] = v;
    }
}

// ---------------------------------------------------------------------------
// Standalone activation: a workgroup owns kActT padded positions of kChunk
// channels (32 threads per channel, as in the conv producers), computes them
// into LDS rows and stores them packed: each thread writes the 16-byte group
// of one (hi, position), so every wave stores 1 KB contiguous.
// ---------------------------------------------------------------------------
constexpr int kActT = 256;

template <int W, bool PIECES>
__global__ void __launch_bounds__(256) act_kernel(ActArgs a) {
    constexpr int CI = kChunk;
    // each channel's result row reuses its x row (dead after the up pass)
    static_assert(act_xs_len(W) >= W, "result rows alias the x rows");
    __shared__ __attribute__((aligned(16))) float xs[CI * act_xs_len(W)];
    __shared__ __attribute__((aligned(16))) float ss[CI * act_ss_len(W)];
    float* as = xs;
    const int t0 = blockIdx.x * W - kPkPadL;  // first position (pads included)
    const int chunk = blockIdx.y;
    const int b = blockIdx.z;
    const int ci = threadIdx.x >> 5, lane32 = threadIdx.x & 31;
    constexpr int NPL = PIECES ? kPieces : 2;  // planes per chunk: pieces, or channel parities
    float* yc = a.y + (int64_t)b * a.y_bstride + (int64_t)chunk * NPL * a.lp * 4;
    if (t0 >= a.l || t0 + W <= 0) {
        // all padding
        for (int idx = threadIdx.x; idx < NPL * W; idx += 256) {
            const int hi = idx / W, w = idx - hi * W;
            const int q = t0 + kPkPadL + w;
            if (q < a.lp) *reinterpret_cast<float4*>(yc + ((int64_t)hi * a.lp + q) * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const ActTaps f = load_act_taps(a.act.taps);
    constexpr int XS = act_xs_len(W);
    stage_act<CI, W>(as, xs, ss, a.x + (int64_t)b * a.x_bstride, chunk * CI, a.c, a.l, t0, f, a.act.ab, ci, lane32, XS);
    __syncthreads();
    if constexpr (PIECES) {
        // one position per thread: the 8 channels' pieces, 16 bytes per plane
        for (int w = threadIdx.x; w < W; w += 256) {
            const int q = t0 + kPkPadL + w;
            if (q >= a.lp) continue;
            static_assert(CI == 8, "one 16-byte group per piece");
            float v8[8];
#pragma unroll
            for (int c = 0; c < CI; ++c) v8[c] = as[c * XS + w];
            uint4 g[kPieces];
            split3_pack8(v8, g);
#pragma unroll
            for (int p = 0; p < kPieces; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
        }
        return;
    }
    for (int idx = threadIdx.x; idx < 2 * W; idx += 256) {
        const int hi = idx / W, w = idx - hi * W;
        const int q = t0 + kPkPadL + w;  // index in the padded row
        if (q >= a.lp) continue;
        const float4 v =
            make_float4(as[hi * XS + w], as[(2 + hi) * XS + w], as[(4 + hi) * XS + w], as[(6 + hi) * XS + w]);
        *reinterpret_cast<float4*>(yc + ((int64_t)hi * a.lp + q) * 4) = v;
    }
}

hipError_t launch_act(const ActArgs& a, int batch, hipStream_t stream) {
    if (a.c < 1 || a.l < 1 || batch < 1 || !a.act.taps || a.lp != a.l + kPkPadL + kPkPadR) return hipErrorInvalidValue;
    dim3 grid((a.lp + kActT - 1) / kActT, (a.c + kChunk - 1) / kChunk, batch);
    if (a.pieces != 0 && a.pieces != kPieces) return hipErrorInvalidValue;
    if (a.pieces)
        hipLaunchKernelGGL((act_kernel<kActT, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((act_kernel<kActT, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One AMP residual unit per launch, for narrow stages (8 to 32 channels):
//   y = scale * (x + conv2(act2(conv1(act1(x)))) + sum_in)
// A workgroup of four waves owns T output positions [p0, p0 + T) of one
// batch item and every channel, and keeps the unit's intermediates in LDS:
//   x rows  over [x_lo, x_lo + act_xs_len(W1))   replicate-clamped loads
//   act1 -> A1 over [a1_lo, a1_lo + W1)          zero outside [0, l): conv1's padding
//   conv1 -> Y1 over [y1_lo, y1_lo + XS2)        into the x region; positions outside
//                                                [0, l) then take the edge values
//                                                (act2's replicate padding)
//   act2 -> A2 over [a2_lo, a2_lo + W2)          into the A1 region
//   conv2 + bias + x (+ sum_in), * scale -> y over [p0, p0 + T)
// where a2_lo = p0 - R2 (R2 = (K - 1) / 2, conv2's reach), y1_lo = a2_lo - 6
// (the origin act_from_xs expects of its input row), a1_lo = y1_lo - dil R2
// (conv1's reach) and x_lo = a1_lo - 6. HBM sees x once (plus the residual
// re-read, an L2 hit), y once and sum_in once, against three tensor reads
// and two writes per conv when the convs run apart.
//
// Both convs run on v_mfma_f32_16x16x4f32: M = output channels in 16-row
// blocks, N = positions in 16-column blocks, K = (input channel, tap) in the
// order of pack_conv_weights16. Each wave keeps its row block's whole weight
// set in registers and streams the operand from LDS rows: one 4-byte read
// per lane gives 16 consecutive positions of 4 channels, with a row stride
// of 16 mod 64 floats, so the 64 lanes hit 64 distinct banks.
// ---------------------------------------------------------------------------
template <int C, int K, int T>
struct UnitGeom {
    static constexpr int R2 = (K - 1) / 2;
    static constexpr int W2 = T + 2 * R2;                      // act2 outputs (conv2 operand)
    static constexpr int XS2 = act_xs_len(W2);                 // Y1 row = act2 input row
    static constexpr int NY1 = (XS2 + 15) / 16 * 16;           // conv1 outputs computed
    static constexpr int W1MAX = NY1 + 2 * kUnitMaxDil * R2;   // act1 outputs at the widest dilation
    static constexpr int XS1MAX = act_xs_len(W1MAX);
    static constexpr int SA = (W1MAX + 47) / 64 * 64 + 16;     // A row stride: >= W1MAX, 16 mod 64
    static constexpr int XR = XS1MAX > XS2 ? XS1MAX : XS2;
    static constexpr int LDS_X = C * XR;
    static constexpr int LDS_A = C * SA;
    static constexpr int LDS_S = kChunk * act_ss_len(W1MAX);
    static constexpr int LDS_FLOATS = LDS_X + LDS_A + LDS_S;
    static_assert(C % kChunk == 0 && C <= 32, "8, 16 or 32 channels");
    static_assert(T % 16 == 0, "whole 16-column blocks");
};

// Work split of one unit conv over the four waves: MB row blocks, WPM waves
// per row block, each wave taking every WPM-th column block in NBAT batches
// of NBB blocks (accumulators in flight).
template <int C, int NOUT>
struct UnitConvSplit {
    static constexpr int MB = (C + 15) / 16;
    static constexpr int WPM = 4 / MB;
    static constexpr int NBLK = NOUT / 16;
    static constexpr int MYN = (NBLK + WPM - 1) / WPM;
    static constexpr int NBAT = (MYN + 5) / 6;
    static constexpr int NBB = (MYN + NBAT - 1) / NBAT;
};

// out[co][n] = bias[co] + sum_{ci, j} W[co][ci][j] A[ci][n + j dil] for n in
// [0, NOUT); A rows at stride SA. pre(q, mb, nb) runs before a batch's
// matrix-core work (for loads whose latency that work hides), epi(q, acc,
// mb, nb) after it, for each real block of the batch.
template <int C, int K, int SA, int NOUT, typename Pre, typename Epi>
__device__ __forceinline__ void unit_conv(const float* __restrict__ A, const float* __restrict__ wp,
                                          const float* __restrict__ bias, int dil, Pre pre, Epi epi) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    using S = UnitConvSplit<C, NOUT>;
    constexpr int G = (C / kChunk) * K;  // float2 weight groups: (chunk of 8 channels, tap)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mb = wave / S::WPM, ws = wave % S::WPM;
    float2 wr[G];
    const float2* wp2 = reinterpret_cast<const float2*>(wp) + (int64_t)mb * G * 64 + lane;
#pragma unroll
    for (int g = 0; g < G; ++g) wr[g] = wp2[g * 64];
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = mb * 16 + 4 * (lane >> 4) + r;
        bv[r] = co < C ? bias[co] : 0.0f;
    }
    const float* al = A + (lane >> 4) * SA + (lane & 15);
    for (int bt = 0; bt < S::NBAT; ++bt) {
        int nbq[S::NBB];
        v4f acc[S::NBB];
#pragma unroll
        for (int q = 0; q < S::NBB; ++q) {
            const int nb = ws + S::WPM * (bt * S::NBB + q);
            nbq[q] = nb < S::NBLK ? nb : S::NBLK - 1;  // spare slots repeat the last block
            if (nb < S::NBLK) pre(q, mb, nb);
            acc[q] = v4f{bv[0], bv[1], bv[2], bv[3]};
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
#pragma unroll
            for (int ch = 0; ch < C / kChunk; ++ch) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float wv = h ? wr[ch * K + j].y : wr[ch * K + j].x;
#pragma unroll
                    for (int q = 0; q < S::NBB; ++q) {
                        const float b = al[(ch * kChunk + 4 * h) * SA + nbq[q] * 16 + j * dil];
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv, b, acc[q], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < S::NBB; ++q) {
            const int nb = ws + S::WPM * (bt * S::NBB + q);
            if (nb < S::NBLK) epi(q, acc[q], mb, nb);
        }
    }
}

template <int C, int K, int T>
__global__ void __launch_bounds__(256, 2) unit_kernel(UnitArgs a) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    using G = UnitGeom<C, K, T>;
    using S2 = UnitConvSplit<C, T>;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xr = lds;               // x rows (stride act_xs_len(W1)), then Y1 rows (stride XS2)
    float* ar = lds + G::LDS_X;    // A1 rows, then A2 rows (stride SA)
    float* ss = ar + G::LDS_A;     // 2x-rate rows of the activation, one per channel in flight
    const int tid = threadIdx.x, lane = tid & 63;
    const int ci = tid >> 5, lane32 = tid & 31;
    const int b = blockIdx.y;
    const int p0 = blockIdx.x * T;
    const int L = a.l, dil = a.dil;
    const float* xb = a.x + (int64_t)b * a.bstride;
    const int a2_lo = p0 - G::R2, y1_lo = a2_lo - 6;
    const int W1 = G::NY1 + 2 * dil * G::R2;
    const int a1_lo = y1_lo - dil * G::R2, x_lo = a1_lo - 6;
    const int XS1 = act_xs_len(W1);

    const ActTaps f1 = load_act_taps(a.act1.taps);
    // x rows, replicate-clamped; each batch of 8 rows has all its loads in
    // flight before the stores
    {
        constexpr int NW = (G::XS1MAX + 255) / 256;
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += 8) {
            float v[8][NW];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < NW; ++u)
                    v[r][u] = xb[(c0 + r) * L + clampi(x_lo + tid + 256 * u, 0, L - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < NW; ++u)
                    if (tid + 256 * u < XS1) xr[(c0 + r) * XS1 + tid + 256 * u] = v[r][u];
        }
    }
    __syncthreads();
    // act1, 8 channels at a time (32 lanes per channel)
#pragma unroll
    for (int c0 = 0; c0 < C; c0 += kChunk) {
        act_from_xs<kChunk>(ar + c0 * G::SA, xr + c0 * XS1, ss, c0, C, L, a1_lo, W1, f1, a.act1.ab[c0 + ci], ci,
                            lane32, G::SA);
        wave_lds_sync();  // this wave's 2x-rate rows are reused by its next channels
    }
    __syncthreads();
    // conv1 -> Y1 rows
    unit_conv<C, K, G::SA, G::NY1>(
        ar, a.w1, a.b1, dil, [](int, int, int) {},
        [&](int, v4f acc, int mb, int nb) {
            const int n = nb * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = mb * 16 + 4 * (lane >> 4) + r;
                if (co < C && n < G::XS2) xr[co * G::XS2 + n] = acc[r];
            }
        });
    __syncthreads();
    // Y1 past the sequence ends repeats its edge values
    if (y1_lo < 0 || y1_lo + G::XS2 > L) {
        const int i0 = -y1_lo, i1 = L - 1 - y1_lo;  // row indices of positions 0 and L - 1
        for (int idx = tid; idx < C * G::XS2; idx += 256) {
            const int co = idx / G::XS2, w = idx - co * G::XS2;
            const int src = w < i0 ? i0 : (w > i1 ? i1 : -1);
            if (src >= 0) xr[co * G::XS2 + w] = xr[co * G::XS2 + src];
        }
        __syncthreads();
    }
    // act2 -> A2 rows (A1 is dead)
    {
        const ActTaps f2 = load_act_taps(a.act2.taps);
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += kChunk) {
            act_from_xs<kChunk>(ar + c0 * G::SA, xr + c0 * G::XS2, ss, c0, C, L, a2_lo, G::W2, f2, a.act2.ab[c0 + ci],
                                ci, lane32, G::SA);
            wave_lds_sync();
        }
    }
    __syncthreads();
    // conv2 + residual (+ running sum), scaled, -> y; the residual and sum
    // loads are issued before each batch's matrix-core work
    float rs[S2::NBB][4];
    const float* sb = a.sum_in ? a.sum_in + (int64_t)b * a.bstride : nullptr;
    float* yb = a.y + (int64_t)b * a.bstride;
    unit_conv<C, K, G::SA, T>(
        ar, a.w2, a.b2, 1,
        [&](int q, int mb, int nb) {
            const int n = min(p0 + nb * 16 + (lane & 15), L - 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = min(mb * 16 + 4 * (lane >> 4) + r, C - 1);
                rs[q][r] = xb[co * L + n] + (sb ? sb[co * L + n] : 0.0f);
            }
        },
        [&](int q, v4f acc, int mb, int nb) {
            const int n = p0 + nb * 16 + (lane & 15);
            if (n >= L) return;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = mb * 16 + 4 * (lane >> 4) + r;
                if (co < C) yb[co * L + n] = (acc[r] + rs[q][r]) * a.scale;
            }
        });
}

// Split-product form of the unit kernel: the same unit, with both convs on
// v_mfma_f32_16x16x32_bf16 over three bf16 pieces of the activations and of
// the weights (the six products of order <= 2, fp32 accumulation; see
// kPieces). K = 32 per instruction: lane l holds 8 consecutive channels of
// channel block cb at tap ks * TG + tsub, where (cb, tsub) enumerate the
// lane's K-group l / 16 (CB = C / 8 channel blocks, TG = 4 / CB taps per
// instruction; padded taps carry zero weights and re-read the last tap).
// LDS: the fp32 rows (x, then the activation in place, then Y1, then the
// second activation in place) and one region that is first the
// activation's 2x-rate scratch, then the pieces of A1, of A2:
// [piece][position][C bf16], one 16-byte group per (position, channel block).
template <int C, int K, int T>
struct Unit6Geom {
    using G = UnitGeom<C, K, T>;
    static constexpr int CB = C / 8, TG = 4 / CB, KS = (K + TG - 1) / TG;
    static constexpr int WP = G::W1MAX;                          // positions per piece plane
    static constexpr int PC = kPieces * WP * CB * 4;             // floats of the three planes
    static constexpr int SS = kChunk * act_ss_len(G::W1MAX);     // floats of the 2x-rate scratch
    static constexpr int LDS_P = PC > SS ? PC : SS;
    static constexpr int LDS_FLOATS = G::LDS_X + LDS_P;
    static_assert(C == 8 || C == 16 || C == 32, "8, 16 or 32 channels");
};

// fp32 rows (stride rs) of n positions -> pieces (16-byte group per
// position and channel block, planes of WP positions)
template <int C, int WP>
__device__ __forceinline__ void unit_pack6(const float* rows, int rs, int n, uint4* pc) {
    constexpr int CB = C / 8;
    for (int idx = threadIdx.x; idx < n * CB; idx += 256) {
        const int w = idx / CB, cb = idx - w * CB;
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = rows[(cb * 8 + i) * rs + w];
        uint4 g[kPieces];
        split3_pack8(v8, g);
#pragma unroll
        for (int p = 0; p < kPieces; ++p) pc[p * WP * CB + idx] = g[p];
    }
}

// out[co][n] = bias[co] + sum W[co][ci][j] A[ci][n + j dil], A as pieces
template <int C, int K, int WP, int NOUT, int NPROD, typename Pre, typename Epi>
__device__ __forceinline__ void unit_conv6(const uint4* __restrict__ pc, const float* __restrict__ wp,
                                           const float* __restrict__ bias, int dil, Pre pre, Epi epi) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
    using S = UnitConvSplit<C, NOUT>;
    constexpr int CB = C / 8, TG = 4 / CB, KS = (K + TG - 1) / TG;
    constexpr int NPU = NPROD == 3 ? 2 : kPieces;  // pieces used
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mb = wave / S::WPM, ws = wave % S::WPM;
    const int g4 = lane >> 4, cb = g4 % CB, tsub = g4 / CB, col = lane & 15;
    v4u wr[KS][kPieces];
    const v4u* w6 = reinterpret_cast<const v4u*>(wp) + (int64_t)mb * KS * kPieces * 64 + lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int p = 0; p < NPU; ++p) wr[ks][p] = w6[(ks * kPieces + p) * 64];
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = mb * 16 + 4 * g4 + r;
        bv[r] = co < C ? bias[co] : 0.0f;
    }
    const v4u* pcv = reinterpret_cast<const v4u*>(pc);
    constexpr int TA[6] = {0, 0, 1, 0, 1, 2}, TB[6] = {0, 1, 0, 2, 1, 0};
    for (int bt = 0; bt < S::NBAT; ++bt) {
        int nbq[S::NBB];
        v4f acc[S::NBB];
#pragma unroll
        for (int q = 0; q < S::NBB; ++q) {
            const int nb = ws + S::WPM * (bt * S::NBB + q);
            nbq[q] = nb < S::NBLK ? nb : S::NBLK - 1;
            if (nb < S::NBLK) pre(q, mb, nb);
            acc[q] = v4f{bv[0], bv[1], bv[2], bv[3]};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int tap = min(ks * TG + tsub, K - 1);  // padded taps re-read the last one (zero weights)
            const int off = (col + tap * dil) * CB + cb;
            v4u b[S::NBB][kPieces];
#pragma unroll
            for (int q = 0; q < S::NBB; ++q)
#pragma unroll
                for (int p = 0; p < NPU; ++p) b[q][p] = pcv[p * WP * CB + nbq[q] * 16 * CB + off];
#pragma unroll
            for (int t = 0; t < NPROD; ++t)
#pragma unroll
                for (int q = 0; q < S::NBB; ++q)
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wr[ks][TA[t]]),
                                                                     __builtin_bit_cast(v8bf, b[q][TB[t]]), acc[q], 0,
                                                                     0, 0);
        }
#pragma unroll
        for (int q = 0; q < S::NBB; ++q) {
            const int nb = ws + S::WPM * (bt * S::NBB + q);
            if (nb < S::NBLK) epi(q, acc[q], mb, nb);
        }
    }
}

template <int C, int K, int T, int NPROD>
__global__ void __launch_bounds__(256, 2) unit6_kernel(UnitArgs a) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    using G = UnitGeom<C, K, T>;
    using G6 = Unit6Geom<C, K, T>;
    using S2 = UnitConvSplit<C, T>;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xr = lds;                                             // fp32 rows
    uint4* pc = reinterpret_cast<uint4*>(lds + G::LDS_X);      // pieces (or the 2x-rate scratch)
    float* ss = lds + G::LDS_X;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ci = tid >> 5, lane32 = tid & 31;
    const int b = blockIdx.y;
    const int p0 = blockIdx.x * T;
    const int L = a.l, dil = a.dil;
    const float* xb = a.x + (int64_t)b * a.bstride;
    const int a2_lo = p0 - G::R2, y1_lo = a2_lo - 6;
    const int W1 = G::NY1 + 2 * dil * G::R2;
    const int a1_lo = y1_lo - dil * G::R2, x_lo = a1_lo - 6;
    const int XS1 = act_xs_len(W1);

    const ActTaps f1 = load_act_taps(a.act1.taps);
    {
        constexpr int NW = (G::XS1MAX + 255) / 256;
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += 8) {
            float v[8][NW];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < NW; ++u)
                    v[r][u] = xb[(c0 + r) * L + clampi(x_lo + tid + 256 * u, 0, L - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < NW; ++u)
                    if (tid + 256 * u < XS1) xr[(c0 + r) * XS1 + tid + 256 * u] = v[r][u];
        }
    }
    __syncthreads();
    // act1 in place over the x rows (a channel's x row is dead after its up pass)
#pragma unroll
    for (int c0 = 0; c0 < C; c0 += kChunk) {
        act_from_xs<kChunk>(xr + c0 * XS1, xr + c0 * XS1, ss, c0, C, L, a1_lo, W1, f1, a.act1.ab[c0 + ci], ci, lane32,
                            XS1);
        wave_lds_sync();
    }
    __syncthreads();
    unit_pack6<C, G6::WP>(xr, XS1, W1, pc);
    __syncthreads();
    // conv1 -> Y1 rows
    unit_conv6<C, K, G6::WP, G::NY1, NPROD>(
        pc, a.w1, a.b1, dil, [](int, int, int) {},
        [&](int, v4f acc, int mb, int nb) {
            const int n = nb * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = mb * 16 + 4 * (lane >> 4) + r;
                if (co < C && n < G::XS2) xr[co * G::XS2 + n] = acc[r];
            }
        });
    __syncthreads();
    if (y1_lo < 0 || y1_lo + G::XS2 > L) {
        const int i0 = -y1_lo, i1 = L - 1 - y1_lo;
        for (int idx = tid; idx < C * G::XS2; idx += 256) {
            const int co = idx / G::XS2, w = idx - co * G::XS2;
            const int src = w < i0 ? i0 : (w > i1 ? i1 : -1);
            if (src >= 0) xr[co * G::XS2 + w] = xr[co * G::XS2 + src];
        }
        __syncthreads();
    }
    {
        const ActTaps f2 = load_act_taps(a.act2.taps);
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += kChunk) {
            act_from_xs<kChunk>(xr + c0 * G::XS2, xr + c0 * G::XS2, ss, c0, C, L, a2_lo, G::W2, f2,
                                a.act2.ab[c0 + ci], ci, lane32, G::XS2);
            wave_lds_sync();
        }
    }
    __syncthreads();
    unit_pack6<C, G6::WP>(xr, G::XS2, G::W2, pc);
    __syncthreads();
    float rs[S2::NBB][4];
    const float* sb = a.sum_in ? a.sum_in + (int64_t)b * a.bstride : nullptr;
    float* yb = a.y + (int64_t)b * a.bstride;
    unit_conv6<C, K, G6::WP, T, NPROD>(
        pc, a.w2, a.b2, 1,
        [&](int q, int mb, int nb) {
            const int n = min(p0 + nb * 16 + (lane & 15), L - 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = min(mb * 16 + 4 * (lane >> 4) + r, C - 1);
                rs[q][r] = xb[co * L + n] + (sb ? sb[co * L + n] : 0.0f);
            }
        },
        [&](int q, v4f acc, int mb, int nb) {
            const int n = p0 + nb * 16 + (lane & 15);
            if (n >= L) return;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = mb * 16 + 4 * (lane >> 4) + r;
                if (co < C) yb[co * L + n] = (acc[r] + rs[q][r]) * a.scale;
            }
        });
}

template <int C, int K, int T, int NPROD>
static hipError_t launch_unit6_t(const UnitArgs& a, int batch, hipStream_t stream) {
    constexpr size_t lds = sizeof(float) * Unit6Geom<C, K, T>::LDS_FLOATS;
    static_assert(2 * lds <= 160 * 1024, "two workgroups per compute unit");
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)unit6_kernel<C, K, T, NPROD>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.l + T - 1) / T, batch);
    hipLaunchKernelGGL((unit6_kernel<C, K, T, NPROD>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

bool unit_supported(int c, int taps, int dil) {
    return (c == 8 || c == 16 || c == 32) && (taps == 3 || taps == 7 || taps == 11) && dil >= 1 &&
           dil <= kUnitMaxDil;
}

template <int C, int K, int T>
static hipError_t launch_unit_t(const UnitArgs& a, int batch, hipStream_t stream) {
    constexpr size_t lds = sizeof(float) * UnitGeom<C, K, T>::LDS_FLOATS;
    static_assert(2 * lds <= 160 * 1024, "two workgroups per compute unit");
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)unit_kernel<C, K, T>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.l + T - 1) / T, batch);
    hipLaunchKernelGGL((unit_kernel<C, K, T>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

// Tile widths: 128 positions at 32 channels, 256 at 16, 512 at 8 (about
// 60-80 KB of LDS each, two workgroups per compute unit).
hipError_t launch_unit(const UnitArgs& a, int batch, hipStream_t stream) {
    if (!unit_supported(a.c, a.taps, a.dil) || (a.split != 0 && a.split != 3 && a.split != 6) || a.l < 1 || batch < 1 ||
        batch > 65535 || !a.x || !a.y ||
        a.x == a.y || !a.w1 || !a.w2 || !a.b1 || !a.b2 || !a.act1.taps || !a.act2.taps)
        return hipErrorInvalidValue;
#define MH3A_UNIT(C_, K_, T_)                                                  \
    if (a.c == C_ && a.taps == K_)                                             \
        return a.split == 6   ? launch_unit6_t<C_, K_, T_, 6>(a, batch, stream)                             \
               : a.split == 3 ? launch_unit6_t<C_, K_, T_, 3>(a, batch, stream)                             \
                              : launch_unit_t<C_, K_, T_>(a, batch, stream);
    MH3A_UNIT(32, 3, 128) MH3A_UNIT(32, 7, 128) MH3A_UNIT(32, 11, 128)
    MH3A_UNIT(16, 3, 256) MH3A_UNIT(16, 7, 256) MH3A_UNIT(16, 11, 256)
    MH3A_UNIT(8, 3, 512) MH3A_UNIT(8, 7, 512) MH3A_UNIT(8, 11, 512)
#undef MH3A_UNIT
    return hipErrorInvalidValue;
}

// x (B, c, l) rows -> the split-product packed layout (kPieces planes per
// chunk of 8 channels, zero pads): one padded position per thread, the 8
// channels' pieces written as three 16-byte groups.
__global__ void __launch_bounds__(256) split_kernel(ActArgs a) {
    const int q = blockIdx.x * 256 + threadIdx.x;  // index in the padded row
    const int chunk = blockIdx.y, b = blockIdx.z;
    if (q >= a.lp) return;
    const int n = q - kPkPadL;
    const bool in = n >= 0 && n < a.l;
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    float v8[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const int ch = chunk * kChunk + i;
        v8[i] = (in && ch < a.c) ? xb[(int64_t)ch * a.l + n] : 0.0f;
    }
    uint4 g[kPieces];
    split3_pack8(v8, g);
    float* yc = a.y + (int64_t)b * a.y_bstride + (int64_t)chunk * kPieces * a.lp * 4;
#pragma unroll
    for (int p = 0; p < kPieces; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
}

hipError_t launch_split(const ActArgs& a, int batch, hipStream_t stream) {
    if (a.c < 1 || a.l < 1 || batch < 1 || batch > 65535 || a.pieces != kPieces || a.lp != a.l + kPkPadL + kPkPadR)
        return hipErrorInvalidValue;
    dim3 grid((a.lp + 255) / 256, (a.c + kChunk - 1) / kChunk, batch);
    hipLaunchKernelGGL(split_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Plain Snake with an optional space-to-depth regrouping (encoder):
// output channel c s + r at position t holds snake(x[c, t s + r - shift]),
// snake(v) = v + sin^2(alpha v) / (alpha + 1e-9) = v + hb (1 - cos(2 alpha v))
// with hb = 0.5 / (alpha + 1e-9), the cosine on the hardware unit as in
// snake_beta; zero outside [0, l) (the
// Snake of a zero is zero, so padding before or after it is the same).
// Packed output: one padded position of one 8-channel chunk per thread, as
// split_kernel. Plain output: one (channel, position) per thread.
__device__ __forceinline__ float snake_at(const SnakeArgs& a, const float* xb, int oc, int t) {
    const int c = oc / a.s, r = oc - c * a.s;
    const int64_t n = (int64_t)t * a.s + r - a.shift;
    if (c >= a.c || t < 0 || t >= a.l_out || n < 0 || n >= a.l) return 0.0f;
    const float2 ab = a.ab[c];
    return snake_beta(xb[(int64_t)c * a.l + n], ab.x, ab.y);
}

__global__ void __launch_bounds__(256) snake_packed_kernel(SnakeArgs a) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int chunk = blockIdx.y, b = blockIdx.z;
    if (q >= a.lp) return;
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    float v8[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) v8[i] = snake_at(a, xb, chunk * kChunk + i, q - kPkPadL);
    uint4 g[kPieces];
    split3_pack8(v8, g);
    float* yc = a.y + (int64_t)b * a.y_bstride + (int64_t)chunk * kPieces * a.lp * 4;
#pragma unroll
    for (int p = 0; p < kPieces; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
}

__global__ void __launch_bounds__(256) snake_rows_kernel(SnakeArgs a) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int oc = blockIdx.y, b = blockIdx.z;
    if (t >= a.l_out) return;
    a.y[(int64_t)b * a.y_bstride + (int64_t)oc * a.l_out + t] = snake_at(a, a.x + (int64_t)b * a.x_bstride, oc, t);
}

hipError_t launch_snake(const SnakeArgs& a, int batch, hipStream_t stream) {
    const int64_t oc = (int64_t)a.c * a.s;
    if (a.c < 1 || a.l < 1 || a.s < 1 || a.l_out < 1 || batch < 1 || batch > 65535 || oc > 65535 * (int64_t)kChunk)
        return hipErrorInvalidValue;
    if (a.lp > 0) {
        if (a.lp != a.l_out + kPkPadL + kPkPadR) return hipErrorInvalidValue;
        dim3 grid((a.lp + 255) / 256, (unsigned)((oc + kChunk - 1) / kChunk), batch);
        hipLaunchKernelGGL(snake_packed_kernel, grid, dim3(256), 0, stream, a);
    } else {
        if (oc > 65535) return hipErrorInvalidValue;
        dim3 grid((a.l_out + 255) / 256, (unsigned)oc, batch);
        hipLaunchKernelGGL(snake_rows_kernel, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_final(const FinalArgs& a, int batch, hipStream_t stream) {
    dim3 grid((a.l + kFinalT - 1) / kFinalT, batch);
    hipLaunchKernelGGL(final_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mh3a
