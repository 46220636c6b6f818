// gfx950 kernels of the BigVGAN decode path other than the conv kernel
// (mh3a_conv.h, one translation unit per tile shape), and the conv launch
// dispatch.
//
// act_kernel: the anti-aliased SnakeBeta alone, (B, C, L) rows -> the packed
//   operand layout, for AMP convs that take their activated input from
//   memory (their producer waves then copy it to LDS with no arithmetic).
// unit_kernel / unit6_kernel: one AMP residual unit of a narrow stage.
// final_kernel: activation_post + conv_post (C -> 1, k = 7, pad 3) + clamp.
// split_kernel / snake_*_kernel: the split-product input form, the
//   encoder's Snake.
//
// Method: FastVideo API docs "minimax_h3_audio_vae" (MLXMiniMaxH3AudioVAE.decode,
// module overview), diffusers docs "AutoencoderKLMiniMaxH3Audio" (decode).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "mh3a_device.h"
#include "mh3a_internal.h"
#include "mh3a_tiles.h"

namespace mh3a {

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

hipError_t launch_conv(const ConvArgs& a, TileId tile, hipStream_t stream) {
    // the kernel cuts the chunks into ksplit equal ranges
    const int nch = (a.c_in + kChunk - 1) / kChunk;
    if (a.ksplit < 1 || nch % a.ksplit != 0 || (a.ksplit > 1 && !a.partial)) return hipErrorInvalidValue;
    if (tile == TILE_16x256) return launch_tile_of<TILE_16x256>(a, stream);
    hipError_t e = hipSuccess;
    switch (tile) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: e = launch_tile_of<id>(a, stream); break;
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
        // clamp to [-1, 1]; NaN stays NaN (as torch.clamp and mx.clip do):
        // fmax / fmin alone would map it to -1 and hide a non-finite signal
        if (a.clamp && !__builtin_isnan(v)) v = fminf(fmaxf(v, -1.0f), 1.0f);
        a.y[(int64_t)b * a.l + t] = v;
    }
}

// ---------------------------------------------------------------------------
// Standalone activation: a workgroup owns kActT padded positions of kChunk
// channels (32 threads per channel, as in the conv producers), computes them
// into LDS rows and stores them packed: each thread writes the 16-byte group
// of one (hi, position), so every wave stores 1 KB contiguous.
// ---------------------------------------------------------------------------
// Interior tiles take four up-sampling pairs and four outputs per lane
// (act_interior4): W + 6 = 128 pairs and 122 outputs are one pass of 32
// lanes per channel, and 8 workgroups fill a CU's 32 wave slots. (Measured
// 1.7% faster than two per lane on 186-position tiles; the build-time
// options MH3A_ACT_T / MH3A_ACT_P = 2 select other widths and the two-per-lane path.)
#ifndef MH3A_ACT_T
#define MH3A_ACT_T 122
#endif
#ifndef MH3A_ACT_P
#define MH3A_ACT_P 4
#endif
constexpr int kActT = MH3A_ACT_T;
constexpr int kActP = MH3A_ACT_P;
static_assert(kActP == 2 || (kActP == 4 && kActT % 4 == 2), "four per lane needs W = 2 mod 4");

// PC: 0 writes the fp32 packed layout (two channel-parity planes); kPieces /
// kPiecesH the split-product forms (bf16 x 3 / fp16 x 2 planes).
template <int W, int PC>
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
    constexpr int NPL = PC ? PC : 2;  // planes per chunk: pieces, or channel parities
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
    stage_act<CI, W, kActP>(as, xs, ss, a.x + (int64_t)b * a.x_bstride, chunk * CI, a.c, a.l, t0, f, a.act.ab, ci,
                            lane32, XS);
    __syncthreads();
    if constexpr (PC != 0) {
        // one position per thread: the 8 channels' pieces, 16 bytes per plane
        for (int w = threadIdx.x; w < W; w += 256) {
            const int q = t0 + kPkPadL + w;
            if (q >= a.lp) continue;
            static_assert(CI == 8, "one 16-byte group per piece");
            float v8[8];
#pragma unroll
            for (int c = 0; c < CI; ++c) v8[c] = as[c * XS + w];
            uint4 g[PC];
            split_pack8<PC>(v8, g);
#pragma unroll
            for (int p = 0; p < PC; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
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
    if (a.pieces == kPieces)
        hipLaunchKernelGGL((act_kernel<kActT, kPieces>), grid, dim3(256), 0, stream, a);
    else if (a.pieces == kPiecesH)
        hipLaunchKernelGGL((act_kernel<kActT, kPiecesH>), grid, dim3(256), 0, stream, a);
    else if (a.pieces == 0)
        hipLaunchKernelGGL((act_kernel<kActT, 0>), grid, dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Transposed conv of the narrow stages (8-32 channels) on the vector ALU. In
// the polyphase form output t = R m + ph is the bias plus, over input
// channels i and taps q with (ph + P - q) divisible by R (P = (K - R) / 2),
// W[i][o][q] x[i][m + (ph + P - q) / R], zero outside the sequence. A
// workgroup owns 256 input positions of one batch item: their window of x
// (every channel) is staged in LDS, and each thread produces all R phases
// of its position for every output channel (R CO accumulators). The weights
// are read at uniform addresses (scalar loads); the outputs of a position
// are R consecutive floats per channel, stored as one vector per thread.
// HBM sees x once and y once; these stages have too few channels to fill
// matrix-core tiles (a 32-row block would be half padding at 16 outputs).
// ---------------------------------------------------------------------------
constexpr int ups_off_min(int R, int K) {
    int v = 1 << 20;
    for (int ph = 0; ph < R; ++ph)
        for (int q = 0; q < K; ++q)
            if ((ph + (K - R) / 2 - q) % R == 0 && (ph + (K - R) / 2 - q) / R < v) v = (ph + (K - R) / 2 - q) / R;
    return v;
}
constexpr int ups_off_max(int R, int K) {
    int v = -(1 << 20);
    for (int ph = 0; ph < R; ++ph)
        for (int q = 0; q < K; ++q)
            if ((ph + (K - R) / 2 - q) % R == 0 && (ph + (K - R) / 2 - q) / R > v) v = (ph + (K - R) / 2 - q) / R;
    return v;
}
constexpr int kUpsT = 256;

template <int CI, int CO, int R, int K>
__global__ void __launch_bounds__(256) ups_vec_kernel(UpsVecArgs a) {
    constexpr int P = (K - R) / 2;
    constexpr int DLO = ups_off_min(R, K), DHI = ups_off_max(R, K);
    constexpr int ND = DHI - DLO + 1;
    constexpr int XW = kUpsT + ND - 1;
    __shared__ float xs[CI * XW];
    const int b = blockIdx.y;
    const int m0 = blockIdx.x * kUpsT;
    const int L = a.l;
    const float* xb = a.x + (int64_t)b * CI * L;
    for (int idx = threadIdx.x; idx < CI * XW; idx += 256) {
        const int i = idx / XW, w = idx - i * XW;
        const int m = m0 + DLO + w;
        xs[idx] = (m >= 0 && m < L) ? xb[(int64_t)i * L + m] : 0.0f;
    }
    __syncthreads();
    const int m = m0 + threadIdx.x;
    if (m >= L) return;
    float acc[R][CO];
#pragma unroll
    for (int o = 0; o < CO; ++o) {
        const float bo = a.bias[o];
#pragma unroll
        for (int ph = 0; ph < R; ++ph) acc[ph][o] = bo;
    }
    const float* __restrict__ w = a.w;
#pragma unroll 2
    for (int i = 0; i < CI; ++i) {
        float xv[ND];
#pragma unroll
        for (int e = 0; e < ND; ++e) xv[e] = xs[i * XW + threadIdx.x + e];
#pragma unroll
        for (int ph = 0; ph < R; ++ph)
#pragma unroll
            for (int q = 0; q < K; ++q) {
                if ((ph + P - q) % R != 0) continue;
                const float xq = xv[(ph + P - q) / R - DLO];
#pragma unroll
                for (int o = 0; o < CO; ++o) acc[ph][o] = fmaf(w[(i * CO + o) * K + q], xq, acc[ph][o]);
            }
    }
    float* yb = a.y + (int64_t)b * CO * R * L + (int64_t)R * m;
#pragma unroll
    for (int o = 0; o < CO; ++o) {
        if constexpr (R == 2) {
            *reinterpret_cast<float2*>(yb + (int64_t)o * R * L) = make_float2(acc[0][o], acc[1][o]);
        } else {
#pragma unroll
            for (int ph = 0; ph < R; ++ph) yb[(int64_t)o * R * L + ph] = acc[ph][o];
        }
    }
}

bool ups_vec_supported(int ci, int co, int r, int k) {
    return r == 2 && k == 4 && ((ci == 32 && co == 16) || (ci == 16 && co == 8));
}

hipError_t launch_ups_vec(const UpsVecArgs& a, int batch, hipStream_t stream) {
    if (!ups_vec_supported(a.ci, a.co, a.r, a.k) || a.l < 1 || batch < 1 || batch > 65535 || !a.x || !a.y ||
        !a.w || !a.bias || a.x == a.y)
        return hipErrorInvalidValue;
    dim3 grid((a.l + kUpsT - 1) / kUpsT, batch);
    if (a.ci == 32)
        hipLaunchKernelGGL((ups_vec_kernel<32, 16, 2, 4>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((ups_vec_kernel<16, 8, 2, 4>), grid, dim3(256), 0, stream, a);
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
                            lane32, G::SA, XS1);
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
                                ci, lane32, G::SA, G::XS2);
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
// v_mfma_f32_16x16x32_{bf16,f16} over pieces of the activations and of the
// weights (fp32 accumulation; see kPieces, kPiecesH). K = 32 per
// instruction: lane l holds 8 consecutive channels of channel block cb at
// tap ks * TG + tsub, where (cb, tsub) enumerate the lane's K-group l / 16
// (CB = C / 8 channel blocks, TG = 4 / CB taps per instruction; padded taps
// carry zero weights and re-read the last tap).
// LDS: the fp32 rows (x, then the activation in place, then Y1, then the
// second activation in place) and one region that is first the
// activation's 2x-rate scratch, then the pieces of A1, of A2:
// [piece][C / 8][position][8 channels], one 16-byte group per (piece,
// channel block, position). Rows are laid out at a stride of 4 mod 16
// floats, which keeps conv1's stores of Y1 free of LDS bank conflicts.
// conv1 runs whole 16-column blocks over the NX2 positions act2 reads; the
// columns past NX2 read stale pieces beyond A1 (inside the planes) and are
// never stored, so act1 covers only NX2 + 2 dil R2 positions.
__host__ __device__ constexpr int unit_row_stride(int n) { return ((n + 11) & ~15) + 4; }

template <int C, int K, int T, int NPC>
struct Unit6Geom {
    static constexpr int R2 = (K - 1) / 2;
    static constexpr int W2 = T + 2 * R2;                          // act2 outputs (conv2 operand)
    static constexpr int NX2 = W2 + 12;                            // Y1 positions = act2's input row
    static constexpr int RS2 = unit_row_stride(NX2);
    static constexpr int NY1 = (NX2 + 15) / 16 * 16;               // conv1 outputs computed
    static constexpr int W1MAX = NY1 + 2 * kUnitMaxDil * R2;       // conv1's operand reach at the widest dilation
    static constexpr int RS1MAX = unit_row_stride(NX2 + 2 * kUnitMaxDil * R2 + 12);
    static constexpr int XR = RS1MAX > RS2 ? RS1MAX : RS2;
    static constexpr int LDS_X = C * XR;
    static constexpr int CB = C / 8, TG = 4 / CB, KS = (K + TG - 1) / TG;
    static constexpr int WP = W1MAX;                               // positions per piece plane
    static constexpr int PC = NPC * WP * CB * 4;                   // floats of the piece planes
    static constexpr int SS = kChunk * act_ss_len(W1MAX);          // floats of the 2x-rate scratch
    static constexpr int LDS_P = PC > SS ? PC : SS;
    static constexpr int LDS_FLOATS = LDS_X + LDS_P;
    static_assert(C == 8 || C == 16 || C == 32, "8, 16 or 32 channels");
    static_assert(T % 16 == 0, "whole 16-column blocks");
};

// fp32 rows (stride rs) of n positions -> pieces: plane p holds, per channel
// block cb, WP consecutive 16-byte groups (the 8 channels of the block at
// one position). A wave's items are consecutive positions of one block, so
// its 8 row reads and its piece stores are contiguous (no bank conflicts),
// and so are the conv's operand reads (16 consecutive positions per
// 16-lane group). NPC = kPieces bf16 or kPiecesH fp16 pieces.
template <int C, int WP, int NPC>
__device__ __forceinline__ void unit_pack6(const float* rows, int rs, int n, uint4* pc) {
    constexpr int CB = C / 8;
    for (int idx = threadIdx.x; idx < n * CB; idx += 256) {
        const int cb = idx / n, w = idx - cb * n;
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = rows[(cb * 8 + i) * rs + w];
        uint4 g[NPC];
        split_pack8<NPC>(v8, g);
#pragma unroll
        for (int p = 0; p < NPC; ++p) pc[(p * CB + cb) * WP + w] = g[p];
    }
}

// out[co][n] = bias[co] + sum W[co][ci][j] A[ci][n + j dil], A as pieces.
// PF: 6 = bf16 pieces, six products; 3 = bf16 pieces, three; 2 = fp16
// pieces, three, the weights scaled by wscale (2^e) and the sums by its
// inverse before epi.
template <int C, int K, int WP, int NOUT, int PF, typename Pre, typename Epi>
__device__ __forceinline__ void unit_conv6(const uint4* __restrict__ pc, const float* __restrict__ wp,
                                           const float* __restrict__ bias, int dil, float wscale, Pre pre, Epi epi) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
    typedef _Float16 v8h __attribute__((ext_vector_type(8)));
    using S = UnitConvSplit<C, NOUT>;
    constexpr bool H16 = PF == 2;
    constexpr int NPROD = PF == 6 ? 6 : 3;
    constexpr int NPW = H16 ? kPiecesH : kPieces;  // weight pieces in the packing
    constexpr int NPU = NPROD == 3 ? 2 : kPieces;  // pieces used
    constexpr int CB = C / 8, TG = 4 / CB, KS = (K + TG - 1) / TG;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mb = wave / S::WPM, ws = wave % S::WPM;
    const int g4 = lane >> 4, cb = g4 % CB, tsub = g4 / CB, col = lane & 15;
    v4u wr[KS][NPW];
    const v4u* w6 = reinterpret_cast<const v4u*>(wp) + (int64_t)mb * KS * NPW * 64 + lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int p = 0; p < NPU; ++p) wr[ks][p] = w6[(ks * NPW + p) * 64];
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = mb * 16 + 4 * g4 + r;
        bv[r] = co < C ? bias[co] : 0.0f;
        if constexpr (H16) bv[r] *= wscale;  // the sums carry 2^e until epi
    }
    const float out_scale = 1.0f / wscale;  // exact: a power of two
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
            const int off = cb * WP + col + tap * dil;
            v4u b[S::NBB][NPW];
#pragma unroll
            for (int q = 0; q < S::NBB; ++q)
#pragma unroll
                for (int p = 0; p < NPU; ++p) b[q][p] = pcv[p * WP * CB + nbq[q] * 16 + off];
#pragma unroll
            for (int t = 0; t < NPROD; ++t)
#pragma unroll
                for (int q = 0; q < S::NBB; ++q) {
                    if constexpr (H16)
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, wr[ks][TA[t]]),
                                                                        __builtin_bit_cast(v8h, b[q][TB[t]]), acc[q],
                                                                        0, 0, 0);
                    else
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, wr[ks][TA[t]]),
                                                                         __builtin_bit_cast(v8bf, b[q][TB[t]]), acc[q],
                                                                         0, 0, 0);
                }
        }
#pragma unroll
        for (int q = 0; q < S::NBB; ++q) {
            const int nb = ws + S::WPM * (bt * S::NBB + q);
            if constexpr (H16) acc[q] *= out_scale;
            if (nb < S::NBLK) epi(q, acc[q], mb, nb);
        }
    }
}

// DIL > 0 fixes the dilation at compile time (then row strides, window
// widths and conv1's tap offsets are constants: the pieces' pack loop needs
// no runtime division and its row reads take immediate offsets); DIL = 0
// reads it from the arguments.
template <int C, int K, int T, int PF, int OCC, int DIL>
__global__ void __launch_bounds__(256, OCC) unit6_kernel(UnitArgs a) {
    constexpr int NPC = PF == 2 ? kPiecesH : kPieces;  // pieces per value in LDS
    typedef float v4f __attribute__((ext_vector_type(4)));
    using G6 = Unit6Geom<C, K, T, NPC>;
    using S2 = UnitConvSplit<C, T>;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xr = lds;                                             // fp32 rows
    uint4* pc = reinterpret_cast<uint4*>(lds + G6::LDS_X);     // pieces (or the 2x-rate scratch)
    float* ss = lds + G6::LDS_X;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ci = tid >> 5, lane32 = tid & 31;
    const int b = blockIdx.y;
    const int p0 = blockIdx.x * T;
    const int L = a.l, dil = DIL > 0 ? DIL : a.dil;
    const float* xb = a.x + (int64_t)b * a.bstride;
    const int a2_lo = p0 - G6::R2, y1_lo = a2_lo - 6;
    const int W1 = G6::NX2 + 2 * dil * G6::R2;
    const int a1_lo = y1_lo - dil * G6::R2, x_lo = a1_lo - 6;
    const int NX1 = W1 + 12, RS1 = unit_row_stride(NX1);

    const ActTaps f1 = load_act_taps(a.act1.taps);
    {
        constexpr int NW = (G6::NX2 + 2 * (DIL > 0 ? DIL : kUnitMaxDil) * G6::R2 + 12 + 255) / 256;
        // inside the sequence: one address per row, the loads at immediate offsets
        const bool inside = x_lo >= 0 && x_lo + 256 * NW <= L;
        const int pos0 = inside ? x_lo + tid : 0;
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += 8) {
            float v[8][NW];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float* row = xb + (int64_t)(c0 + r) * L;
                if (inside) {
#pragma unroll
                    for (int u = 0; u < NW; ++u) v[r][u] = row[pos0 + 256 * u];
                } else {
#pragma unroll
                    for (int u = 0; u < NW; ++u) v[r][u] = row[clampi(x_lo + tid + 256 * u, 0, L - 1)];
                }
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int u = 0; u < NW; ++u)
                    if (tid + 256 * u < NX1) xr[(c0 + r) * RS1 + tid + 256 * u] = v[r][u];
        }
    }
    __syncthreads();
    // act1 in place over the x rows (a channel's x row is dead after its up pass)
#pragma unroll
    for (int c0 = 0; c0 < C; c0 += kChunk) {
        act_from_xs<kChunk>(xr + c0 * RS1, xr + c0 * RS1, ss, c0, C, L, a1_lo, W1, f1, a.act1.ab[c0 + ci], ci, lane32,
                            RS1, RS1);
        wave_lds_sync();
    }
    __syncthreads();
    unit_pack6<C, G6::WP, NPC>(xr, RS1, W1, pc);
    __syncthreads();
    // conv1 -> Y1 rows
    unit_conv6<C, K, G6::WP, G6::NY1, PF>(
        pc, a.w1, a.b1, dil, a.wscale1, [](int, int, int) {},
        [&](int, v4f acc, int mb, int nb) {
            const int n = nb * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = mb * 16 + 4 * (lane >> 4) + r;
                if (co < C && n < G6::NX2) xr[co * G6::RS2 + n] = acc[r];
            }
        });
    __syncthreads();
    if (y1_lo < 0 || y1_lo + G6::NX2 > L) {
        const int i0 = -y1_lo, i1 = L - 1 - y1_lo;
        for (int idx = tid; idx < C * G6::NX2; idx += 256) {
            const int co = idx / G6::NX2, w = idx - co * G6::NX2;
            const int src = w < i0 ? i0 : (w > i1 ? i1 : -1);
            if (src >= 0) xr[co * G6::RS2 + w] = xr[co * G6::RS2 + src];
        }
        __syncthreads();
    }
    {
        const ActTaps f2 = load_act_taps(a.act2.taps);
#pragma unroll
        for (int c0 = 0; c0 < C; c0 += kChunk) {
            act_from_xs<kChunk>(xr + c0 * G6::RS2, xr + c0 * G6::RS2, ss, c0, C, L, a2_lo, G6::W2, f2,
                                a.act2.ab[c0 + ci], ci, lane32, G6::RS2, G6::RS2);
            wave_lds_sync();
        }
    }
    __syncthreads();
    unit_pack6<C, G6::WP, NPC>(xr, G6::RS2, G6::W2, pc);
    __syncthreads();
    float rs[S2::NBB][4];
    const float* sb = a.sum_in ? a.sum_in + (int64_t)b * a.bstride : nullptr;
    float* yb = a.y + (int64_t)b * a.bstride;
    unit_conv6<C, K, G6::WP, T, PF>(
        pc, a.w2, a.b2, 1, a.wscale2,
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

template <int C, int K, int T, int PF, int OCC, int DIL>
static hipError_t launch_unit6_t(const UnitArgs& a, int batch, hipStream_t stream) {
    constexpr int NPC = PF == 2 ? kPiecesH : kPieces;
    constexpr size_t lds = sizeof(float) * Unit6Geom<C, K, T, NPC>::LDS_FLOATS;
    static_assert(OCC * lds <= 160 * 1024, "OCC workgroups per compute unit");
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)unit6_kernel<C, K, T, PF, OCC, DIL>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.l + T - 1) / T, batch);
    hipLaunchKernelGGL((unit6_kernel<C, K, T, PF, OCC, DIL>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

// The default (fp16 piece) form has instances for the dilations 1, 3 and 5
// of the residual blocks; other dilations and forms read it at run time.
template <int C, int K, int T, int PF, int OCC>
static hipError_t launch_unit6_d(const UnitArgs& a, int batch, hipStream_t stream) {
    if constexpr (PF == 2) {
        if (a.dil == 1) return launch_unit6_t<C, K, T, PF, OCC, 1>(a, batch, stream);
        if (a.dil == 3) return launch_unit6_t<C, K, T, PF, OCC, 3>(a, batch, stream);
        if (a.dil == 5) return launch_unit6_t<C, K, T, PF, OCC, 5>(a, batch, stream);
    }
    return launch_unit6_t<C, K, T, PF, OCC, 0>(a, batch, stream);
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

// Tile widths of the split-product unit kernels (positions T, workgroups per
// compute unit OCC, from the LDS size): the widest tiles that keep three or
// four workgroups resident, so that one workgroup's loads and barriers
// overlap the others' vector and matrix work. The fp32 form keeps 128
// positions at 32 channels, 256 at 16 and 512 at 8 (two workgroups).
hipError_t launch_unit(const UnitArgs& a, int batch, hipStream_t stream) {
    if (!unit_supported(a.c, a.taps, a.dil) || (a.split != 0 && a.split != 2 && a.split != 3 && a.split != 6) ||
        a.l < 1 || batch < 1 ||
        batch > 65535 || !a.x || !a.y ||
        a.x == a.y || !a.w1 || !a.w2 || !a.b1 || !a.b2 || !a.act1.taps || !a.act2.taps)
        return hipErrorInvalidValue;
#define MH3A_UNIT(C_, K_, T0_, T6_, O6_, T2_, O2_)                                                     \
    if (a.c == C_ && a.taps == K_)                                                                     \
        return a.split == 6   ? launch_unit6_d<C_, K_, T6_, 6, O6_>(a, batch, stream)                   \
               : a.split == 3 ? launch_unit6_d<C_, K_, T6_, 3, O6_>(a, batch, stream)                   \
               : a.split == 2 ? launch_unit6_d<C_, K_, T2_, 2, O2_>(a, batch, stream)                   \
                              : launch_unit_t<C_, K_, T0_>(a, batch, stream);
    //        C   K  fp32  bf16 pieces  fp16 pieces
    MH3A_UNIT(32, 3, 128,  96, 3,       112, 4)
    MH3A_UNIT(32, 7, 128,  96, 3,       112, 3)
    MH3A_UNIT(32, 11, 128, 96, 2,       112, 3)
    MH3A_UNIT(16, 3, 256,  176, 4,      240, 4)
    MH3A_UNIT(16, 7, 256,  192, 3,      224, 4)
    MH3A_UNIT(16, 11, 256, 192, 3,      240, 3)
    MH3A_UNIT(8, 3, 512,   384, 3,      384, 4)
    MH3A_UNIT(8, 7, 512,   336, 3,      336, 3)
    MH3A_UNIT(8, 11, 512,  320, 3,      320, 4)
#undef MH3A_UNIT
    return hipErrorInvalidValue;
}

// x (B, c, l) rows -> a split-product packed layout (PC planes per chunk of
// 8 channels, zero pads; PC = kPieces bf16 or kPiecesH fp16 pieces): one
// padded position per thread, the 8 channels' pieces written as PC 16-byte
// groups.
template <int PC>
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
    uint4 g[PC];
    split_pack8<PC>(v8, g);
    float* yc = a.y + (int64_t)b * a.y_bstride + (int64_t)chunk * PC * a.lp * 4;
#pragma unroll
    for (int p = 0; p < PC; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
}

hipError_t launch_split(const ActArgs& a, int batch, hipStream_t stream) {
    if (a.c < 1 || a.l < 1 || batch < 1 || batch > 65535 || a.lp != a.l + kPkPadL + kPkPadR) return hipErrorInvalidValue;
    dim3 grid((a.lp + 255) / 256, (a.c + kChunk - 1) / kChunk, batch);
    if (a.pieces == kPieces)
        hipLaunchKernelGGL(split_kernel<kPieces>, grid, dim3(256), 0, stream, a);
    else if (a.pieces == kPiecesH)
        hipLaunchKernelGGL(split_kernel<kPiecesH>, grid, dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
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

template <int PC>
__global__ void __launch_bounds__(256) snake_packed_kernel(SnakeArgs a) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int chunk = blockIdx.y, b = blockIdx.z;
    if (q >= a.lp) return;
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    float v8[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) v8[i] = snake_at(a, xb, chunk * kChunk + i, q - kPkPadL);
    uint4 g[PC];
    split_pack8<PC>(v8, g);
    float* yc = a.y + (int64_t)b * a.y_bstride + (int64_t)chunk * PC * a.lp * 4;
#pragma unroll
    for (int p = 0; p < PC; ++p) *reinterpret_cast<uint4*>(yc + ((int64_t)p * a.lp + q) * 4) = g[p];
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
        if (a.lp != a.l_out + kPkPadL + kPkPadR || (a.pieces != kPieces && a.pieces != kPiecesH))
            return hipErrorInvalidValue;
        dim3 grid((a.lp + 255) / 256, (unsigned)((oc + kChunk - 1) / kChunk), batch);
        if (a.pieces == kPiecesH)
            hipLaunchKernelGGL(snake_packed_kernel<kPiecesH>, grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(snake_packed_kernel<kPieces>, grid, dim3(256), 0, stream, a);
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
