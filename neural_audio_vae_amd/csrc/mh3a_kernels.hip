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
// final_kernel: activation_post + conv_post (C -> 1, k = 7, pad 3) + clamp.
//
// Method: FastVideo API docs "minimax_h3_audio_vae" (MLXMiniMaxH3AudioVAE.decode,
// module overview), diffusers docs "AutoencoderKLMiniMaxH3Audio" (decode).

#include <hip/hip_runtime.h>

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
// LDS: xs[CI][W + 12] holds X[n_lo - 6 ...], ss[CI][2W + 12] holds
// s[clamp(2 n_lo - 5 + mm)], as[CI][W] the result.
template <int CI>
__device__ __forceinline__ void stage_act(float* __restrict__ as, float* __restrict__ xs, float* __restrict__ ss,
                                          const float* __restrict__ xb, int ch0, int c_in, int l_in, int n_lo,
                                          int W, const ActParams& ap, int ci, int lane32) {
    const int ch = ch0 + ci;
    const bool live = ch < c_in;
    const int XS = W + 12, SS = 2 * W + 12;
    float* xrow = xs + ci * XS;
    float* srow = ss + ci * SS;
    float* arow = as + ci * W;
    const float* xc = xb + (int64_t)(live ? ch : 0) * l_in;
    for (int w = lane32; w < XS; w += 32) {
        xrow[w] = live ? xc[clampi(n_lo - 6 + w, 0, l_in - 1)] : 0.0f;
    }
    wave_lds_sync();
    const float* tp = ap.taps;
    float fe[6], fo[6];
#pragma unroll
    for (int e = 0; e < 6; ++e) {
        fe[e] = tp[e];
        fo[e] = tp[6 + e];
    }
    float2 ab = live ? ap.ab[ch] : make_float2(0.0f, 0.0f);
    // pairs t' = n_lo - 3 + idx, idx in [0, W + 6): slot 2 idx - 1 <- s[2t'], slot 2 idx <- s[2t' + 1]
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
        if (idx > 0) srow[2 * idx - 1] = se;
        srow[2 * idx] = so;
    }
    wave_lds_sync();
    float fd[12];
#pragma unroll
    for (int q = 0; q < 12; ++q) fd[q] = tp[12 + q];
    for (int w = lane32; w < W; w += 32) {
        const int n = n_lo + w;
        float v = 0.0f;
        if (live && n >= 0 && n < l_in) {
            const float* sv = srow + 2 * w;
#pragma unroll
            for (int q = 0; q < 12; ++q) v = fmaf(fd[q], sv[q], v);
        }
        arow[w] = v;
    }
}

// Plain staging: as[ci][w] = x[ch0 + ci, n_lo + w], zero outside.
__device__ __forceinline__ void stage_plain(float* __restrict__ as, const float* __restrict__ xb, int ch0, int c_in,
                                            int l_in, int n_lo, int W, int ci, int lane32) {
    const int ch = ch0 + ci;
    const bool live = ch < c_in;
    const float* xc = xb + (int64_t)(live ? ch : 0) * l_in;
    float* arow = as + ci * W;
    for (int w = lane32; w < W; w += 32) {
        const int n = n_lo + w;
        arow[w] = (live && n >= 0 && n < l_in) ? xc[n] : 0.0f;
    }
}

__device__ __forceinline__ float round_bf16(float v) {
    // round to nearest even at bfloat16 precision, kept in an fp32 register
    unsigned u = __float_as_uint(v);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return __uint_as_float(u);
}

// LDS floats of the conv kernel for window width W.
__host__ __device__ constexpr int conv_lds_floats(int W, bool act) {
    return 2 * kChunk * W + (act ? kChunk * (W + 12) + kChunk * (2 * W + 12) : 0);
}

// Wave-specialized implicit-GEMM conv. 512 threads: waves 0-3 are the
// consumers (matrix-core loop, WM x WN of them, each MBW x NBW blocks of
// 32 x 32 outputs); waves 4-7 are the producers, which stage the next
// K-chunk's (activated) input window into the other half of a
// double-buffered LDS tile while the consumers work on the current one.
// One workgroup barrier per chunk hands the buffers over.
template <int MBW, int NBW, int WM, int WN, bool ACT, bool BF16>
__global__ void __launch_bounds__(512) conv_kernel(ConvArgs a) {
    static_assert(WM * WN == 4, "four consumer waves");
    constexpr int CI = kChunk;
    constexpr int NWG = WN * NBW * 32;
    constexpr int MWG = WM * MBW * 32;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool producer = wave >= 4;
    const int ph = blockIdx.z % a.phases;
    const int b = blockIdx.z / a.phases;
    const int p0 = blockIdx.x * NWG;
    const int m0 = blockIdx.y * MWG;
    const int W = NWG + (a.taps - 1) * a.dil;
    const int n_lo = p0 + a.in_off[ph];
    float* abuf = lds;                       // [2][CI][W]
    float* xs = lds + 2 * CI * W;            // [CI][W + 12]   (act only)
    float* ss = xs + CI * (W + 12);          // [CI][2W + 12]  (act only)
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    const int nch = (a.c_in + CI - 1) / CI;
    const int G = nch * a.taps;

    // producer identity: 256 threads, 32 per channel
    const int ptid = tid - 256;
    const int pci = ptid >> 5, plane = ptid & 31;

    // consumer identity
    const int wm = wave % WM, wn = wave / WM;
    const int mb_tot = (a.c_out + 31) >> 5;
    const int mb_base = (m0 >> 5) + wm * MBW;
    const bool wave_live = !producer && mb_base < mb_tot;
    const int hi = lane >> 5, lo = lane & 31;
    const int colbase = wn * NBW * 32 + lo;
    const float4* wp = reinterpret_cast<const float4*>(a.w + (int64_t)ph * a.w_phase_stride);

    auto stage = [&](int c, float* dst) {
        if constexpr (ACT) {
            stage_act<CI>(dst, xs, ss, xb, c * CI, a.c_in, a.l_in, n_lo, W, a.act, pci, plane);
        } else {
            stage_plain(dst, xb, c * CI, a.c_in, a.l_in, n_lo, W, pci, plane);
        }
    };

    v16f acc[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    float4 An[MBW];
    auto load_a = [&](int g) {
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int mbg = mb_base + mb;
            An[mb] = (mbg < mb_tot && g < G) ? wp[((int64_t)mbg * G + g) * 64 + lane]
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    if (producer) stage(0, abuf);
    if (wave_live) load_a(0);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        if (producer) {
            if (c + 1 < nch) stage(c + 1, abuf + ((c + 1) & 1) * CI * W);
        } else if (wave_live) {
            const float* cur = abuf + (c & 1) * CI * W;
            for (int j = 0; j < a.taps; ++j) {
                const int g = c * a.taps + j;
                float4 Ac[MBW];
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) Ac[mb] = An[mb];
                load_a(g + 1);
                const float* brow = cur + hi * W + colbase + j * a.dil;
                float Bv[4][NBW];
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) Bv[p][nb] = brow[2 * p * W + nb * 32];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
                        const float av = p == 0 ? Ac[mb].x : (p == 1 ? Ac[mb].y : (p == 2 ? Ac[mb].z : Ac[mb].w));
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
            }
        }
        __syncthreads();
    }

    if (!wave_live) return;
    const int64_t ostride = (int64_t)a.out_mul * a.positions;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int pos = p0 + wn * NBW * 32 + nb * 32 + lo;
            if (pos >= a.positions) continue;
            const int t = a.out_mul * pos + a.out_add[ph];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int o = (mb_base + mb) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (o >= a.c_out) continue;
                const int64_t idx = (int64_t)b * a.y_bstride + (int64_t)o * ostride + t;
                float v = acc[mb][nb][r];
                if (a.bias) v += a.bias[o];
                if (a.res) v += a.res[idx];
                if (a.sum_in) v += a.sum_in[idx];
                a.y[idx] = v * a.scale;
            }
        }
    }
}

TileShape tile_shape(TileId t) {
    switch (t) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: return {wm * mbw * 32, wn * nbw * 32};
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return {0, 0};
    }
}

template <int MBW, int NBW, int WM, int WN>
static hipError_t launch_tile(const ConvArgs& a, int batch, hipStream_t stream) {
    constexpr int NWG = WN * NBW * 32;
    constexpr int MWG = WM * MBW * 32;
    const int W = NWG + (a.taps - 1) * a.dil;
    dim3 grid((a.positions + NWG - 1) / NWG, (a.c_out + MWG - 1) / MWG, batch * a.phases);
    const bool act = a.act.taps != nullptr;
    const size_t lds = sizeof(float) * (size_t)conv_lds_floats(W, act);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    if (act && a.bf16) {
        auto k = conv_kernel<MBW, NBW, WM, WN, true, true>;
        if (lds > 64 * 1024) hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k, grid, dim3(512), lds, stream, a);
    } else if (act) {
        auto k = conv_kernel<MBW, NBW, WM, WN, true, false>;
        if (lds > 64 * 1024) hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k, grid, dim3(512), lds, stream, a);
    } else {
        auto k = conv_kernel<MBW, NBW, WM, WN, false, false>;
        if (lds > 64 * 1024) hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k, grid, dim3(512), lds, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, int batch, TileId tile, hipStream_t stream) {
    switch (tile) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: return launch_tile<mbw, nbw, wm, wn>(a, batch, stream);
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// activation_post + conv_post + clamp. A workgroup owns kFinalT outputs;
// the act window is [t0 - 3, t0 + kFinalT + 3).
// ---------------------------------------------------------------------------
constexpr int kFinalT = 256;

__global__ void __launch_bounds__(256) final_kernel(FinalArgs a) {
    constexpr int CI = kChunk;
    constexpr int W = kFinalT + 6;
    __shared__ float as[CI * W];
    __shared__ float xs[CI * (W + 12)];
    __shared__ float ss[CI * (2 * W + 12)];
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * kFinalT;
    const float* xb = a.x + (int64_t)b * a.x_bstride;
    const int t = t0 + threadIdx.x;
    float acc = 0.0f;
    for (int c0 = 0; c0 < a.c; c0 += CI) {
        __syncthreads();
        stage_act<CI>(as, xs, ss, xb, c0, a.c, a.l, t0 - 3, W, a.act, threadIdx.x >> 5, threadIdx.x & 31);
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

hipError_t launch_final(const FinalArgs& a, int batch, hipStream_t stream) {
    dim3 grid((a.l + kFinalT - 1) / kFinalT, batch);
    hipLaunchKernelGGL(final_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mh3a
