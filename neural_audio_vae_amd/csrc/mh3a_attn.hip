// gfx950 kernels of the encoder's attention projection and posterior mean.
//
// Method: FastVideo API docs "minimax_h3_audio_vae", module overview
// (Encoder bullet: causal multi-head attention over the latent stream with
// q/v biases and a forced zero k bias, head averaging, average pooling into
// latent_channels streams, output projection, GeGLU MLP) and the source of
// MLXMiniMaxH3AudioVAE.encode (the block on the time-major hidden state,
// then mean_proj as a 1x1 conv); diffusers docs
// "AutoencoderKLMiniMaxH3Audio" (is_causal=True; the pipeline consumes the
// posterior mean).
//
// The q/k/v projection is a pointwise conv on the conv kernel; then
//   attn_kernel:     per (item, head, 32 queries) the causal softmax
//                    attention with an online (running max / running sum)
//                    softmax over 32-key blocks, fp32 throughout; the
//                    heads' outputs are written side by side.
//   pre_tail_kernel: per (item, 64 tokens) the head sum, the output
//                    projection with the head mean and the average pooling
//                    folded into its weights, the GeGLU MLP and mean_proj.
// Both are small next to the convolution stack (~12 GFLOP of attention per
// 2 x 30 s encode against ~2 TFLOP of convs), so they run on the vector
// ALU in fp32.

#include <hip/hip_runtime.h>

#include "mh3a_internal.h"

namespace mh3a {

constexpr int kAttnT = 32;      // tokens per query block and per key block

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// LDS: Qs, Ks, Vs token-major [32][HD + 4] (the pad staggers the rows over
// the banks), Ps [32][33]. Thread t: row tq = t / 8 of the block (queries
// for the scores and the output), lane kk = t % 8 of that row: keys
// kk + 8 j for the scores, dimensions 4 kk + 32 m + i for the output. A
// tile's loads are all issued before its LDS stores (HD / 8 per thread).
template <int HD>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs a) {
    constexpr int SD = HD + 4;
    constexpr int NL = HD * kAttnT / 256;  // tile values per thread
    constexpr int NM = (HD + 31) / 32;      // output float4 groups per lane
    extern __shared__ float lds[];
    float* Qs = lds;
    float* Ks = Qs + kAttnT * SD;
    float* Vs = Ks + kAttnT * SD;
    float* Ps = Vs + kAttnT * SD;
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, tq = tid >> 3, kk = tid & 7;
    const float* base = a.qkv + (int64_t)b * a.qkv_bstride;
    const float* qg = base + (int64_t)h * HD * a.n;
    const float* kg = base + (int64_t)(a.dim + h * HD) * a.n;
    const float* vg = base + (int64_t)(2 * a.dim + h * HD) * a.n;
    const int t0 = qb * kAttnT;
    const int t = t0 + tq;

    // (d, token u0 + j) of the channel-major rows -> X[j][d]; coalesced along tokens
    auto fetch = [&](const float* g, int u0, float (&r)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + 256 * i, d = idx >> 5, u = u0 + (idx & 31);
            r[i] = u < a.n ? g[(int64_t)d * a.n + u] : 0.0f;
        }
    };
    auto put = [&](float* X, const float (&r)[NL]) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int idx = tid + 256 * i;
            X[(idx & 31) * SD + (idx >> 5)] = r[i];
        }
    };
    {
        float r[NL];
        fetch(qg, t0, r);
        put(Qs, r);
    }
    const float scale = 1.4426950408889634f * a.inv_sqrt_hd;  // scores in log2 units
    float m = -INFINITY, l = 0.0f;
    float acc[4 * NM];
#pragma unroll
    for (int i = 0; i < 4 * NM; ++i) acc[i] = 0.0f;

    for (int kb = 0; kb <= qb; ++kb) {
        float rk[NL], rv[NL];
        fetch(kg, kb * kAttnT, rk);
        fetch(vg, kb * kAttnT, rv);
        __syncthreads();  // the previous block's products are done with Ks, Vs, Ps
        put(Ks, rk);
        put(Vs, rv);
        __syncthreads();
        float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
        for (int d = 0; d < HD; d += 4) {
            const float4 q4 = *reinterpret_cast<const float4*>(&Qs[tq * SD + d]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 k4 = *reinterpret_cast<const float4*>(&Ks[(kk + 8 * j) * SD + d]);
                s[j] = fmaf(q4.x, k4.x, s[j]);
                s[j] = fmaf(q4.y, k4.y, s[j]);
                s[j] = fmaf(q4.z, k4.z, s[j]);
                s[j] = fmaf(q4.w, k4.w, s[j]);
            }
        }
        // causal mask: key u attends only for u <= t (every processed block
        // holds key kb * 32 <= t, so each row keeps a finite maximum)
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = kb * kAttnT + kk + 8 * j;
            s[j] = u <= t ? s[j] * scale : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        mx = fmaxf(mx, shfl_xor_f(mx, 1));
        mx = fmaxf(mx, shfl_xor_f(mx, 2));
        mx = fmaxf(mx, shfl_xor_f(mx, 4));
        const float mn = fmaxf(m, mx);
        const float corr = exp2f(m - mn);  // 0 on the first block (m = -inf)
        float ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p = exp2f(s[j] - mn);
            Ps[tq * 33 + kk + 8 * j] = p;
            ps += p;
        }
        ps += shfl_xor_f(ps, 1);
        ps += shfl_xor_f(ps, 2);
        ps += shfl_xor_f(ps, 4);
        l = l * corr + ps;
        m = mn;
#pragma unroll
        for (int i = 0; i < 4 * NM; ++i) acc[i] *= corr;
        __syncthreads();  // Ps complete
#pragma unroll 4
        for (int u = 0; u < kAttnT; ++u) {
            const float p = Ps[tq * 33 + u];
            const float* vr = &Vs[u * SD];
#pragma unroll
            for (int mm = 0; mm < NM; ++mm) {
                const int d = 4 * kk + 32 * mm;
                if (d < HD) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&vr[d]);
                    acc[4 * mm + 0] = fmaf(p, v4.x, acc[4 * mm + 0]);
                    acc[4 * mm + 1] = fmaf(p, v4.y, acc[4 * mm + 1]);
                    acc[4 * mm + 2] = fmaf(p, v4.z, acc[4 * mm + 2]);
                    acc[4 * mm + 3] = fmaf(p, v4.w, acc[4 * mm + 3]);
                }
            }
        }
    }
    if (t >= a.n) return;
    const float inv_l = 1.0f / l;
    float* ob = a.o + (int64_t)b * a.o_bstride + (int64_t)h * HD * a.n + t;
#pragma unroll
    for (int mm = 0; mm < NM; ++mm) {
        const int d = 4 * kk + 32 * mm;
        if (d < HD) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[(int64_t)(d + i) * a.n] = acc[4 * mm + i] * inv_l;
        }
    }
}

size_t attn_lds_bytes(int hd) { return sizeof(float) * (size_t)(3 * kAttnT * (hd + 4) + kAttnT * 33); }

template <int HD>
static hipError_t launch_attention_hd(const AttnArgs& a, int batch, hipStream_t stream) {
    const size_t lds = attn_lds_bytes(HD);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<HD>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.n + kAttnT - 1) / kAttnT, a.heads, batch);
    hipLaunchKernelGGL(attn_kernel<HD>, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

bool attn_head_width_ok(int hd) { return hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256; }

hipError_t launch_attention(const AttnArgs& a, int batch, hipStream_t stream) {
    if (!attn_head_width_ok(a.hd) || a.heads < 1 || a.dim != a.heads * a.hd || a.n < 1 || batch < 1 ||
        batch > 65535 || a.heads > 65535)
        return hipErrorInvalidValue;
    switch (a.hd) {
        case 8: return launch_attention_hd<8>(a, batch, stream);
        case 16: return launch_attention_hd<16>(a, batch, stream);
        case 32: return launch_attention_hd<32>(a, batch, stream);
        case 64: return launch_attention_hd<64>(a, batch, stream);
        case 128: return launch_attention_hd<128>(a, batch, stream);
        default: return launch_attention_hd<256>(a, batch, stream);
    }
}

// ---------------------------------------------------------------------------
// Head sum -> output projection (head mean and pooling folded into wf) ->
// GeGLU MLP -> mean_proj, per token. A workgroup owns 64 tokens of one item;
// every intermediate is kept in LDS channel-major ([feature][token]), and
// one wave's 64 lanes are the 64 tokens of one feature, so weight reads are
// uniform across the wave.
// ---------------------------------------------------------------------------
constexpr int kTailT = 64;

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

__global__ void __launch_bounds__(256) pre_tail_kernel(PreTailArgs a) {
    extern __shared__ float lds[];
    float* A = lds;                  // [hd][64] head sum
    float* Y = A + a.hd * kTailT;    // [c][64]  projection
    float* G = Y + a.c * kTailT;     // [f][64]  value * GELU(gate)
    float* Y2 = G + a.f * kTailT;    // [c][64]  MLP output
    const int b = blockIdx.y, t0 = blockIdx.x * kTailT, tid = threadIdx.x;
    const float* ob = a.o + (int64_t)b * a.o_bstride;
    for (int idx = tid; idx < a.hd * kTailT; idx += 256) {
        const int j = idx / kTailT, u = t0 + idx % kTailT;
        float s = 0.0f;
        if (u < a.n)
            for (int h = 0; h < a.heads; ++h) s += ob[(int64_t)(h * a.hd + j) * a.n + u];
        A[idx] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < a.c * kTailT; idx += 256) {
        const int o = idx / kTailT, t = idx % kTailT;
        const float* w = a.wf + (int64_t)o * a.hd;
        float s = a.bf[o];
        for (int j = 0; j < a.hd; ++j) s = fmaf(w[j], A[j * kTailT + t], s);
        Y[idx] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < a.f * kTailT; idx += 256) {
        const int o = idx / kTailT, t = idx % kTailT;
        const float* wv = a.w1 + (int64_t)o * a.c;
        const float* wg = a.w1 + (int64_t)(a.f + o) * a.c;
        float v = a.b1[o], g = a.b1[a.f + o];
        for (int j = 0; j < a.c; ++j) {
            const float y = Y[j * kTailT + t];
            v = fmaf(wv[j], y, v);
            g = fmaf(wg[j], y, g);
        }
        G[idx] = v * gelu_erf(g);
    }
    __syncthreads();
    for (int idx = tid; idx < a.c * kTailT; idx += 256) {
        const int o = idx / kTailT, t = idx % kTailT;
        const float* w = a.w2 + (int64_t)o * a.f;
        float s = a.b2[o];
        for (int j = 0; j < a.f; ++j) s = fmaf(w[j], G[j * kTailT + t], s);
        Y2[idx] = s;
    }
    __syncthreads();
    float* yb = a.y + (int64_t)b * a.y_bstride;
    for (int idx = tid; idx < a.lc * kTailT; idx += 256) {
        const int o = idx / kTailT, t = idx % kTailT, u = t0 + t;
        if (u >= a.n) continue;
        const float* w = a.wm + (int64_t)o * a.c;
        float s = a.bm[o];
        for (int j = 0; j < a.c; ++j) s = fmaf(w[j], Y2[j * kTailT + t], s);
        yb[(int64_t)o * a.n + u] = s;
    }
}

size_t pre_tail_lds_bytes(int hd, int c, int f) { return sizeof(float) * (size_t)kTailT * (hd + 2 * c + f); }

hipError_t launch_pre_tail(const PreTailArgs& a, int batch, hipStream_t stream) {
    if (a.n < 1 || a.hd < 1 || a.c < 1 || a.f < 1 || a.lc < 1 || a.heads < 1 || batch < 1 || batch > 65535)
        return hipErrorInvalidValue;
    const size_t lds = pre_tail_lds_bytes(a.hd, a.c, a.f);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)pre_tail_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.n + kTailT - 1) / kTailT, batch);
    hipLaunchKernelGGL(pre_tail_kernel, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

}  // namespace mh3a
