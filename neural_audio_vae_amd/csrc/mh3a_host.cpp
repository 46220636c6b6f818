// Host side of the mh3a C ABI: argument validation, parameter lookup,
// weight-norm folding, Kaiser-sinc filter design, weight packing for the
// matrix-core kernels, workspace layout and the decode launch sequence.
//
// The decode order follows FastVideo API docs "minimax_h3_audio_vae",
// MLXMiniMaxH3AudioVAE.decode; the interface contract follows diffusers docs
// "AutoencoderKLMiniMaxH3Audio", section "decode".

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "mh3a.h"
#include "mh3a_internal.h"

using namespace mh3a;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return MH3A_OK;
}

// ---------------------------------------------------------------------------
// Kaiser-windowed sinc low-pass of the anti-aliased activation (FastVideo
// "minimax_h3_audio_vae", the Activation1d samplers' filter design). Kaiser's
// design rules (J. F. Kaiser, 1974): a window of N taps and transition width
// dw (fraction of Nyquist) reaches A = 7.95 + 2.285 (N - 1) pi dw dB, and A dB
// asks for beta = 0 below 21 dB, 0.5842 (A - 21)^0.4 + 0.07886 (A - 21) up
// to 50 dB, 0.1102 (A - 8.7) above. The released filter evaluates them at
// N = K / 2 and dw = 4 * half_width. Window I0(beta sqrt(1 - r^2)) / I0(beta);
// taps 2 fc w[n] sinc(2 fc t_n) on a half-integer grid for even K, normalized
// to unit sum. Evaluated in double.
// ---------------------------------------------------------------------------
double bessel_i0(double x) {
    const double q = 0.25 * x * x;
    double term = 1.0, sum = 1.0;
    for (int m = 1; m < 500; ++m) {
        term *= q / ((double)m * m);
        sum += term;
        if (term < 1e-17 * sum) break;
    }
    return sum;
}

static double kaiser_attenuation(int taps, double width) { return 7.95 + 2.285 * (taps - 1) * M_PI * width; }

static double kaiser_beta_for(double a) {
    if (a < 21.0) return 0.0;
    if (a <= 50.0) return 0.5842 * std::pow(a - 21.0, 0.4) + 0.07886 * (a - 21.0);
    return 0.1102 * (a - 8.7);
}

void design_lowpass(double cutoff, double half_width, int k, float* out) {
    const int half = k / 2;
    const double beta = kaiser_beta_for(kaiser_attenuation(half, 4.0 * half_width));
    std::vector<double> f(k);
    double sum = 0.0;
    const double i0b = bessel_i0(beta);
    for (int n = 0; n < k; ++n) {
        const double r = (k > 1) ? 2.0 * n / (k - 1) - 1.0 : 0.0;
        const double w = bessel_i0(beta * std::sqrt(std::fmax(0.0, 1.0 - r * r))) / i0b;
        const double t = (k % 2 == 0) ? (n - half + 0.5) : (double)(n - half);
        const double x = 2.0 * cutoff * t;
        const double sinc = (x == 0.0) ? 1.0 : std::sin(M_PI * x) / (M_PI * x);
        f[n] = 2.0 * cutoff * w * sinc;
        sum += f[n];
    }
    for (int n = 0; n < k; ++n) out[n] = (float)(f[n] / sum);
}

// ---------------------------------------------------------------------------
// Parameter table
// ---------------------------------------------------------------------------
struct Param {
    const float* data;
    int ndim;
    int64_t shape[3];
    int64_t numel() const {
        int64_t n = 1;
        for (int i = 0; i < ndim; ++i) n *= shape[i];
        return n;
    }
};

struct Table {
    std::map<std::string, Param> m;
    const Param* get(const std::string& name) const {
        auto it = m.find(name);
        return it == m.end() ? nullptr : &it->second;
    }
};

// Shape check ignoring leading/trailing singleton differences of 1-D
// vectors: a (C,) and a (C, 1, 1) view are both accepted for vectors.
bool shape_is(const Param* p, int64_t a, int64_t b = -1, int64_t c = -1) {
    int64_t want[3] = {a, b, c};
    int wn = c >= 0 ? 3 : (b >= 0 ? 2 : 1);
    if (p->ndim == wn) {
        for (int i = 0; i < wn; ++i)
            if (p->shape[i] != want[i]) return false;
        return true;
    }
    return false;
}

bool vector_of(const Param* p, int64_t n) {
    if (p->numel() != n) return false;
    int non1 = 0;
    for (int i = 0; i < p->ndim; ++i)
        if (p->shape[i] != 1) ++non1;
    return non1 <= 1;
}

// ---------------------------------------------------------------------------
// Decoder object
// ---------------------------------------------------------------------------
struct ConvLayer {
    int c_in = 0, c_out = 0, taps = 1, dil = 1, phases = 1, out_mul = 1;
    int in_off[kMaxPhases] = {0};
    int out_add[kMaxPhases] = {0};
    int64_t w_off = -1;
    int64_t w16_off = -1;  // 16-row MFMA packing (AMP convs of <= 32 channels), or -1
    int64_t w6_off = -1;   // bf16 pieces for split products, or -1
    int64_t w6u_off = -1;  // bf16 pieces for the split-product unit kernel (<= 32 channels), or -1
    int64_t w6_phase_stride = 0;
    int64_t wh_off = -1;   // fp16 pieces of the weights scaled by wh_scale (kPiecesH form), or -1
    int64_t whu_off = -1;  // the same in the unit kernel's order (<= 32 channels), or -1
    int64_t wh_phase_stride = 0;
    float wh_scale = 1.0f; // 2^e
    int64_t w_phase_stride = 0;
    int64_t b_off = -1;
    int64_t wv_off = -1;   // transposed convs run on the vector ALU: the folded weight [c_in][c_out][k], or -1
    int act = -1;       // index into acts, -1 = none
    int alg_taps = 1;   // taps per input sample the layer's definition uses
    int kind = 0;       // timing class
};

enum Kind {
    KIND_IN_PROJ = 0,
    KIND_CONV_PRE,
    KIND_UPSAMPLE,
    KIND_AMP,
    KIND_AMP_ACT,
    KIND_FINAL,
    KIND_AMP_UNIT,
    KIND_SPLIT,
    KIND_ENC_UNIT_CONV,  // encoder: the residual units' dilated k7 convs
    KIND_ENC_CONV,       // encoder: pointwise, strided, first and last convs
    KIND_ENC_SNAKE,      // encoder: Snake (and space-to-depth) passes
    KIND_ENC_ATTN,       // encoder: causal attention of the attention projection
    KIND_ENC_TAIL,       // encoder: head sum, projection, GeGLU MLP, mean_proj
    KIND_COUNT
};
const char* const kKindNames[KIND_COUNT] = {"dec_in_proj", "conv_pre",   "ups_transposed_conv", "amp_conv",
                                            "amp_act",     "act_post_conv_post", "amp_unit", "input_split",
                                            "enc_unit_conv", "enc_conv", "enc_snake", "enc_attention",
                                            "enc_proj_mlp_mean"};
static_assert(KIND_COUNT <= MH3A_MAX_KERNEL_KINDS, "timing classes fit mh3a_timing_read's table");

struct TimingRec {
    int kind;
    double flops, bytes;
    int ev;  // index of the start event; ev + 1 is the stop event
};

struct Timing {
    bool on = false;
    bool amp_only = false;  // only the AMP conv launches
    std::vector<hipEvent_t> evs;
    int used = 0;
    std::vector<TimingRec> recs;
};

struct ActLayer {
    int64_t taps_off = -1;
    int64_t ab_off = -1;
};

}  // namespace

// Launch shape of one conv: (layer, positions, batch, bf16 operands | batch-invariant plan << 1).
using PlanKey = std::tuple<const void*, int, int, int>;

// What the launch helpers need of a decoder or an encoder: the device, the
// parameter blob, activation constants, timing state and the plan cache.
struct mh3a_net {
    int device = 0;
    float* blob = nullptr;
    int64_t blob_floats = 0;
    std::vector<ActLayer> acts;
    int num_cus = 256;          // compute units of `device`
    mutable Timing timing;
    mutable std::mutex plan_mu;                          // guards plans
    mutable std::map<PlanKey, std::pair<int, int>> plans;  // (tile, ksplit) per launch shape
};

struct mh3a_decoder : mh3a_net {
    mh3a_config cfg;
    ConvLayer in_proj, in_proj_dn, conv_pre;
    std::vector<ConvLayer> ups;                 // [num_ups]
    std::vector<std::vector<ConvLayer>> amp;    // [stage][(block * ndil + d) * 2 + {0,1}]
    int post_act = -1;
    int64_t post_w_off = -1;
    float post_bias = 0.0f;
    std::vector<int> stage_c;   // output channels per stage
    bool pk_ok = false;         // every AMP conv can read a packed activated input
    bool bx6_ok = false;        // ... and has split-product weights (see kPieces)
    bool h16_ok = false;        // ... and fp16 weight pieces (see kPiecesH)
    // Concurrent AMP blocks of small decodes (see fork_ways): one side stream
    // per residual block but the last, the event that releases them at a
    // stage's start and one per side block marking its last conv; created
    // at create time (default priority), used under fork_mu.
    std::vector<hipStream_t> side;
    hipEvent_t fork_ev = nullptr;
    std::vector<hipEvent_t> done_ev;
    std::mutex fork_mu;
};

namespace {

struct Blob {
    std::vector<float> h;
    int64_t add(const float* src, int64_t n) {
        int64_t off = (int64_t)h.size();
        h.resize(off + ((n + 63) / 64) * 64, 0.0f);
        if (src) std::memcpy(h.data() + off, src, sizeof(float) * n);
        return off;
    }
    int64_t reserve(int64_t n) { return add(nullptr, n); }
};

int check_config(const mh3a_config* c) {
    if (c->latent_channels < 1 || c->latent_dim < 1 || c->decoder_dim < 1)
        return fail(MH3A_E_CONFIG, "channel counts must be positive");
    if (c->num_ups < 1 || c->num_ups > MH3A_MAX_STAGES)
        return fail(MH3A_E_CONFIG, "num_ups must be in [1, %d]", MH3A_MAX_STAGES);
    long long prod = 1;
    for (int s = 0; s < c->num_ups; ++s) {
        if (c->rates[s] < 1 || c->rates[s] > kMaxPhases)
            return fail(MH3A_E_CONFIG, "rate %d of stage %d out of range [1, %d]", c->rates[s], s, kMaxPhases);
        if (c->kernels[s] < c->rates[s])
            return fail(MH3A_E_CONFIG, "stage %d: kernel %d smaller than rate %d", s, c->kernels[s], c->rates[s]);
        prod *= c->rates[s];
    }
    if (prod != c->hop_length)
        return fail(MH3A_E_CONFIG, "product of decoder rates (%lld) must equal hop_length (%d)", prod, c->hop_length);
    if ((c->decoder_dim >> c->num_ups) < 1 || (c->decoder_dim % (1 << c->num_ups)) != 0)
        return fail(MH3A_E_CONFIG, "decoder_dim %d cannot be halved %d times", c->decoder_dim, c->num_ups);
    if (c->num_resblocks < 1) return fail(MH3A_E_CONFIG, "decoder has no residual blocks");
    if (c->num_resblocks > MH3A_MAX_RESBLOCKS) return fail(MH3A_E_CONFIG, "too many residual blocks");
    if (c->num_dilations < 1 || c->num_dilations > MH3A_MAX_DILATIONS)
        return fail(MH3A_E_CONFIG, "num_dilations must be in [1, %d]", MH3A_MAX_DILATIONS);
    for (int j = 0; j < c->num_resblocks; ++j) {
        if (c->rb_kernels[j] < 1 || c->rb_kernels[j] % 2 == 0 || c->rb_kernels[j] > 15)
            return fail(MH3A_E_CONFIG, "residual-block kernel %d must be odd and <= 15", c->rb_kernels[j]);
        for (int d = 0; d < c->num_dilations; ++d)
            if (c->rb_dilations[j][d] < 1 || c->rb_dilations[j][d] > 16)
                return fail(MH3A_E_CONFIG, "dilation %d out of range [1, 16]", c->rb_dilations[j][d]);
    }
    if (c->filter_taps != kTaps) return fail(MH3A_E_CONFIG, "only %d-tap resampling filters are supported", kTaps);
    if (!(c->filter_cutoff > 0.0 && c->filter_cutoff < 0.5 && c->filter_half_width > 0.0))
        return fail(MH3A_E_CONFIG, "bad filter cutoff / half width");
    if (c->matrix_form != MH3A_MATRIX_SPLIT && c->matrix_form != MH3A_MATRIX_FP32 &&
        c->matrix_form != MH3A_MATRIX_SPLIT_F16)
        return fail(MH3A_E_CONFIG, "unknown matrix_form %d", c->matrix_form);
    return MH3A_OK;
}

// Fold weight norm: w = g v / ||v|| per axis-0 slice of v (n0 slices of
// `inner` elements). Accepts an already folded "<prefix>.weight" instead.
int fetch_weight(const Table& t, const std::string& prefix, int64_t d0, int64_t d1, int64_t d2,
                 std::vector<float>& w) {
    const Param* wt = t.get(prefix + ".weight");
    const Param* v = t.get(prefix + ".weight_v");
    const Param* g = t.get(prefix + ".weight_g");
    w.assign((size_t)(d0 * d1 * d2), 0.0f);
    if (v) {
        if (!g) return fail(MH3A_E_MISSING_TENSOR, "missing %s.weight_g", prefix.c_str());
        if (!shape_is(v, d0, d1, d2))
            return fail(MH3A_E_SHAPE, "%s.weight_v must be (%lld, %lld, %lld)", prefix.c_str(), (long long)d0,
                        (long long)d1, (long long)d2);
        if (!vector_of(g, d0)) return fail(MH3A_E_SHAPE, "%s.weight_g must hold %lld values", prefix.c_str(), (long long)d0);
        const int64_t inner = d1 * d2;
        for (int64_t o = 0; o < d0; ++o) {
            double ss = 0.0;
            for (int64_t i = 0; i < inner; ++i) {
                const double x = v->data[o * inner + i];
                ss += x * x;
            }
            const double s = (double)g->data[o] / std::sqrt(ss);
            for (int64_t i = 0; i < inner; ++i) w[o * inner + i] = (float)(s * (double)v->data[o * inner + i]);
        }
        return MH3A_OK;
    }
    if (wt) {
        if (!shape_is(wt, d0, d1, d2))
            return fail(MH3A_E_SHAPE, "%s.weight must be (%lld, %lld, %lld)", prefix.c_str(), (long long)d0,
                        (long long)d1, (long long)d2);
        std::memcpy(w.data(), wt->data, sizeof(float) * w.size());
        return MH3A_OK;
    }
    return fail(MH3A_E_MISSING_TENSOR, "missing %s.weight_v (or %s.weight)", prefix.c_str(), prefix.c_str());
}

int fetch_vector(const Table& t, const std::string& name, int64_t n, const float** out) {
    const Param* p = t.get(name);
    if (!p) return fail(MH3A_E_MISSING_TENSOR, "missing %s", name.c_str());
    if (!vector_of(p, n)) return fail(MH3A_E_SHAPE, "%s must hold %lld values", name.c_str(), (long long)n);
    *out = p->data;
    return MH3A_OK;
}

// Upload a conv layer (c_out, c_in, taps) with its bias.
void add_conv(Blob& blob, ConvLayer& L, const std::vector<float>& w, const float* bias, int c_out, int c_in,
              int taps) {
    L.c_in = c_in;
    L.c_out = c_out;
    L.taps = taps;
    const int64_t n = packed_weight_floats(c_out, c_in, taps);
    L.w_off = blob.reserve(n);
    pack_conv_weights(w.data(), c_out, c_in, taps, blob.h.data() + L.w_off);
    if (bias) {
        L.b_off = blob.add(bias, c_out);
    } else {
        L.b_off = blob.reserve(c_out);  // zeros: the kernels always add a bias
    }
}

// A conv (all phases) can read its input in the packed split-product form:
// a compile-time tap count the kernel has instances for, whole two-chunk
// items, and windows (output tiles up to 256 positions plus the dilated
// span) inside the packed row's pads.
bool split_input_ok(const ConvLayer& L) {
    if (!(L.taps == 2 || L.taps == 3 || L.taps == 7 || L.taps == 11)) return false;
    if (L.c_in % 16 || L.c_out < 32 || L.dil < 1 || L.dil > kBx6MaxDil) return false;
    if ((L.c_in / kChunk) % bx6_cpi_max(L.taps)) return false;  // whole pipeline items
    for (int ph = 0; ph < L.phases; ++ph)
        if (-L.in_off[ph] > kPkPadL || 255 + (L.taps - 1) * L.dil + L.in_off[ph] > kPkPadR) return false;
    return true;
}

int add_act(Blob& blob, const Table& t, const std::string& prefix, int c, const float* designed,
            std::vector<ActLayer>& acts) {
    const float *alpha, *beta;
    int rc;
    if ((rc = fetch_vector(t, prefix + ".act.alpha", c, &alpha))) return rc;
    if ((rc = fetch_vector(t, prefix + ".act.beta", c, &beta))) return rc;
    const float* up = designed;
    const float* dn = designed;
    if (const Param* p = t.get(prefix + ".upsample.filter")) {
        if (!vector_of(p, kTaps)) return fail(MH3A_E_SHAPE, "%s.upsample.filter must hold %d taps", prefix.c_str(), kTaps);
        up = p->data;
    }
    if (const Param* p = t.get(prefix + ".downsample.lowpass.filter")) {
        if (!vector_of(p, kTaps))
            return fail(MH3A_E_SHAPE, "%s.downsample.lowpass.filter must hold %d taps", prefix.c_str(), kTaps);
        dn = p->data;
    }
    float taps[24];
    for (int e = 0; e < 6; ++e) {
        taps[e] = 2.0f * up[1 + 2 * e];  // even outputs: gain 2
        taps[6 + e] = 2.0f * up[2 * e];  // odd outputs
    }
    for (int q = 0; q < 12; ++q) taps[12 + q] = dn[q];
    std::vector<float> ab(2 * (size_t)c);
    for (int i = 0; i < c; ++i) {
        if (!(beta[i] != 0.0f)) return fail(MH3A_E_SHAPE, "%s.act.beta[%d] is zero", prefix.c_str(), i);
        ab[2 * i] = (float)((double)alpha[i] / M_PI);
        ab[2 * i + 1] = (float)(0.5 / (double)beta[i]);
    }
    ActLayer a;
    a.taps_off = blob.add(taps, 24);
    a.ab_off = blob.add(ab.data(), 2 * c);
    acts.push_back(a);
    return MH3A_OK;
}

ActParams act_params(const mh3a_net* d, int idx) {
    ActParams p{nullptr, nullptr};
    if (idx >= 0) {
        p.taps = d->blob + d->acts[idx].taps_off;
        p.ab = reinterpret_cast<const float2*>(d->blob + d->acts[idx].ab_off);
    }
    return p;
}

// fused: the layer's activation runs in the conv's operand staging (else the
// conv reads an already activated input)
ConvShape shape_of(const ConvLayer& L, bool fused, bool bx6 = false) {
    return {L.c_in, L.c_out, L.taps, L.dil, L.phases, fused && L.act >= 0, L.kind == KIND_AMP,
            L.w16_off >= 0 && L.c_out <= 16, bx6};
}

int64_t plan_partial_floats(const ConvLayer& L, int positions, int groups, const ConvPlan& p, bool fused) {
    return mh3a::plan_partial_floats(shape_of(L, fused), positions, groups, p);
}

// Whether packed AMP inputs take a split-product form (every matrix form but
// fp32, when every AMP conv has the weights for it): bf16 pieces with six
// products (kPieces), or, in the default form, fp16 pieces with three
// (kPiecesH; use_h16).
bool use_bx6(const mh3a_decoder* d) { return d->bx6_ok && d->cfg.matrix_form != MH3A_MATRIX_FP32; }
bool use_h16(const mh3a_decoder* d) { return use_bx6(d) && d->h16_ok && d->cfg.matrix_form == MH3A_MATRIX_SPLIT_F16; }

// Whether an AMP conv of a (batch, C, L) activation fuses its activation.
// Fused, the producer waves compute it per tile on the SIMDs whose matrix
// cores the consumer waves keep busy, and their vector work barely advances
// while the MFMAs stream (measured: ~3.5x slower than alone), so the tile
// waits on it; at 256+ channels it is also repeated per M tile. Separate,
// a standalone pass writes the packed input and the conv's producers only
// copy it to LDS. Measured per stage (B=2 x 1200 latents): separate wins at
// 128 to 512 channels, ties at 64 and loses below, where the pass (~30 us
// per 15 M samples) costs more than the contention saves. Small launches
// stay fused (one launch, less latency).
bool amp_act_fused(const mh3a_decoder* d, int64_t batch, int64_t c, int64_t len) {
    if (!d->pk_ok) return true;
    // split-product convs gain enough from matrix-core speed to pay for the
    // separate pass from 64 channels on
    return c < (use_bx6(d) ? 64 : 128) || batch * c * len < kSeparateActMin;
}

// Whether the AMP convs of a (batch, C, L) stage read the packed input in the
// split-product form.
// (with the bf16 operand flag the convs take the three-product variant)
bool stage_px(const mh3a_decoder* d, int64_t batch, int c, int64_t len, bool bf16) {
    (void)bf16;
    return !amp_act_fused(d, batch, c, len) && use_bx6(d) && c % 64 == 0;  // whole items of up to 8 chunks
}

// Whether conv_pre / a transposed conv reads its input in the split-product
// form (a split pass, then the packed path): layers packed for it at create.
bool pre_bx6(const mh3a_decoder* d, const ConvLayer& L) { return use_bx6(d) && L.w6_off >= 0; }
// ... and in the fp16 form
bool pre_h16(const mh3a_decoder* d, const ConvLayer& L) { return pre_bx6(d, L) && use_h16(d) && L.wh_off >= 0; }

// Plans are cached per launch shape.
// `ways`: launches of the same kind that run at once (the concurrent
// residual blocks), see mh3a::plan_conv.
ConvPlan plan_conv(const mh3a_net* d, const ConvLayer& L, int positions, int batch, bool bf16, bool invariant,
                   bool fused, bool bx6 = false, int ways = 1) {
    const PlanKey key{&L, positions, batch,
                      (bf16 ? 1 : 0) | (invariant ? 2 : 0) | (fused ? 4 : 0) | (bx6 ? 8 : 0) | (ways << 4)};
    std::lock_guard<std::mutex> lock(d->plan_mu);
    auto it = d->plans.find(key);
    if (it != d->plans.end()) return {(TileId)it->second.first, it->second.second};
    const ConvPlan p = mh3a::plan_conv(shape_of(L, fused, bx6), positions, batch, bf16, invariant, d->num_cus, ways);
#ifdef MH3A_PLAN_LOG
    // (build-time option: -DMH3A_PLAN_LOG prints each new plan to stderr)
    {
        const TileShape ts = tile_shape(p.tile);
        std::fprintf(stderr, "mh3a plan: %s c_in %d c_out %d taps %d dil %d positions %d batch %d%s%s -> tile %dx%d ksplit %d\n",
                     kKindNames[L.kind], L.c_in, L.c_out, L.taps, L.dil, positions, batch, invariant ? " (invariant)" : "",
                     (L.act >= 0 && !fused) ? " (act separate)" : "", ts.m, ts.n, p.ksplit);
    }
#endif
    if (d->plans.size() > 4096) d->plans.clear();
    d->plans.emplace(key, std::make_pair((int)p.tile, p.ksplit));
    return p;
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
struct Buf {
    float* p;
    int64_t bstride;
};

// Brackets a launch with timing events when timing is enabled.
struct TimedLaunch {
    const mh3a_net* d;
    hipStream_t st;
    int ev = -1;
    TimedLaunch(const mh3a_net* d_, hipStream_t st_, int kind) : d(d_), st(st_) {
        Timing& t = d->timing;
        if (!t.on || (t.amp_only && kind != KIND_AMP && kind != KIND_ENC_UNIT_CONV)) return;
        while ((int)t.evs.size() < t.used + 2) {
            hipEvent_t e;
            // timing-only events: no system-scope fence (no cache writeback between launches)
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
            t.evs.push_back(e);
        }
        ev = t.used;
        t.used += 2;
        hipEventRecord(t.evs[ev], st);
    }
    void done(int kind, double flops, double bytes) {
        if (ev < 0) return;
        Timing& t = d->timing;
        hipEventRecord(t.evs[ev + 1], st);
        t.recs.push_back({kind, flops, bytes, ev});
    }
};

// `partial` holds at least the plan's partial sums (plan_partial_floats).
hipError_t run_conv(const mh3a_net* d, const ConvLayer& L, const float* x, int64_t x_bstride, int l_in,
                    int positions, float* y, int64_t y_bstride, int batch, const float* res, const float* sum_in,
                    float scale, bool bf16, bool invariant, bool fused, float* partial, hipStream_t st,
                    int pk_lp = 0, bool bx6 = false, bool h16 = false, int ways = 1) {
    ConvArgs a;
    std::memset(&a, 0, sizeof a);
    a.pk_lp = pk_lp;
    a.bx6 = bx6 ? 1 : 0;
    a.w6 = L.w6_off >= 0 ? d->blob + L.w6_off : nullptr;
    a.w6_phase_stride = L.w6_phase_stride;
    a.wscale = 1.0f;
    a.out_scale = 1.0f;
    if (h16) {
        if (!bx6 || L.wh_off < 0) return hipErrorInvalidValue;
        a.h16 = 1;
        a.w6 = d->blob + L.wh_off;
        a.w6_phase_stride = L.wh_phase_stride;
        a.wscale = L.wh_scale;
        a.out_scale = 1.0f / L.wh_scale;  // exact: a power of two
    }
    a.x = x;
    a.x_bstride = x_bstride;
    a.c_in = L.c_in;
    a.l_in = l_in;
    a.w = d->blob + L.w_off;
    a.w16 = L.w16_off >= 0 ? d->blob + L.w16_off : nullptr;
    a.w_phase_stride = L.w_phase_stride;
    a.bias = L.b_off >= 0 ? d->blob + L.b_off : nullptr;
    a.y = y;
    a.y_bstride = y_bstride;
    a.c_out = L.c_out;
    a.positions = positions;
    a.taps = L.taps;
    a.dil = L.dil;
    a.out_mul = L.out_mul;
    a.phases = L.phases;
    a.groups = batch * L.phases;
    for (int i = 0; i < kMaxPhases; ++i) {
        a.in_off[i] = L.in_off[i];
        a.out_add[i] = L.out_add[i];
    }
    a.res = res;
    a.sum_in = sum_in;
    a.scale = scale;
    a.act = fused ? act_params(d, L.act) : ActParams{nullptr, nullptr};
    a.bf16 = bf16 ? 1 : 0;
    const ConvPlan plan = plan_conv(d, L, positions, batch, bf16, invariant, fused, bx6, ways);
    a.ksplit = plan.ksplit;
    a.partial = partial;
    if (plan.ksplit > 1 && !partial) return hipErrorInvalidValue;
    TimedLaunch tl(d, st, L.kind);
    hipError_t e = launch_conv(a, plan.tile, st);
    const double outs = (double)batch * L.c_out * L.out_mul * positions;
    const double flops = 2.0 * L.c_out * (double)L.c_in * L.alg_taps * positions * batch;
    const double bytes = 4.0 * ((double)batch * L.c_in * l_in + outs * (1 + (res ? 1 : 0) + (sum_in ? 1 : 0)) +
                                (double)L.c_out * L.c_in * L.alg_taps + L.c_out);
    tl.done(L.kind, flops, bytes);
    return e;
}

#define HIP_TRY(expr)                                                                              \
    do {                                                                                           \
        hipError_t e_ = (expr);                                                                    \
        if (e_ != hipSuccess) return fail(MH3A_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

int64_t max_cl(const mh3a_decoder* d, int64_t frames) {
    const mh3a_config& c = d->cfg;
    int64_t m = std::max<int64_t>((int64_t)c.latent_dim * frames, (int64_t)c.decoder_dim * frames);
    int64_t len = frames;
    for (int s = 0; s < c.num_ups; ++s) {
        len *= c.rates[s];
        m = std::max<int64_t>(m, (int64_t)d->stage_c[s] * len);
    }
    return m;
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Packed activated input of one (C, L) item (see kPkPadL): row length and
// floats per item.
int64_t pk_lp(int64_t len) { return len + kPkPadL + kPkPadR; }

// Floats per item of a packed input: per chunk of 8 channels, two fp32
// planes or kPieces bf16 planes of lp 16-byte groups.
int64_t pk_item_floats(const mh3a_decoder* d, int c, int64_t len) {
    const int planes = use_bx6(d) ? kPieces : 2;
    return (int64_t)((c + kChunk - 1) / kChunk) * planes * 4 * pk_lp(len);
}

// The standalone activation of AMP layer `act_idx`: y = act(x), x (B, C, L)
// rows, y packed.
hipError_t run_act(const mh3a_decoder* d, int act_idx, const float* x, float* y, int batch, int c, int64_t len,
                   int pieces, hipStream_t st) {
    ActArgs a;
    a.x = x;
    a.x_bstride = (int64_t)c * len;
    a.y = y;
    a.y_bstride = pk_item_floats(d, c, len);
    a.c = c;
    a.l = (int)len;
    a.lp = (int)pk_lp(len);
    a.pieces = pieces;
    a.act = act_params(d, act_idx);
    TimedLaunch tl(d, st, KIND_AMP_ACT);
    hipError_t e = launch_act(a, batch, st);
    const double n = (double)batch * c * len;
    // 12 up + 12 down multiply-adds and the SnakeBeta per sample; in and out
    tl.done(KIND_AMP_ACT, 48.0 * n, 8.0 * n);
    return e;
}

// A narrow stage's transposed conv on the vector ALU: x (B, c_in, len) ->
// y (B, c_out, r len).
hipError_t run_ups_vec(const mh3a_decoder* d, const ConvLayer& U, const float* x, float* y, int batch, int len,
                       int k, hipStream_t st) {
    UpsVecArgs a;
    a.x = x;
    a.y = y;
    a.w = d->blob + U.wv_off;
    a.bias = d->blob + U.b_off;
    a.ci = U.c_in;
    a.co = U.c_out;
    a.r = U.phases;
    a.k = k;
    a.l = len;
    TimedLaunch tl(d, st, KIND_UPSAMPLE);
    hipError_t e = launch_ups_vec(a, batch, st);
    const double flops = 2.0 * U.c_out * (double)U.c_in * k * len * batch;
    const double bytes = 4.0 * ((double)batch * U.c_in * len + (double)batch * U.c_out * U.phases * len +
                                (double)U.c_in * U.c_out * k + U.c_out);
    tl.done(KIND_UPSAMPLE, flops, bytes);
    return e;
}

// The split pass of a conv input: x (B, c, len) rows -> y in the packed
// split-product form.
hipError_t run_split(const mh3a_decoder* d, const float* x, float* y, int batch, int c, int64_t len, int pieces,
                     hipStream_t st) {
    ActArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.x_bstride = (int64_t)c * len;
    a.y = y;
    a.y_bstride = pk_item_floats(d, c, len);
    a.c = c;
    a.l = (int)len;
    a.lp = (int)pk_lp(len);
    a.pieces = pieces;
    TimedLaunch tl(d, st, KIND_SPLIT);
    hipError_t e = launch_split(a, batch, st);
    const double n = (double)batch * c * len;
    tl.done(KIND_SPLIT, 0.0, (4.0 + 2.0 * pieces) * n);  // 4 bytes in, 2 per piece out
    return e;
}

// AMP set of one stage: h (B, C, L) read-only; x_buf, t_buf, a_buf scratch;
// result in s_buf. Blocks run from the same h and are averaged in the
// epilogue of each block's last conv. Each conv's activation is fused into
// its operand staging, or (large tensors) runs as its own pass into a_buf.
// Whether stage s's unit kernels can use split products (every layer has the weights)
bool amp_unit_split(const mh3a_decoder* d, int stage) {
    if (!use_bx6(d)) return false;
    for (const ConvLayer& L : d->amp[stage])
        if (L.w6u_off < 0) return false;
    return true;
}

// Whether stage s runs each residual unit as one launch (unit_kernel): fp32
// operands, a channel count and every conv's taps and dilation that the
// kernel has instances for.
bool amp_unit_path(const mh3a_decoder* d, int stage, bool bf16) {
    for (const ConvLayer& L : d->amp[stage])
        if (L.w16_off < 0 || L.b_off < 0 || L.act < 0 || !unit_supported(L.c_out, L.taps, L.dil)) return false;
    // the bf16 operand flag needs the split-product unit kernel (three products)
    return !bf16 || amp_unit_split(d, stage);
}


// The residual units of one AMP stage as unit_kernel launches. Unit n of a
// block reads the block input h (n = 0) or the previous unit's output, and
// writes x_buf / t_buf alternately (a unit reads its input around its own
// outputs, so it cannot update in place); the block's last unit adds into
// the running sum s_buf, scaled by 1 / blocks at the last block.
// Scratch and stream of one residual block of an AMP set. With `fork` the
// blocks run concurrently: block j < nrb - 1 on side stream j with scratch of
// its own, the last block on the caller's stream; the stage's start releases
// the side streams, and block j's last conv (the one that adds the running
// sum in s_buf) waits for block j - 1's, so the sum accumulates in the
// sequential order and the results are the same bits.
struct BlockBufs {
    float* x;
    float* t;
    float* a;
    float* partial;
    hipStream_t st;
};

hipError_t fork_begin(const mh3a_decoder* d, const BlockBufs* bb, int nrb, hipStream_t st) {
    hipError_t e = hipEventRecord(d->fork_ev, st);
    for (int j = 0; j + 1 < nrb && e == hipSuccess; ++j) e = hipStreamWaitEvent(bb[j].st, d->fork_ev, 0);
    return e;
}

int run_amp_units(const mh3a_decoder* d, int stage, const float* h, const BlockBufs* bb, bool fork, float* s_buf,
                  int batch, int64_t len, bool bf16) {
    const mh3a_config& c = d->cfg;
    const int C = d->stage_c[stage];
    const int nrb = c.num_resblocks, nd = c.num_dilations;
    const bool split = amp_unit_split(d, stage);
    // fp16 pieces in the default matrix form (the bf16 flag keeps bf16 pieces)
    bool h16 = split && !bf16 && d->cfg.matrix_form == MH3A_MATRIX_SPLIT_F16;
    for (const ConvLayer& L : d->amp[stage])
        if (L.whu_off < 0) h16 = false;
    if (fork) HIP_TRY(fork_begin(d, bb, nrb, bb[nrb - 1].st));
    for (int j = 0; j < nrb; ++j) {
        const float* xin = h;
        float* const x_buf = bb[j].x;
        float* const t_buf = bb[j].t;
        const hipStream_t st = bb[j].st;
        for (int n = 0; n < nd; ++n) {
            const ConvLayer& c1 = d->amp[stage][(j * nd + n) * 2 + 0];
            const ConvLayer& c2 = d->amp[stage][(j * nd + n) * 2 + 1];
            const bool last = (n == nd - 1);
            if (fork && last && j > 0) HIP_TRY(hipStreamWaitEvent(st, d->done_ev[j - 1], 0));
            UnitArgs u;
            u.x = xin;
            u.y = last ? s_buf : ((n & 1) ? t_buf : x_buf);
            u.sum_in = (last && j > 0) ? s_buf : nullptr;
            u.scale = (last && j == nrb - 1) ? 1.0f / (float)nrb : 1.0f;
            u.bstride = (int64_t)C * len;
            u.c = C;
            u.l = (int)len;
            u.taps = c1.taps;
            u.dil = c1.dil;
            u.split = split ? (h16 ? 2 : (bf16 ? 3 : 6)) : 0;
            u.w1 = d->blob + (h16 ? c1.whu_off : (split ? c1.w6u_off : c1.w16_off));
            u.b1 = d->blob + c1.b_off;
            u.act1 = act_params(d, c1.act);
            u.w2 = d->blob + (h16 ? c2.whu_off : (split ? c2.w6u_off : c2.w16_off));
            u.wscale1 = h16 ? c1.wh_scale : 1.0f;
            u.wscale2 = h16 ? c2.wh_scale : 1.0f;
            u.b2 = d->blob + c2.b_off;
            u.act2 = act_params(d, c2.act);
            if (c2.taps != c1.taps || c2.dil != 1) return fail(MH3A_E_INVALID_ARG, "unit convs disagree");
            TimedLaunch tl(d, st, KIND_AMP_UNIT);
            HIP_TRY(launch_unit(u, batch, st));
            const double n_out = (double)batch * C * len;
            // two convs of 2 C k multiply-adds per output
            tl.done(KIND_AMP_UNIT, 2.0 * 2.0 * C * (double)c1.alg_taps * n_out,
                    4.0 * (n_out * (2 + (u.sum_in ? 1 : 0)) + 2.0 * C * C * c1.alg_taps + 2.0 * C));
            if (fork && last && j + 1 < nrb) HIP_TRY(hipEventRecord(d->done_ev[j], st));
            xin = u.y;
        }
    }
    return MH3A_OK;
}

int run_amp(const mh3a_decoder* d, int stage, const float* h, const BlockBufs* bb, bool fork, float* s_buf,
            int batch, int64_t len, bool bf16, bool invariant, int ways = 1) {
    const mh3a_config& c = d->cfg;
    const int C = d->stage_c[stage];
    const int64_t bs = (int64_t)C * len;
    const int nrb = c.num_resblocks, nd = c.num_dilations;
    const int L = (int)len;
    if (amp_unit_path(d, stage, bf16)) return run_amp_units(d, stage, h, bb, fork, s_buf, batch, len, bf16);
    const bool fused = amp_act_fused(d, batch, C, len);
    const int64_t pbs = pk_item_floats(d, C, len);  // packed batch stride
    const int plp = fused ? 0 : (int)pk_lp(len);
    const bool px = stage_px(d, batch, C, len, bf16);  // packed inputs in a split-product form
    const bool h16 = px && use_h16(d) && !bf16;         // ... the fp16 one (the bf16 flag keeps bf16 pieces)
    const int pieces = px ? (h16 ? kPiecesH : kPieces) : 0;
    if (fork) HIP_TRY(fork_begin(d, bb, nrb, bb[nrb - 1].st));
    for (int j = 0; j < nrb; ++j) {
        float* const x_buf = bb[j].x;
        float* const t_buf = bb[j].t;
        float* const a_buf = bb[j].a;
        float* const partial = bb[j].partial;
        const hipStream_t st = bb[j].st;
        for (int n = 0; n < nd; ++n) {
            const ConvLayer& c1 = d->amp[stage][(j * nd + n) * 2 + 0];
            const ConvLayer& c2 = d->amp[stage][(j * nd + n) * 2 + 1];
            const float* xin = (n == 0) ? h : x_buf;
            const float* in1 = xin;
            if (!fused) {
                HIP_TRY(run_act(d, c1.act, xin, a_buf, batch, C, len, pieces, st));
                in1 = a_buf;
            }
            HIP_TRY(run_conv(d, c1, in1, fused ? bs : pbs, L, L, t_buf, bs, batch, nullptr, nullptr, 1.0f, bf16,
                             invariant, fused, partial, st, plp, px, h16, ways));
            const float* in2 = t_buf;
            if (!fused) {
                HIP_TRY(run_act(d, c2.act, t_buf, a_buf, batch, C, len, pieces, st));
                in2 = a_buf;
            }
            const bool last = (n == nd - 1);
            float* yout = last ? s_buf : x_buf;
            const float* sum_in = (last && j > 0) ? s_buf : nullptr;
            const float scale = (last && j == nrb - 1) ? 1.0f / (float)nrb : 1.0f;
            if (fork && last && j > 0) HIP_TRY(hipStreamWaitEvent(st, d->done_ev[j - 1], 0));
            HIP_TRY(run_conv(d, c2, in2, fused ? bs : pbs, L, L, yout, bs, batch, xin, sum_in, scale, bf16, invariant,
                             fused, partial, st, plp, px, h16, ways));
            if (fork && last && j + 1 < nrb) HIP_TRY(hipEventRecord(d->done_ev[j], st));
        }
    }
    return MH3A_OK;
}

int check_decode_args(const mh3a_decoder* d, int64_t batch, int64_t frames, uint32_t flags) {
    if (!d) return fail(MH3A_E_INVALID_ARG, "decoder is null");
    if (batch < 1 || batch > 4096) return fail(MH3A_E_INVALID_ARG, "batch must be in [1, 4096]");
    if (frames < 1) return fail(MH3A_E_INVALID_ARG, "frames must be >= 1");
    if (flags & ~MH3A_FLAG_ALL) return fail(MH3A_E_INVALID_ARG, "unknown flags 0x%x", flags & ~MH3A_FLAG_ALL);
    // every per-item length must fit the kernels' 32-bit positions
    if ((int64_t)d->cfg.hop_length * frames > (int64_t)1 << 30)
        return fail(MH3A_E_INVALID_ARG, "frames too large: %lld output samples per item", (long long)(d->cfg.hop_length * frames));
    // the kernels address one batch item's tensor with 32-bit byte offsets
    if (max_cl(d, frames) >= ((int64_t)1 << 29)) return fail(MH3A_E_INVALID_ARG, "frames too large for one item");
    return MH3A_OK;
}

// Largest partial-sum region any conv of one AMP stage needs.
int64_t amp_partial_floats(const mh3a_decoder* d, int stage, int batch, int len, bool bf16, bool inv,
                           int ways = 1) {
    int64_t m = 0;
    if (amp_unit_path(d, stage, bf16)) return 0;  // the unit kernel splits no contraction
    const bool fused = amp_act_fused(d, batch, d->stage_c[stage], len);
    const bool px = stage_px(d, batch, d->stage_c[stage], len, bf16);
    for (const ConvLayer& L : d->amp[stage])
        m = std::max(m, plan_partial_floats(L, len, batch * L.phases,
                                            plan_conv(d, L, len, batch, bf16, inv, fused, px, ways), fused));
    return m;
}

// Largest partial-sum region any conv of a decode needs.
// (in_proj, conv_pre and the upsamplers always run full fp32 operands.)
int64_t decode_partial_floats(const mh3a_decoder* d, int batch, int frames, bool bf16, bool inv,
                              int ways = 1) {
    const mh3a_config& c = d->cfg;
    int64_t m = 0;
    for (const ConvLayer* L : {&d->in_proj, &d->in_proj_dn, &d->conv_pre})
        m = std::max(m, plan_partial_floats(*L, frames, batch * L->phases,
                                            plan_conv(d, *L, frames, batch, false, inv, true, pre_bx6(d, *L)), true));
    int64_t len = frames;
    for (int s = 0; s < c.num_ups; ++s) {
        const ConvLayer& U = d->ups[s];
        m = std::max(m, plan_partial_floats(U, (int)len, batch * U.phases,
                                            plan_conv(d, U, (int)len, batch, false, inv, true, pre_bx6(d, U)), true));
        len *= c.rates[s];
        m = std::max(m, amp_partial_floats(d, s, batch, (int)len, bf16, inv, ways));
    }
    return m;
}

// Floats of the packed activated input of stage s (0 when its convs fuse the
// activation).
int64_t stage_pk_floats(const mh3a_decoder* d, int stage, int64_t batch, int64_t len) {
    if (amp_act_fused(d, batch, d->stage_c[stage], len)) return 0;
    return round_up(batch * pk_item_floats(d, d->stage_c[stage], len), 64);
}

int64_t decode_pk_floats(const mh3a_decoder* d, int64_t batch, int64_t frames) {
    int64_t m = 0, len = frames;
    if (pre_bx6(d, d->conv_pre)) m = round_up(batch * pk_item_floats(d, d->conv_pre.c_in, frames), 64);
    for (int s = 0; s < d->cfg.num_ups; ++s) {
        if (pre_bx6(d, d->ups[s])) m = std::max(m, round_up(batch * pk_item_floats(d, d->ups[s].c_in, len), 64));
        len *= d->cfg.rates[s];
        m = std::max(m, stage_pk_floats(d, s, batch, len));
    }
    return m;
}

// Decodes of at most this many latents (batch x frames) run the residual
// blocks of each AMP set concurrently (see BlockBufs): their launches fill a
// fraction of the GPU each, and the decode is a chain of ~190 of them.
constexpr int64_t kForkMaxLatents = 800;

// Residual blocks that run at once in a decode (1: one after another).
int fork_ways(const mh3a_decoder* d, int64_t batch, int64_t frames, bool allow) {
    const int nrb = d->cfg.num_resblocks;
    if (!allow || nrb < 2 || (int)d->side.size() < nrb - 1 || batch * frames > kForkMaxLatents) return 1;
    return nrb;
}

// Workspace: slots S, H, X, T, then the packed activated input, then the
// partial sums of split launches; with concurrent blocks, then per side
// block its own X, T, packed input and partial sums.
struct DecodeLayout {
    int64_t slot, pk, partial;
    int ways;        // residual blocks that run at once in this call
    int plan_ways;   // ... in a decode of this shape: what the AMP conv plans assume
    int64_t per_block() const { return 2 * slot + pk + partial; }
    int64_t floats() const { return 4 * slot + pk + partial + (ways - 1) * per_block(); }
};

DecodeLayout decode_layout(const mh3a_decoder* d, int64_t batch, int64_t frames, uint32_t flags, bool allow_fork) {
    const bool bf16 = (flags & MH3A_FLAG_BF16_MFMA) != 0;
    const bool inv = (flags & MH3A_FLAG_BATCH_INVARIANT) != 0;
    DecodeLayout l;
    l.slot = round_up(max_cl(d, frames) * batch, 64);
    l.pk = decode_pk_floats(d, batch, frames);
    l.ways = fork_ways(d, batch, frames, allow_fork);
    // the plans depend on the shape only, so that the no-allocation decode
    // (blocks one after another) gives the same bits
    l.plan_ways = fork_ways(d, batch, frames, true);
    l.partial = round_up(decode_partial_floats(d, (int)batch, (int)frames, bf16, inv, l.plan_ways), 64);
    return l;
}

size_t decode_ws_bytes(const mh3a_decoder* d, int64_t batch, int64_t frames, uint32_t flags, bool allow_fork = true) {
    return (size_t)(decode_layout(d, batch, frames, flags, allow_fork).floats() * (int64_t)sizeof(float));
}

int run_decode(mh3a_decoder* d, const float* z, int64_t batch, int64_t frames, float* wave, int upto,
               float* out, void* ws, size_t ws_bytes, uint32_t flags, hipStream_t st, bool allow_fork = true) {
    int rc = check_decode_args(d, batch, frames, flags);
    if (rc) return rc;
    if (!z || (!wave && !out)) return fail(MH3A_E_INVALID_ARG, "null latents or output pointer");
    if (!ws) return fail(MH3A_E_WORKSPACE, "workspace is null");
    if ((uintptr_t)ws % 256) return fail(MH3A_E_WORKSPACE, "workspace must be 256-byte aligned");
    const DecodeLayout lay = decode_layout(d, batch, frames, flags, allow_fork);
    const size_t need = (size_t)(lay.floats() * (int64_t)sizeof(float));
    if (ws_bytes < need) return fail(MH3A_E_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    const mh3a_config& c = d->cfg;
    const int B = (int)batch;
    const int N = (int)frames;
    const int64_t slot = lay.slot;
    float* bufS = static_cast<float*>(ws);
    float* bufH = bufS + slot;
    float* bufX = bufH + slot;
    float* bufT = bufX + slot;
    float* bufA = bufT + slot;
    float* partial = bufA + lay.pk;
    // per residual block: its scratch and stream (the last block, or every
    // block when they run one after another, on the caller's stream)
    const int nrb = c.num_resblocks;
    const bool fork = lay.ways > 1;
    std::vector<BlockBufs> blocks(nrb, BlockBufs{bufX, bufT, bufA, partial, st});
    if (fork) {
        float* p = partial + lay.partial;
        for (int j = 0; j + 1 < nrb; ++j, p += lay.per_block())
            blocks[j] = BlockBufs{p, p + slot, p + 2 * slot, p + 2 * slot + lay.pk, d->side[j]};
    }
    std::unique_lock<std::mutex> fork_lock(d->fork_mu, std::defer_lock);
    if (fork) fork_lock.lock();  // one forked decode enqueues at a time (shared side streams and events)
    const bool bf16 = (flags & MH3A_FLAG_BF16_MFMA) != 0;
    const bool invariant = (flags & MH3A_FLAG_BATCH_INVARIANT) != 0;
    HIP_TRY(hipSetDevice(d->device));

    auto finish = [&](const float* src, int64_t count) -> int {
        HIP_TRY(hipMemcpyAsync(out, src, sizeof(float) * count, hipMemcpyDeviceToDevice, st));
        return ok();
    };

    const ConvLayer& inp = (flags & MH3A_FLAG_DENORMALIZE) ? d->in_proj_dn : d->in_proj;
    const int64_t zb = (int64_t)c.latent_channels * N;
    HIP_TRY(run_conv(d, inp, z, zb, N, N, bufX, (int64_t)c.latent_dim * N, B, nullptr, nullptr, 1.0f, false, invariant,
                     true, partial, st));
    if (upto == 0) return finish(bufX, (int64_t)B * c.latent_dim * N);
    if (pre_bx6(d, d->conv_pre)) {
        const bool h16 = pre_h16(d, d->conv_pre);
        HIP_TRY(run_split(d, bufX, bufA, B, c.latent_dim, N, h16 ? kPiecesH : kPieces, st));
        HIP_TRY(run_conv(d, d->conv_pre, bufA, pk_item_floats(d, c.latent_dim, N), N, N, bufS,
                         (int64_t)c.decoder_dim * N, B, nullptr, nullptr, 1.0f, false, invariant, true, partial, st,
                         (int)pk_lp(N), true, h16));
    } else {
        HIP_TRY(run_conv(d, d->conv_pre, bufX, (int64_t)c.latent_dim * N, N, N, bufS, (int64_t)c.decoder_dim * N, B,
                         nullptr, nullptr, 1.0f, false, invariant, true, partial, st));
    }
    if (upto == 1) return finish(bufS, (int64_t)B * c.decoder_dim * N);
    int64_t len = N;
    int cin = c.decoder_dim;
    for (int s = 0; s < c.num_ups; ++s) {
        const int C = d->stage_c[s];
        const int64_t lout = len * c.rates[s];
        if (d->ups[s].wv_off >= 0) {
            HIP_TRY(run_ups_vec(d, d->ups[s], bufS, bufH, B, (int)len, c.kernels[s], st));
        } else if (pre_bx6(d, d->ups[s])) {
            const bool h16 = pre_h16(d, d->ups[s]);
            HIP_TRY(run_split(d, bufS, bufA, B, cin, len, h16 ? kPiecesH : kPieces, st));
            HIP_TRY(run_conv(d, d->ups[s], bufA, pk_item_floats(d, cin, len), (int)len, (int)len, bufH,
                             (int64_t)C * lout, B, nullptr, nullptr, 1.0f, false, invariant, true, partial, st,
                             (int)pk_lp(len), true, h16));
        } else {
            HIP_TRY(run_conv(d, d->ups[s], bufS, (int64_t)cin * len, (int)len, (int)len, bufH, (int64_t)C * lout, B,
                             nullptr, nullptr, 1.0f, false, invariant, true, partial, st));
        }
        if (upto == 2 + 2 * s) return finish(bufH, (int64_t)B * C * lout);
        rc = run_amp(d, s, bufH, blocks.data(), fork, bufS, B, lout, bf16, invariant, lay.plan_ways);
        if (rc) return rc;
        if (upto == 3 + 2 * s) return finish(bufS, (int64_t)B * C * lout);
        len = lout;
        cin = C;
    }
    FinalArgs fa;
    fa.x = bufS;
    fa.x_bstride = (int64_t)cin * len;
    fa.c = cin;
    fa.l = (int)len;
    fa.act = act_params(d, d->post_act);
    fa.w = d->blob + d->post_w_off;
    fa.bias = d->post_bias;
    fa.y = wave;
    fa.clamp = (flags & MH3A_FLAG_NO_CLAMP) ? 0 : 1;
    if (upto >= 0) return fail(MH3A_E_INVALID_ARG, "layer index %d out of range", upto);
    TimedLaunch tl(d, st, KIND_FINAL);
    HIP_TRY(launch_final(fa, B, st));
    tl.done(KIND_FINAL, 2.0 * 7 * cin * (double)len * B, 4.0 * ((double)B * cin * len + (double)B * len + 7 * cin));
    return ok();
}

// Latents of context a decoded window needs on each side so that its
// interior equals the full decode: an upper bound on how far one output
// sample's dependence reaches, summed over the layers at the latent rate.
// conv_pre (k = 7) reaches 3; a transposed conv of kernel k and stride r
// reaches ceil(k / r) inputs; a "same" conv of kernel k and dilation d
// reaches d (k - 1) / 2; an anti-aliased activation (2x up, SnakeBeta,
// 2x down, both low-pass filters `filter_taps` long) reaches at most
// filter_taps / 2 samples; the AMP blocks of a stage run side by side, so
// the widest counts; act_post + conv_post (k = 7) close the chain.
int64_t decode_margin(const mh3a_decoder* d) {
    const mh3a_config& c = d->cfg;
    const double act = c.filter_taps / 2;
    double reach = 3.0, rate = 1.0;
    for (int s = 0; s < c.num_ups; ++s) {
        reach += (double)((c.kernels[s] + c.rates[s] - 1) / c.rates[s]) / rate;
        rate *= c.rates[s];
        double block = 0.0;
        for (int j = 0; j < c.num_resblocks; ++j) {
            const int k = c.rb_kernels[j];
            double b = 0.0;
            for (int i = 0; i < c.num_dilations; ++i)
                b += c.rb_dilations[j][i] * (k - 1) / 2 + (k - 1) / 2 + 2 * act;
            block = std::max(block, b);
        }
        reach += block / rate;
    }
    reach += (act + 3.0) / rate;
    return (int64_t)std::ceil(reach) + 1;
}

// Chunk k of a chunked decode: output latents [n0, n1) decoded from the
// window [w0, w1) = [n0 - margin, n1 + margin) cut to the sequence.
struct Chunk {
    int64_t n0, n1, w0, w1;
};
Chunk chunk_at(int64_t k, int64_t frames, int64_t cf, int64_t margin) {
    Chunk ch;
    ch.n0 = k * cf;
    ch.n1 = std::min(frames, ch.n0 + cf);
    ch.w0 = std::max<int64_t>(0, ch.n0 - margin);
    ch.w1 = std::min(frames, ch.n1 + margin);
    return ch;
}

// Distinct window lengths of a chunked decode. Chunks at least
// edge = ceil(margin / cf) + 1 away from both ends have windows of exactly
// cf + 2 margin latents, so one of them stands for all.
std::set<int64_t> chunk_window_lengths(int64_t frames, int64_t cf, int64_t margin) {
    std::set<int64_t> lens;
    const int64_t K = (frames + cf - 1) / cf;
    const int64_t edge = (margin + cf - 1) / cf + 1;
    for (int64_t k = 0; k < K; ++k) {
        const Chunk ch = chunk_at(k, frames, cf, margin);
        lens.insert(ch.w1 - ch.w0);
        if (k == edge && K - 1 - edge > k + 1) k = K - 2 - edge;
    }
    return lens;
}

int check_chunk_args(const mh3a_decoder* d, int64_t batch, int64_t frames, int64_t cf, uint32_t flags) {
    if (!d) return fail(MH3A_E_INVALID_ARG, "decoder is null");
    if (cf < 1) return fail(MH3A_E_INVALID_ARG, "chunk_frames must be >= 1");
    if (batch < 1 || batch > 4096) return fail(MH3A_E_INVALID_ARG, "batch must be in [1, 4096]");
    if (frames < 1 || frames > ((int64_t)1 << 40) / d->cfg.hop_length / batch)
        return fail(MH3A_E_INVALID_ARG, "frames out of range");
    if (flags & ~MH3A_FLAG_ALL) return fail(MH3A_E_INVALID_ARG, "unknown flags 0x%x", flags & ~MH3A_FLAG_ALL);
    return MH3A_OK;
}

// Workspace of a chunked decode: the window decode's own workspace (largest
// over the window lengths used), then the latent window and the wave
// window. One chunk covering the sequence decodes in place: no windows.
int chunked_ws_bytes(const mh3a_decoder* d, int64_t batch, int64_t frames, int64_t cf, uint32_t flags, size_t* bytes,
                     size_t* dec_bytes, int64_t* wmax) {
    *bytes = *dec_bytes = 0;
    *wmax = 0;
    int rc = check_chunk_args(d, batch, frames, cf, flags);
    if (rc) return rc;
    const int64_t margin = decode_margin(d);
    for (int64_t wl : chunk_window_lengths(frames, cf, margin)) {
        rc = check_decode_args(d, batch, wl, flags);
        if (rc) return rc;
        *dec_bytes = std::max(*dec_bytes, (size_t)round_up((int64_t)decode_ws_bytes(d, batch, wl, flags), 256));
        *wmax = std::max(*wmax, wl);
    }
    *bytes = *dec_bytes;
    if (cf < frames)
        *bytes += (size_t)(round_up(batch * d->cfg.latent_channels * *wmax, 64) +
                           round_up(batch * d->cfg.hop_length * *wmax, 64)) *
                  sizeof(float);
    return MH3A_OK;
}

// Timing state of a decoder or an encoder (mh3a_timing_enable / _read).
int timing_enable(mh3a_net* d, int enable) {
    if (!d) return fail(MH3A_E_INVALID_ARG, "handle is null");
    if (enable < 0 || enable > MH3A_TIMING_AMP_CONV) return fail(MH3A_E_INVALID_ARG, "bad timing mode %d", enable);
    d->timing.on = enable != 0;
    d->timing.amp_only = enable == MH3A_TIMING_AMP_CONV;
    d->timing.used = 0;
    d->timing.recs.clear();
    return ok();
}

int timing_read(mh3a_net* d, mh3a_kernel_stats* stats, int max_stats, int* n_stats) {
    if (!d || !n_stats || (max_stats > 0 && !stats)) return fail(MH3A_E_INVALID_ARG, "null argument");
    *n_stats = 0;
    Timing& t = d->timing;
    std::vector<int> order;
    double ms[KIND_COUNT] = {0}, fl[KIND_COUNT] = {0}, by[KIND_COUNT] = {0};
    int64_t cnt[KIND_COUNT] = {0};
    HIP_TRY(hipSetDevice(d->device));
    for (const TimingRec& r : t.recs) {
        HIP_TRY(hipEventSynchronize(t.evs[r.ev + 1]));
        float e = 0.0f;
        HIP_TRY(hipEventElapsedTime(&e, t.evs[r.ev], t.evs[r.ev + 1]));
        if (cnt[r.kind] == 0) order.push_back(r.kind);
        ms[r.kind] += e;
        fl[r.kind] += r.flops;
        by[r.kind] += r.bytes;
        cnt[r.kind] += 1;
    }
    t.recs.clear();
    t.used = 0;
    int n = 0;
    for (int k : order) {
        if (n >= max_stats) break;
        mh3a_kernel_stats& o = stats[n++];
        std::memset(&o, 0, sizeof o);
        std::snprintf(o.name, sizeof o.name, "%s", kKindNames[k]);
        o.launches = cnt[k];
        o.ms = ms[k];
        o.flops = fl[k];
        o.bytes = by[k];
    }
    *n_stats = n;
    return ok();
}

}  // namespace

namespace mh3a {

int64_t packed_weight_floats(int c_out, int c_in, int taps) {
    const int64_t mb = (c_out + 31) / 32;
    const int64_t g = (int64_t)((c_in + kChunk - 1) / kChunk) * taps;
    return mb * g * 64 * 4;
}

// A-operand order of v_mfma_f32_32x32x2f32: for M-block mb, K-group g =
// chunk * taps + tap (4 K-steps = the 4 channel pairs of the chunk), lane l
// and step p, the value is W[mb*32 + l%32, chunk*8 + 2p + l/32, tap].
void pack_conv_weights(const float* w, int c_out, int c_in, int taps, float* out) {
    const int nmb = (c_out + 31) / 32;
    const int nch = (c_in + kChunk - 1) / kChunk;
    const int64_t G = (int64_t)nch * taps;
    for (int mb = 0; mb < nmb; ++mb)
        for (int ch = 0; ch < nch; ++ch)
            for (int j = 0; j < taps; ++j) {
                const int64_t g = (int64_t)ch * taps + j;
                for (int l = 0; l < 64; ++l)
                    for (int p = 0; p < 4; ++p) {
                        const int o = mb * 32 + (l & 31);
                        const int i = ch * kChunk + 2 * p + (l >> 5);
                        float v = 0.0f;
                        if (o < c_out && i < c_in) v = w[((int64_t)o * c_in + i) * taps + j];
                        out[(((int64_t)mb * G + g) * 64 + l) * 4 + p] = v;
                    }
            }
}

int64_t packed_weight_floats16(int c_out, int c_in, int taps) {
    const int64_t mb = (c_out + 15) / 16;
    const int64_t g = (int64_t)((c_in + kChunk - 1) / kChunk) * taps;
    return mb * g * 64 * 2;
}

// A-operand order of v_mfma_f32_16x16x4f32: for 16-row block mb, K-group
// g = chunk * taps + tap, lane l and half s, the value is
// W[mb*16 + l%16, chunk*8 + 4s + l/16, tap].
void pack_conv_weights16(const float* w, int c_out, int c_in, int taps, float* out) {
    const int nmb = (c_out + 15) / 16;
    const int nch = (c_in + kChunk - 1) / kChunk;
    const int64_t G = (int64_t)nch * taps;
    for (int mb = 0; mb < nmb; ++mb)
        for (int ch = 0; ch < nch; ++ch)
            for (int j = 0; j < taps; ++j) {
                const int64_t g = (int64_t)ch * taps + j;
                for (int l = 0; l < 64; ++l)
                    for (int h = 0; h < 2; ++h) {
                        const int o = mb * 16 + (l & 15);
                        const int i = ch * kChunk + 4 * h + (l >> 4);
                        float v = 0.0f;
                        if (o < c_out && i < c_in) v = w[((int64_t)o * c_in + i) * taps + j];
                        out[(((int64_t)mb * G + g) * 64 + l) * 2 + h] = v;
                    }
            }
}

// Split-product weights for v_mfma_f32_32x32x16_bf16. The (chunk, tap)
// slots of a 32-row block run chunk-major, s = chunk * taps + tap, and pair
// P holds slots 2P (lanes 0-31) and 2P + 1 (lanes 32-63): for piece p and
// lane l the 8 bf16 values piece_p(W[mb*32 + l%32, ch*8 + i, j]), i = 0..7,
// with (ch, j) = divmod(2P + l/32, taps) (zero past c_out, c_in or the last
// slot), at 16-byte group ((mb * npairs + P) * kPieces + p) * 64 + l.
// Pieces: v0 = bf16(v), v1 = bf16(v - v0), v2 = bf16(v - v0 - v1), rounded to
// nearest even.
int64_t packed_weight_floats6(int c_out, int c_in, int taps) {
    const int64_t nmb = (c_out + 31) / 32, nch = (c_in + kChunk - 1) / kChunk, np = (nch * taps + 1) / 2;
    return nmb * np * kPieces * 64 * 4;
}

static uint32_t bf16_rne_bits(float v) {
    uint32_t u;
    std::memcpy(&u, &v, 4);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
static float bf16_bits_value(uint32_t b) {
    const uint32_t u = b << 16;
    float v;
    std::memcpy(&v, &u, 4);
    return v;
}

void pack_conv_weights6(const float* w, int c_out, int c_in, int taps, float* out) {
    const int nmb = (c_out + 31) / 32, nch = (c_in + kChunk - 1) / kChunk, np = (nch * taps + 1) / 2;
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    for (int mb = 0; mb < nmb; ++mb)
        for (int q = 0; q < np; ++q)
            for (int l = 0; l < 64; ++l) {
                const int slot = 2 * q + (l >> 5), ch = slot / taps, j = slot % taps;
                uint16_t pc[kPieces][kChunk];
                for (int i = 0; i < kChunk; ++i) {
                    const int m = mb * 32 + (l & 31), c = ch * kChunk + i;
                    const float v = (m < c_out && ch < nch && c < c_in) ? w[((int64_t)m * c_in + c) * taps + j] : 0.0f;
                    const uint32_t p0 = bf16_rne_bits(v);
                    const float r1 = v - bf16_bits_value(p0);
                    const uint32_t p1 = bf16_rne_bits(r1);
                    const uint32_t p2 = bf16_rne_bits(r1 - bf16_bits_value(p1));
                    pc[0][i] = (uint16_t)p0;
                    pc[1][i] = (uint16_t)p1;
                    pc[2][i] = (uint16_t)p2;
                }
                for (int p = 0; p < kPieces; ++p) {
                    uint32_t* g = o + ((((int64_t)mb * np + q) * kPieces + p) * 64 + l) * 4;
                    for (int k = 0; k < 4; ++k) g[k] = (uint32_t)pc[p][2 * k] | ((uint32_t)pc[p][2 * k + 1] << 16);
                }
            }
}

// fp16 pieces of a layer's weights for v_mfma_f32_32x32x16_f16 (see
// kPiecesH): w' = w 2^e with e chosen so that max |w'| lies in [2^14, 2^15),
// w0 = fp16(w'), w1 = fp16(w' - w0), both rounded to nearest even; the
// operand order of pack_conv_weights6 with two pieces.
int weight_exponent_h(const float* w, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) m = std::max(m, std::fabs(w[i]));
    if (!(m > 0.0f) || !std::isfinite(m)) return 0;
    int k = 0;
    std::frexp(m, &k);  // m = f 2^k, f in [0.5, 1)
    return std::min(100, std::max(-100, 15 - k));
}

int64_t packed_weight_floats_h(int c_out, int c_in, int taps) {
    const int64_t nmb = (c_out + 31) / 32, nch = (c_in + kChunk - 1) / kChunk, np = (nch * taps + 1) / 2;
    return nmb * np * kPiecesH * 64 * 4;
}

static uint16_t f16_bits(float v) {
    const _Float16 h = (_Float16)v;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}
static float f16_value(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

void pack_conv_weights_h(const float* w, int c_out, int c_in, int taps, int e, float* out) {
    const int nmb = (c_out + 31) / 32, nch = (c_in + kChunk - 1) / kChunk, np = (nch * taps + 1) / 2;
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    for (int mb = 0; mb < nmb; ++mb)
        for (int q = 0; q < np; ++q)
            for (int l = 0; l < 64; ++l) {
                const int slot = 2 * q + (l >> 5), ch = slot / taps, j = slot % taps;
                uint16_t pc[kPiecesH][kChunk];
                for (int i = 0; i < kChunk; ++i) {
                    const int m = mb * 32 + (l & 31), c = ch * kChunk + i;
                    const float v = (m < c_out && ch < nch && c < c_in)
                                        ? std::ldexp(w[((int64_t)m * c_in + c) * taps + j], e) : 0.0f;
                    const uint16_t p0 = f16_bits(v);
                    pc[0][i] = p0;
                    pc[1][i] = f16_bits(v - f16_value(p0));
                }
                for (int p = 0; p < kPiecesH; ++p) {
                    uint32_t* g = o + ((((int64_t)mb * np + q) * kPiecesH + p) * 64 + l) * 4;
                    for (int k = 0; k < 4; ++k) g[k] = (uint32_t)pc[p][2 * k] | ((uint32_t)pc[p][2 * k + 1] << 16);
                }
            }
}

// Split-product weights of the unit kernel (v_mfma_f32_16x16x32_bf16): for
// 16-row block mb, K-step ks, piece p and lane l, the 8 bf16 values
// piece_p(W[mb*16 + l%16, cb*8 + i, ks*TG + tsub]), i = 0..7, where the
// lane's K-group l/16 is (cb = (l/16) % CB, tsub = (l/16) / CB), CB = c/8
// channel blocks, TG = 4/CB taps per step; zero past c or the last tap.
// 16-byte group ((mb * KS + ks) * kPieces + p) * 64 + l.
int64_t unit_weight_floats6(int c, int taps) {
    const int cb = c / 8, tg = 4 / cb, ks = (taps + tg - 1) / tg, nmb = (c + 15) / 16;
    return (int64_t)nmb * ks * kPieces * 64 * 4;
}

void pack_unit_weights6(const float* w, int c, int taps, float* out) {
    const int CB = c / 8, TG = 4 / CB, KS = (taps + TG - 1) / TG, nmb = (c + 15) / 16;
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    for (int mb = 0; mb < nmb; ++mb)
        for (int ks = 0; ks < KS; ++ks)
            for (int l = 0; l < 64; ++l) {
                const int g4 = l >> 4, cb = g4 % CB, tsub = g4 / CB, m = mb * 16 + (l & 15), j = ks * TG + tsub;
                uint16_t pc[kPieces][8];
                for (int i = 0; i < 8; ++i) {
                    const int ci = cb * 8 + i;
                    const float v = (m < c && ci < c && j < taps) ? w[((int64_t)m * c + ci) * taps + j] : 0.0f;
                    const uint32_t p0 = bf16_rne_bits(v);
                    const float r1 = v - bf16_bits_value(p0);
                    const uint32_t p1 = bf16_rne_bits(r1);
                    const uint32_t p2 = bf16_rne_bits(r1 - bf16_bits_value(p1));
                    pc[0][i] = (uint16_t)p0;
                    pc[1][i] = (uint16_t)p1;
                    pc[2][i] = (uint16_t)p2;
                }
                for (int p = 0; p < kPieces; ++p) {
                    uint32_t* g = o + ((((int64_t)mb * KS + ks) * kPieces + p) * 64 + l) * 4;
                    for (int k = 0; k < 4; ++k) g[k] = (uint32_t)pc[p][2 * k] | ((uint32_t)pc[p][2 * k + 1] << 16);
                }
            }
}

// The same operand order with two fp16 pieces of w 2^e (see
// pack_conv_weights_h).
int64_t unit_weight_floats_h(int c, int taps) {
    const int cb = c / 8, tg = 4 / cb, ks = (taps + tg - 1) / tg, nmb = (c + 15) / 16;
    return (int64_t)nmb * ks * kPiecesH * 64 * 4;
}

void pack_unit_weights_h(const float* w, int c, int taps, int e, float* out) {
    const int CB = c / 8, TG = 4 / CB, KS = (taps + TG - 1) / TG, nmb = (c + 15) / 16;
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    for (int mb = 0; mb < nmb; ++mb)
        for (int ks = 0; ks < KS; ++ks)
            for (int l = 0; l < 64; ++l) {
                const int g4 = l >> 4, cb = g4 % CB, tsub = g4 / CB, m = mb * 16 + (l & 15), j = ks * TG + tsub;
                uint16_t pc[kPiecesH][8];
                for (int i = 0; i < 8; ++i) {
                    const int ci = cb * 8 + i;
                    const float v =
                        (m < c && ci < c && j < taps) ? std::ldexp(w[((int64_t)m * c + ci) * taps + j], e) : 0.0f;
                    const uint16_t p0 = f16_bits(v);
                    pc[0][i] = p0;
                    pc[1][i] = f16_bits(v - f16_value(p0));
                }
                for (int p = 0; p < kPiecesH; ++p) {
                    uint32_t* g = o + ((((int64_t)mb * KS + ks) * kPiecesH + p) * 64 + l) * 4;
                    for (int k = 0; k < 4; ++k) g[k] = (uint32_t)pc[p][2 * k] | ((uint32_t)pc[p][2 * k + 1] << 16);
                }
            }
}

}  // namespace mh3a

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

void mh3a_config_default(mh3a_config* c) {
    if (!c) return;
    std::memset(c, 0, sizeof *c);
    c->latent_channels = 32;
    c->latent_dim = 2048;
    c->decoder_dim = 1024;
    c->hop_length = 800;
    c->num_ups = 7;
    const int rates[7] = {5, 5, 2, 2, 2, 2, 2};
    const int kernels[7] = {9, 9, 4, 4, 4, 4, 4};
    for (int s = 0; s < 7; ++s) {
        c->rates[s] = rates[s];
        c->kernels[s] = kernels[s];
    }
    c->num_resblocks = 3;
    c->rb_kernels[0] = 3;
    c->rb_kernels[1] = 7;
    c->rb_kernels[2] = 11;
    c->num_dilations = 3;
    for (int j = 0; j < 3; ++j) {
        c->rb_dilations[j][0] = 1;
        c->rb_dilations[j][1] = 3;
        c->rb_dilations[j][2] = 5;
    }
    c->filter_taps = 12;
    c->filter_cutoff = 0.25;
    c->filter_half_width = 0.3;
    c->matrix_form = MH3A_MATRIX_SPLIT_F16;
}

const char* mh3a_last_error(void) { return g_err.c_str(); }

namespace {
// The side streams (default priority, not synchronizing with the null
// stream) and ordering events of the concurrent AMP blocks, on the current
// device; false if any creation fails (mh3a_destroy releases what exists).
bool create_fork(mh3a_decoder* d) {
    const int nside = d->cfg.num_resblocks - 1;
    if (nside < 1) return true;
    if (hipEventCreateWithFlags(&d->fork_ev, hipEventDisableTiming) != hipSuccess) return false;
    d->done_ev.assign(nside, nullptr);
    for (int j = 0; j < nside; ++j) {
        hipStream_t s;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return false;
        d->side.push_back(s);
        if (hipEventCreateWithFlags(&d->done_ev[j], hipEventDisableTiming) != hipSuccess) return false;
    }
    return true;
}
}  // namespace

int mh3a_decoder_create(const mh3a_config* cfg, const mh3a_tensor* params, int n_params, const float* latents_mean,
                        const float* latents_std, int device, mh3a_decoder** out) {
    if (!out) return fail(MH3A_E_INVALID_ARG, "out is null");
    *out = nullptr;
    if (!cfg) return fail(MH3A_E_INVALID_ARG, "config is null");
    if (n_params < 0 || (n_params > 0 && !params)) return fail(MH3A_E_INVALID_ARG, "bad parameter list");
    if (device < 0) return fail(MH3A_E_INVALID_ARG, "device must be >= 0");
    int rc = check_config(cfg);
    if (rc) return rc;

    Table t;
    for (int i = 0; i < n_params; ++i) {
        const mh3a_tensor& p = params[i];
        if (!p.name || !p.data) return fail(MH3A_E_INVALID_ARG, "parameter %d has a null name or data", i);
        if (p.ndim < 1 || p.ndim > 3) return fail(MH3A_E_SHAPE, "%s: ndim must be 1..3", p.name);
        Param q;
        q.data = p.data;
        q.ndim = p.ndim;
        for (int k = 0; k < 3; ++k) q.shape[k] = k < p.ndim ? p.shape[k] : 1;
        for (int k = 0; k < p.ndim; ++k)
            if (q.shape[k] < 1) return fail(MH3A_E_SHAPE, "%s: non-positive dimension", p.name);
        t.m[p.name] = q;
    }

    mh3a_decoder* d = new (std::nothrow) mh3a_decoder();
    if (!d) return fail(MH3A_E_NOMEM, "out of host memory");
    std::unique_ptr<mh3a_decoder> guard(d);
    d->cfg = *cfg;
    d->device = device;
    const mh3a_config& c = d->cfg;

    float designed[kTaps];
    design_lowpass(c.filter_cutoff, c.filter_half_width, c.filter_taps, designed);

    Blob blob;
    std::vector<float> w;
    const float* bias;

    // dec_in_proj (1x1, no weight norm); de-normalized copy folds
    // z * std + mean: W' = W diag(std), b' = b + W mean.
    {
        const Param* wp = t.get("dec_in_proj.weight");
        if (!wp) return fail(MH3A_E_MISSING_TENSOR, "missing dec_in_proj.weight");
        if ((rc = fetch_weight(t, "dec_in_proj", c.latent_dim, c.latent_channels, 1, w))) return rc;
        if ((rc = fetch_vector(t, "dec_in_proj.bias", c.latent_dim, &bias))) return rc;
        add_conv(blob, d->in_proj, w, bias, c.latent_dim, c.latent_channels, 1);
        d->in_proj.kind = KIND_IN_PROJ;
        std::vector<float> w2(w.size()), b2(c.latent_dim);
        for (int o = 0; o < c.latent_dim; ++o) {
            double bb = bias[o];
            for (int i = 0; i < c.latent_channels; ++i) {
                const double wi = w[(size_t)o * c.latent_channels + i];
                const double sd = latents_std ? latents_std[i] : 1.0;
                const double mu = latents_mean ? latents_mean[i] : 0.0;
                w2[(size_t)o * c.latent_channels + i] = (float)(wi * sd);
                bb += wi * mu;
            }
            b2[o] = (float)bb;
        }
        add_conv(blob, d->in_proj_dn, w2, b2.data(), c.latent_dim, c.latent_channels, 1);
        d->in_proj_dn.kind = KIND_IN_PROJ;
    }
    // conv_pre: k = 7, pad 3
    if (!t.get("decoder.conv_pre.weight_v") && !t.get("decoder.conv_pre.weight"))
        return fail(MH3A_E_MISSING_TENSOR, "missing decoder.conv_pre.weight_v");
    if ((rc = fetch_weight(t, "decoder.conv_pre", c.decoder_dim, c.latent_dim, 7, w))) return rc;
    if ((rc = fetch_vector(t, "decoder.conv_pre.bias", c.decoder_dim, &bias))) return rc;
    add_conv(blob, d->conv_pre, w, bias, c.decoder_dim, c.latent_dim, 7);
    d->conv_pre.in_off[0] = -3;
    d->conv_pre.alg_taps = 7;
    d->conv_pre.kind = KIND_CONV_PRE;
    d->conv_pre.dil = 1;
    if (split_input_ok(d->conv_pre)) {
        d->conv_pre.w6_off = blob.reserve(packed_weight_floats6(c.decoder_dim, c.latent_dim, 7));
        pack_conv_weights6(w.data(), c.decoder_dim, c.latent_dim, 7, blob.h.data() + d->conv_pre.w6_off);
        if (c.matrix_form == MH3A_MATRIX_SPLIT_F16) {
            const int e = weight_exponent_h(w.data(), (int64_t)w.size());
            d->conv_pre.wh_off = blob.reserve(packed_weight_floats_h(c.decoder_dim, c.latent_dim, 7));
            d->conv_pre.wh_scale = std::ldexp(1.0f, e);
            pack_conv_weights_h(w.data(), c.decoder_dim, c.latent_dim, 7, e, blob.h.data() + d->conv_pre.wh_off);
        }
    }

    int cin = c.decoder_dim;
    d->ups.resize(c.num_ups);
    d->amp.resize(c.num_ups);
    d->stage_c.resize(c.num_ups);
    for (int s = 0; s < c.num_ups; ++s) {
        const int C = cin / 2;
        const int r = c.rates[s], k = c.kernels[s], pad = (k - r) / 2;
        d->stage_c[s] = C;
        // Transposed conv, polyphase: output t = r m + ph reads
        // x[m + c_ph - u] with tap q = q0 + r u, q0 = (ph + pad) mod r,
        // c_ph = (ph + pad) div r; as a conv over m with taps jj = ku-1-u.
        const std::string pre = "decoder.ups." + std::to_string(s) + ".0";
        if ((rc = fetch_weight(t, pre, cin, C, k, w))) return rc;
        if ((rc = fetch_vector(t, pre + ".bias", C, &bias))) return rc;
        ConvLayer& U = d->ups[s];
        const int ku = (k + r - 1) / r;
        U.c_in = cin;
        U.c_out = C;
        U.taps = ku;
        U.phases = r;
        U.out_mul = r;
        U.alg_taps = k;
        U.kind = KIND_UPSAMPLE;
        const int64_t per = packed_weight_floats(C, cin, ku);
        U.w_off = blob.reserve(per * r);
        U.w_phase_stride = per;
        for (int ph = 0; ph < r; ++ph) {
            U.in_off[ph] = (ph + pad) / r - (ku - 1);
            U.out_add[ph] = ph;
        }
        const bool split6 = split_input_ok(U);
        const int64_t per6 = split6 ? packed_weight_floats6(C, cin, ku) : 0;
        if (split6) {
            U.w6_off = blob.reserve(per6 * r);
            U.w6_phase_stride = per6;
        }
        const bool splith = split6 && c.matrix_form == MH3A_MATRIX_SPLIT_F16;
        const int64_t perh = splith ? packed_weight_floats_h(C, cin, ku) : 0;
        const int eh = splith ? weight_exponent_h(w.data(), (int64_t)w.size()) : 0;  // one exponent for every phase
        if (splith) {
            U.wh_off = blob.reserve(perh * r);
            U.wh_phase_stride = perh;
            U.wh_scale = std::ldexp(1.0f, eh);
        }
        std::vector<float> wph((size_t)C * cin * ku);
        for (int ph = 0; ph < r; ++ph) {
            const int q0 = (ph + pad) % r;
            for (int o = 0; o < C; ++o)
                for (int i = 0; i < cin; ++i)
                    for (int jj = 0; jj < ku; ++jj) {
                        const int q = q0 + r * (ku - 1 - jj);
                        wph[((size_t)o * cin + i) * ku + jj] = q < k ? w[((size_t)i * C + o) * k + q] : 0.0f;
                    }
            pack_conv_weights(wph.data(), C, cin, ku, blob.h.data() + U.w_off + ph * per);
            if (split6) pack_conv_weights6(wph.data(), C, cin, ku, blob.h.data() + U.w6_off + ph * per6);
            if (splith) pack_conv_weights_h(wph.data(), C, cin, ku, eh, blob.h.data() + U.wh_off + ph * perh);
        }
        U.b_off = blob.add(bias, C);
        if (ups_vec_supported(cin, C, r, k)) U.wv_off = blob.add(w.data(), (int64_t)cin * C * k);
        // AMP blocks
        for (int j = 0; j < c.num_resblocks; ++j) {
            const int kk = c.rb_kernels[j];
            const std::string rb = "decoder.resblocks." + std::to_string(s * c.num_resblocks + j);
            for (int n = 0; n < c.num_dilations; ++n) {
                const int dil = c.rb_dilations[j][n];
                for (int which = 0; which < 2; ++which) {
                    const std::string cp = rb + (which == 0 ? ".convs1." : ".convs2.") + std::to_string(n);
                    if ((rc = fetch_weight(t, cp, C, C, kk, w))) return rc;
                    if ((rc = fetch_vector(t, cp + ".bias", C, &bias))) return rc;
                    ConvLayer L;
                    add_conv(blob, L, w, bias, C, C, kk);
                    if (kk == 3 || kk == 7 || kk == 11) {
                        L.w6_off = blob.reserve(packed_weight_floats6(C, C, kk));
                        pack_conv_weights6(w.data(), C, C, kk, blob.h.data() + L.w6_off);
                        if (c.matrix_form == MH3A_MATRIX_SPLIT_F16) {
                            const int e = weight_exponent_h(w.data(), (int64_t)w.size());
                            L.wh_off = blob.reserve(packed_weight_floats_h(C, C, kk));
                            L.wh_scale = std::ldexp(1.0f, e);
                            pack_conv_weights_h(w.data(), C, C, kk, e, blob.h.data() + L.wh_off);
                        }
                    }
                    if (C <= 32 && C % 8 == 0 && (kk == 3 || kk == 7 || kk == 11)) {
                        L.w6u_off = blob.reserve(unit_weight_floats6(C, kk));
                        pack_unit_weights6(w.data(), C, kk, blob.h.data() + L.w6u_off);
                        if (c.matrix_form == MH3A_MATRIX_SPLIT_F16) {
                            const int e = weight_exponent_h(w.data(), (int64_t)w.size());
                            L.whu_off = blob.reserve(unit_weight_floats_h(C, kk));
                            L.wh_scale = std::ldexp(1.0f, e);
                            pack_unit_weights_h(w.data(), C, kk, e, blob.h.data() + L.whu_off);
                        }
                    }
                    if (C <= 32 && (kk == 3 || kk == 7 || kk == 11)) {
                        L.w16_off = blob.reserve(packed_weight_floats16(C, C, kk));
                        pack_conv_weights16(w.data(), C, C, kk, blob.h.data() + L.w16_off);
                    }
                    L.dil = which == 0 ? dil : 1;
                    L.alg_taps = kk;
                    L.kind = KIND_AMP;
                    L.in_off[0] = -(L.dil * (kk - 1) / 2);
                    const std::string ap = rb + ".activations." + std::to_string(2 * n + which);
                    if ((rc = add_act(blob, t, ap, C, designed, d->acts))) return rc;
                    L.act = (int)d->acts.size() - 1;
                    d->amp[s].push_back(L);
                }
            }
        }
        cin = C;
    }
    if ((rc = add_act(blob, t, "decoder.activation_post", cin, designed, d->acts))) return rc;
    d->post_act = (int)d->acts.size() - 1;
    if (!t.get("decoder.conv_post.weight_v") && !t.get("decoder.conv_post.weight"))
        return fail(MH3A_E_MISSING_TENSOR, "missing decoder.conv_post.weight_v");
    if ((rc = fetch_weight(t, "decoder.conv_post", 1, cin, 7, w))) return rc;
    d->post_w_off = blob.add(w.data(), (int64_t)cin * 7);
    if (const Param* pb = t.get("decoder.conv_post.bias")) {
        if (!vector_of(pb, 1)) return fail(MH3A_E_SHAPE, "decoder.conv_post.bias must hold 1 value");
        d->post_bias = pb->data[0];
    }

    // every AMP conv can read a packed activated input (compile-time taps and
    // pads that cover its halo with output tiles of up to 256 positions)
    d->pk_ok = true;
    for (const auto& stage_layers : d->amp)
        for (const ConvLayer& L : stage_layers) {
            const int pad = -L.in_off[0];
            const bool taps_ok = L.taps == 3 || L.taps == 7 || L.taps == 11;
            if (!taps_ok || L.phases != 1 || pad > kPkPadL || 255 + (L.taps - 1) * L.dil - pad > kPkPadR)
                d->pk_ok = false;
        }
    d->bx6_ok = d->pk_ok;
    for (const auto& stage_layers : d->amp)
        for (const ConvLayer& L : stage_layers)
            if (L.w6_off < 0 || L.dil > kBx6MaxDil) d->bx6_ok = false;
    // the fp16 form needs the pieces of every AMP conv of the split-product stages
    d->h16_ok = d->bx6_ok && c.matrix_form == MH3A_MATRIX_SPLIT_F16;
    for (const auto& stage_layers : d->amp)
        for (const ConvLayer& L : stage_layers)
            if (L.w6_off >= 0 && L.wh_off < 0) d->h16_ok = false;

    // upload
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(MH3A_E_HIP, "no HIP device available");
    if (device >= ndev) return fail(MH3A_E_INVALID_ARG, "device %d out of range (%d devices)", device, ndev);
    HIP_TRY(hipSetDevice(device));
    HIP_TRY(hipDeviceGetAttribute(&d->num_cus, hipDeviceAttributeMultiprocessorCount, device));
    d->num_cus = std::max(1, d->num_cus);
    // the device address of this GPU's static scratch (mh3a_decode_noalloc),
    // looked up once per device
    HIP_TRY(noalloc_scratch_lookup(device));
    d->blob_floats = (int64_t)blob.h.size();
    HIP_TRY(hipMalloc((void**)&d->blob, sizeof(float) * blob.h.size()));
    if (hipMemcpy(d->blob, blob.h.data(), sizeof(float) * blob.h.size(), hipMemcpyHostToDevice) != hipSuccess ||
        !create_fork(d)) {
        mh3a_destroy(guard.release());
        return fail(MH3A_E_HIP, "uploading the parameters or creating the side streams failed");
    }
    *out = guard.release();
    return ok();
}

void mh3a_destroy(mh3a_decoder* d) {
    if (!d) return;
    if (d->blob) {
        hipSetDevice(d->device);
        hipDeviceSynchronize();
        hipFree(d->blob);
        for (hipEvent_t e : d->timing.evs) hipEventDestroy(e);
        for (hipStream_t s : d->side) hipStreamDestroy(s);
        for (hipEvent_t e : d->done_ev)
            if (e) hipEventDestroy(e);
        if (d->fork_ev) hipEventDestroy(d->fork_ev);
    }
    delete d;
}

int mh3a_timing_enable(mh3a_decoder* d, int enable) { return timing_enable(d, enable); }
int mh3a_timing_read(mh3a_decoder* d, mh3a_kernel_stats* stats, int max_stats, int* n_stats) {
    return timing_read(d, stats, max_stats, n_stats);
}

int mh3a_decode_workspace_size(const mh3a_decoder* d, int64_t batch, int64_t frames, uint32_t flags, size_t* bytes) {
    if (!bytes) return fail(MH3A_E_INVALID_ARG, "bytes is null");
    *bytes = 0;
    int rc = check_decode_args(d, batch, frames, flags);
    if (rc) return rc;
    *bytes = decode_ws_bytes(d, batch, frames, flags);
    return ok();
}

int mh3a_decode(mh3a_decoder* d, const float* latents, int64_t batch, int64_t frames, float* wave, void* workspace,
                size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!wave) return fail(MH3A_E_INVALID_ARG, "wave is null");
    return run_decode(d, latents, batch, frames, wave, -1, nullptr, workspace, workspace_bytes, flags,
                      static_cast<hipStream_t>(stream));
}

int mh3a_decode_noalloc(mh3a_decoder* d, const float* latents, int64_t batch, int64_t frames, float* wave,
                        uint32_t flags, void* stream) {
    int rc = check_decode_args(d, batch, frames, flags);
    if (rc) return rc;
    if (!wave) return fail(MH3A_E_INVALID_ARG, "wave is null");
    // (one block after another: the concurrent form needs more scratch)
    const size_t need = decode_ws_bytes(d, batch, frames, flags, false);
    if (need > kNoAllocScratchBytes)
        return fail(MH3A_E_WORKSPACE, "decode of %lld x %lld latents needs %zu bytes of scratch; the static scratch "
                    "holds %zu (use mh3a_decode with a workspace)", (long long)batch, (long long)frames, need,
                    kNoAllocScratchBytes);
    void* ws = noalloc_scratch(d->device);
    if (!ws) return fail(MH3A_E_HIP, "no static scratch address for device %d", d->device);
    return run_decode(d, latents, batch, frames, wave, -1, nullptr, ws, kNoAllocScratchBytes, flags,
                      static_cast<hipStream_t>(stream), false);
}

int mh3a_decode_layer_shape(const mh3a_decoder* d, int64_t frames, int upto, int64_t* channels, int64_t* length) {
    if (!d || !channels || !length) return fail(MH3A_E_INVALID_ARG, "null argument");
    if (frames < 1) return fail(MH3A_E_INVALID_ARG, "frames must be >= 1");
    const mh3a_config& c = d->cfg;
    if (upto < 0 || upto > 1 + 2 * c.num_ups) return fail(MH3A_E_INVALID_ARG, "layer index %d out of range", upto);
    if (upto == 0) {
        *channels = c.latent_dim;
        *length = frames;
        return ok();
    }
    if (upto == 1) {
        *channels = c.decoder_dim;
        *length = frames;
        return ok();
    }
    const int s = (upto - 2) / 2;
    int64_t len = frames;
    for (int i = 0; i <= s; ++i) len *= c.rates[i];
    *channels = d->stage_c[s];
    *length = len;
    return ok();
}

int mh3a_decode_partial(mh3a_decoder* d, const float* latents, int64_t batch, int64_t frames, int upto, float* out,
                        void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!d) return fail(MH3A_E_INVALID_ARG, "decoder is null");
    if (!out) return fail(MH3A_E_INVALID_ARG, "out is null");
    if (upto < 0 || upto > 1 + 2 * d->cfg.num_ups) return fail(MH3A_E_INVALID_ARG, "layer index %d out of range", upto);
    return run_decode(d, latents, batch, frames, nullptr, upto, out, workspace, workspace_bytes, flags,
                      static_cast<hipStream_t>(stream));
}

int mh3a_decode_margin(const mh3a_decoder* d, int64_t* margin) {
    if (!d || !margin) return fail(MH3A_E_INVALID_ARG, "null argument");
    *margin = decode_margin(d);
    return ok();
}

int mh3a_decode_chunked_workspace_size(const mh3a_decoder* d, int64_t batch, int64_t frames, int64_t chunk_frames,
                                       uint32_t flags, size_t* bytes) {
    if (!bytes) return fail(MH3A_E_INVALID_ARG, "bytes is null");
    size_t dec_bytes = 0;
    int64_t wmax = 0;
    int rc = chunked_ws_bytes(d, batch, frames, chunk_frames, flags, bytes, &dec_bytes, &wmax);
    if (rc) return rc;
    return ok();
}

int mh3a_decode_chunked(mh3a_decoder* d, const float* latents, int64_t batch, int64_t frames, int64_t chunk_frames,
                        float* wave, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    size_t need = 0, dec_bytes = 0;
    int64_t wmax = 0;
    int rc = chunked_ws_bytes(d, batch, frames, chunk_frames, flags, &need, &dec_bytes, &wmax);
    if (rc) return rc;
    if (!latents || !wave) return fail(MH3A_E_INVALID_ARG, "null latents or wave");
    if (!workspace) return fail(MH3A_E_WORKSPACE, "workspace is null");
    if ((uintptr_t)workspace % 256) return fail(MH3A_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need) return fail(MH3A_E_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (chunk_frames >= frames)
        return run_decode(d, latents, batch, frames, wave, -1, nullptr, workspace, dec_bytes, flags, st);
    HIP_TRY(hipSetDevice(d->device));
    const int64_t lc = d->cfg.latent_channels, hop = d->cfg.hop_length;
    const int64_t margin = decode_margin(d);
    float* zwin = reinterpret_cast<float*>(static_cast<char*>(workspace) + dec_bytes);
    float* ywin = zwin + round_up(batch * lc * wmax, 64);
    const int64_t K = (frames + chunk_frames - 1) / chunk_frames;
    for (int64_t k = 0; k < K; ++k) {
        const Chunk ch = chunk_at(k, frames, chunk_frames, margin);
        const int64_t wl = ch.w1 - ch.w0;
        // latent window: rows of (batch * lc) channels, wl latents from w0
        HIP_TRY(hipMemcpy2DAsync(zwin, wl * sizeof(float), latents + ch.w0, frames * sizeof(float), wl * sizeof(float),
                                 batch * lc, hipMemcpyDeviceToDevice, st));
        rc = run_decode(d, zwin, batch, wl, ywin, -1, nullptr, workspace, dec_bytes, flags, st);
        if (rc) return rc;
        // keep the samples of latents [n0, n1)
        HIP_TRY(hipMemcpy2DAsync(wave + hop * ch.n0, hop * frames * sizeof(float), ywin + hop * (ch.n0 - ch.w0),
                                 hop * wl * sizeof(float), hop * (ch.n1 - ch.n0) * sizeof(float), batch,
                                 hipMemcpyDeviceToDevice, st));
    }
    return ok();
}

int mh3a_amp_stage_workspace_size(const mh3a_decoder* d, int stage, int64_t batch, int64_t length, size_t* bytes) {
    if (!bytes) return fail(MH3A_E_INVALID_ARG, "bytes is null");
    *bytes = 0;
    if (!d) return fail(MH3A_E_INVALID_ARG, "decoder is null");
    if (stage < 0 || stage >= d->cfg.num_ups) return fail(MH3A_E_INVALID_ARG, "stage %d out of range", stage);
    if (batch < 1 || batch > 4096 || length < 1 || length > ((int64_t)1 << 30) ||
        (int64_t)d->stage_c[stage] * length >= ((int64_t)1 << 29))
        return fail(MH3A_E_INVALID_ARG, "bad batch or length");
    // the partial region covers every flag combination (the flags come later)
    int64_t part = 0;
    for (int f = 0; f < 4; ++f)
        part = std::max(part, amp_partial_floats(d, stage, (int)batch, (int)length, f & 1, f & 2));
    *bytes = (size_t)((2 * round_up(batch * d->stage_c[stage] * length, 64) + stage_pk_floats(d, stage, batch, length) +
                       part) *
                      (int64_t)sizeof(float));
    return ok();
}

int mh3a_amp_stage(mh3a_decoder* d, int stage, const float* x, int64_t batch, int64_t length, float* y,
                   void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    size_t need = 0;
    int rc = mh3a_amp_stage_workspace_size(d, stage, batch, length, &need);
    if (rc) return rc;
    if (!x || !y) return fail(MH3A_E_INVALID_ARG, "null input or output");
    if (flags & ~(MH3A_FLAG_BF16_MFMA | MH3A_FLAG_BATCH_INVARIANT))
        return fail(MH3A_E_INVALID_ARG, "unsupported flags 0x%x", flags);
    if (!workspace) return fail(MH3A_E_WORKSPACE, "workspace is null");
    if ((uintptr_t)workspace % 256) return fail(MH3A_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need) return fail(MH3A_E_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    if (x == y) return fail(MH3A_E_INVALID_ARG, "x and y must not alias");
    HIP_TRY(hipSetDevice(d->device));
    float* xb = static_cast<float*>(workspace);
    float* tb = xb + round_up(batch * d->stage_c[stage] * length, 64);
    float* ab = tb + round_up(batch * d->stage_c[stage] * length, 64);
    float* part = ab + stage_pk_floats(d, stage, batch, length);
    std::vector<BlockBufs> blocks(d->cfg.num_resblocks, BlockBufs{xb, tb, ab, part, static_cast<hipStream_t>(stream)});
    rc = run_amp(d, stage, x, blocks.data(), false, y, (int)batch, length, (flags & MH3A_FLAG_BF16_MFMA) != 0,
                 (flags & MH3A_FLAG_BATCH_INVARIANT) != 0);
    if (rc) return rc;
    return ok();
}

}  // extern "C"

// ===========================================================================
// Encoder convolution stack (FastVideo "minimax_h3_audio_vae", source of
// MLXMiniMaxH3AudioVAE.encode up to the hidden state; module overview: the
// DAC-style encoder of plain-Snake residual units): waveform (B, 1, S) ->
// hidden (B, latent_dim, ceil(S / hop)).
//
// Each strided conv (kernel 2s, stride s, padding p = ceil(s / 2)) runs as a
// 2-tap, stride-1 conv over a space-to-depth regrouping of its Snake input:
// channel c s + r at position t holds snake(x)[c, t s + r - p], so output t
// reads positions t and t + 1 with the weight w[o, c, j s + r] at tap j.
// ===========================================================================

struct SnakeLayer {
    int c = 0;
    int64_t ab_off = -1;  // [c] float2 (alpha / pi, 0.5 / (alpha + 1e-9))
};

struct mh3a_encoder : mh3a_net {
    mh3a_encoder_config cfg;
    ConvLayer conv_in;                 // 1 -> dim, k7, pad 3
    std::vector<ConvLayer> unit_conv;  // [block][unit][k7 dilated, k1]: (block * 3 + unit) * 2 + {0, 1}
    std::vector<ConvLayer> down;       // [block]: the strided conv as a 2-tap conv over C s channels
    ConvLayer conv_out;                // final k3, pad 1
    std::vector<SnakeLayer> snakes;    // [block][unit][0, 1], then [block] before `down`, then the final one
    std::vector<int> block_c;          // input channels of each block
    int hop = 1;
    // the attention projection and mean_proj (present when the parameters
    // hold pre_block.attn.qkv.weight)
    bool has_pre = false;
    ConvLayer qkv;                     // 1x1, latent_dim -> 3 latent_dim, bias (b_q, 0, b_v)
    int pre_hd = 0, pre_f = 0;         // head width, GeGLU width
    int64_t wf_off = -1, bf_off = -1, w1_off = -1, b1_off = -1, w2_off = -1, b2_off = -1, wm_off = -1, bm_off = -1;
};

namespace {

constexpr int kEncDils[3] = {1, 3, 9};

int enc_check_config(const mh3a_encoder_config* c) {
    if (c->encoder_dim < 1 || c->latent_dim < 1) return fail(MH3A_E_CONFIG, "channel counts must be positive");
    if (c->num_blocks < 1 || c->num_blocks > MH3A_MAX_ENC_BLOCKS)
        return fail(MH3A_E_CONFIG, "num_blocks must be in [1, %d]", MH3A_MAX_ENC_BLOCKS);
    int64_t hop = 1, dim = c->encoder_dim;
    for (int i = 0; i < c->num_blocks; ++i) {
        if (c->rates[i] < 1 || c->rates[i] > 16) return fail(MH3A_E_CONFIG, "rate %d of block %d out of [1, 16]", c->rates[i], i);
        hop *= c->rates[i];
        dim *= 2;
    }
    if (hop > 65536 || dim > 65536) return fail(MH3A_E_CONFIG, "encoder hop or width too large");
    if (c->matrix_form != MH3A_MATRIX_SPLIT && c->matrix_form != MH3A_MATRIX_FP32 &&
        c->matrix_form != MH3A_MATRIX_SPLIT_F16)
        return fail(MH3A_E_CONFIG, "unknown matrix_form %d", c->matrix_form);
    if (c->latent_channels < 1 || c->num_attention_heads < 1)
        return fail(MH3A_E_CONFIG, "latent_channels and num_attention_heads must be positive");
    return MH3A_OK;
}

int build_table(const mh3a_tensor* params, int n_params, Table& t) {
    for (int i = 0; i < n_params; ++i) {
        const mh3a_tensor& p = params[i];
        if (!p.name || !p.data) return fail(MH3A_E_INVALID_ARG, "parameter %d has a null name or data", i);
        if (p.ndim < 1 || p.ndim > 3) return fail(MH3A_E_SHAPE, "%s: ndim must be 1..3", p.name);
        Param q;
        q.data = p.data;
        q.ndim = p.ndim;
        for (int k = 0; k < 3; ++k) q.shape[k] = k < p.ndim ? p.shape[k] : 1;
        for (int k = 0; k < p.ndim; ++k)
            if (q.shape[k] < 1) return fail(MH3A_E_SHAPE, "%s: non-positive dimension", p.name);
        t.m[p.name] = q;
    }
    return MH3A_OK;
}

// Whether a conv of the encoder can take the split-product packed input.
bool enc_split_ok(const ConvLayer& L) {
    const bool taps_ok = L.taps == 1 || L.taps == 2 || L.taps == 3 || (L.taps == 7 && L.dil <= kBx6WideDil) ||
                         (L.taps == 11 && L.dil <= kBx6MaxDil);
    if (!taps_ok || L.c_in % 16 || L.c_out < 32 || L.dil < 1) return false;
    if ((L.c_in / kChunk) % bx6_cpi_max(L.taps)) return false;  // whole pipeline items
    return -L.in_off[0] <= kPkPadL && 255 + (L.taps - 1) * L.dil + L.in_off[0] <= kPkPadR;
}

// The split-product weights of an encoder conv (bf16 pieces; in the fp16
// form also the fp16 pieces of the weights scaled by 2^e, see kPiecesH).
void enc_pack_split(Blob& blob, ConvLayer& L, const std::vector<float>& w, int c_out, int c_in, int k, int form) {
    L.w6_off = blob.reserve(packed_weight_floats6(c_out, c_in, k));
    pack_conv_weights6(w.data(), c_out, c_in, k, blob.h.data() + L.w6_off);
    if (form == MH3A_MATRIX_SPLIT_F16) {
        const int e = weight_exponent_h(w.data(), (int64_t)w.size());
        L.wh_off = blob.reserve(packed_weight_floats_h(c_out, c_in, k));
        L.wh_scale = std::ldexp(1.0f, e);
        pack_conv_weights_h(w.data(), c_out, c_in, k, e, blob.h.data() + L.wh_off);
    }
}

// A weight-normalized conv of the encoder: fp32 packing always, split-product
// pieces where the packed path serves it.
int enc_conv(Blob& blob, const Table& t, const std::string& prefix, ConvLayer& L, int c_out, int c_in, int k, int dil,
             int pad, int kind, int form) {
    std::vector<float> w;
    const float* bias = nullptr;
    int rc = fetch_weight(t, prefix, c_out, c_in, k, w);
    if (rc) return rc;
    if ((rc = fetch_vector(t, prefix + ".bias", c_out, &bias))) return rc;
    add_conv(blob, L, w, bias, c_out, c_in, k);
    L.dil = dil;
    L.in_off[0] = -pad;
    L.alg_taps = k;
    L.kind = kind;
    if (enc_split_ok(L)) enc_pack_split(blob, L, w, c_out, c_in, k, form);
    return MH3A_OK;
}

int enc_snake_layer(Blob& blob, const Table& t, const std::string& name, int c, std::vector<SnakeLayer>& out) {
    const float* alpha = nullptr;
    int rc = fetch_vector(t, name, c, &alpha);
    if (rc) return rc;
    std::vector<float> ab(2 * (size_t)c);
    for (int i = 0; i < c; ++i) {
        ab[2 * i] = (float)((double)alpha[i] / M_PI);
        ab[2 * i + 1] = (float)(0.5 / ((double)alpha[i] + 1e-9));
    }
    SnakeLayer S;
    S.c = c;
    S.ab_off = blob.add(ab.data(), 2 * (int64_t)c);
    out.push_back(S);
    return MH3A_OK;
}

// A linear layer's weight (rows, cols), also accepted as (rows, cols, 1).
int fetch_matrix(const Table& t, const std::string& name, int64_t rows, int64_t cols, const float** out) {
    const Param* p = t.get(name);
    if (!p) return fail(MH3A_E_MISSING_TENSOR, "missing %s", name.c_str());
    if (!shape_is(p, rows, cols) && !shape_is(p, rows, cols, 1))
        return fail(MH3A_E_SHAPE, "%s must be (%lld, %lld)", name.c_str(), (long long)rows, (long long)cols);
    *out = p->data;
    return MH3A_OK;
}

// The attention projection and mean_proj (FastVideo "minimax_h3_audio_vae",
// module overview, Encoder bullet, and the source of encode). Readings:
// one fused q/k/v projection `pre_block.attn.qkv.weight` (3 D, D) with bias
// (b_q, 0, b_v) -- `pre_block.attn.q_bias` / `v_bias`, or the q and v thirds
// of a fused `qkv.bias`, absent meaning zero; the k bias is zero whatever
// is stored; H heads of hd = D / H features, scores scaled by 1 / sqrt(hd),
// causal; the heads averaged; average pooling of hd features into C =
// latent_channels streams of hd / C consecutive features; the output
// projection `pre_block.attn.proj` (C -> C); the GeGLU MLP
// `pre_block.mlp.fc1` (C -> 2 F, value half then gate half, exact GELU)
// and `pre_block.mlp.fc2` (F -> C); `mean_proj` (1x1, C -> C). The head
// mean and the pooling are linear, so they are folded here into the output
// projection's weights: wf[o][j] = proj[o][j / g] / (g H), g = hd / C.
int enc_pre_block(Blob& blob, const Table& t, mh3a_encoder* e) {
    const mh3a_encoder_config& c = e->cfg;
    const int D = c.latent_dim, H = c.num_attention_heads, C = c.latent_channels;
    if (D % H) return fail(MH3A_E_CONFIG, "latent_dim %d is not a multiple of num_attention_heads %d", D, H);
    const int hd = D / H;
    if (!attn_head_width_ok(hd)) return fail(MH3A_E_CONFIG, "head width %d must be a power of two in [8, 256]", hd);
    if (hd % C)
        return fail(MH3A_E_CONFIG, "head width %d is not a multiple of latent_channels %d (average pooling)", hd, C);
    int rc;
    const float* wqkv = nullptr;
    if ((rc = fetch_matrix(t, "pre_block.attn.qkv.weight", 3 * (int64_t)D, D, &wqkv))) return rc;
    std::vector<float> bias(3 * (size_t)D, 0.0f);
    const float* bq = nullptr;
    const float* bv = nullptr;
    if (t.get("pre_block.attn.q_bias") || t.get("pre_block.attn.v_bias")) {
        if ((rc = fetch_vector(t, "pre_block.attn.q_bias", D, &bq))) return rc;
        if ((rc = fetch_vector(t, "pre_block.attn.v_bias", D, &bv))) return rc;
    } else if (t.get("pre_block.attn.qkv.bias")) {
        const float* b3 = nullptr;
        if ((rc = fetch_vector(t, "pre_block.attn.qkv.bias", 3 * (int64_t)D, &b3))) return rc;
        bq = b3;
        bv = b3 + 2 * (size_t)D;  // the k third is not read: forced to zero
    }
    for (int i = 0; i < D; ++i) {
        bias[i] = bq ? bq[i] : 0.0f;
        bias[2 * (size_t)D + i] = bv ? bv[i] : 0.0f;
    }
    std::vector<float> w(wqkv, wqkv + 3 * (size_t)D * D);
    ConvLayer& Q = e->qkv;
    add_conv(blob, Q, w, bias.data(), 3 * D, D, 1);
    Q.dil = 1;
    Q.alg_taps = 1;
    Q.kind = KIND_ENC_CONV;
    if (enc_split_ok(Q)) enc_pack_split(blob, Q, w, 3 * D, D, 1, e->cfg.matrix_form);
    const float *wp = nullptr, *bp = nullptr, *w1 = nullptr, *b1 = nullptr, *w2 = nullptr, *b2 = nullptr;
    const float *wm = nullptr, *bm = nullptr;
    if ((rc = fetch_matrix(t, "pre_block.attn.proj.weight", C, C, &wp))) return rc;
    if ((rc = fetch_vector(t, "pre_block.attn.proj.bias", C, &bp))) return rc;
    const Param* p1 = t.get("pre_block.mlp.fc1.weight");
    if (!p1) return fail(MH3A_E_MISSING_TENSOR, "missing pre_block.mlp.fc1.weight");
    const int64_t f2 = p1->shape[0];
    if (f2 < 2 || f2 % 2) return fail(MH3A_E_SHAPE, "pre_block.mlp.fc1.weight needs an even number of rows");
    const int F = (int)(f2 / 2);
    if ((rc = fetch_matrix(t, "pre_block.mlp.fc1.weight", f2, C, &w1))) return rc;
    if ((rc = fetch_vector(t, "pre_block.mlp.fc1.bias", f2, &b1))) return rc;
    if ((rc = fetch_matrix(t, "pre_block.mlp.fc2.weight", C, F, &w2))) return rc;
    if ((rc = fetch_vector(t, "pre_block.mlp.fc2.bias", C, &b2))) return rc;
    if ((rc = fetch_matrix(t, "mean_proj.weight", C, C, &wm))) return rc;
    if ((rc = fetch_vector(t, "mean_proj.bias", C, &bm))) return rc;
    const int g = hd / C;
    std::vector<float> wf((size_t)C * hd);
    for (int o = 0; o < C; ++o)
        for (int j = 0; j < hd; ++j) wf[(size_t)o * hd + j] = (float)((double)wp[(size_t)o * C + j / g] / ((double)g * H));
    e->wf_off = blob.add(wf.data(), (int64_t)wf.size());
    e->bf_off = blob.add(bp, C);
    e->w1_off = blob.add(w1, f2 * C);
    e->b1_off = blob.add(b1, f2);
    e->w2_off = blob.add(w2, (int64_t)C * F);
    e->b2_off = blob.add(b2, C);
    e->wm_off = blob.add(wm, (int64_t)C * C);
    e->bm_off = blob.add(bm, C);
    if (pre_tail_lds_bytes(hd, C, F) > 160 * 1024) return fail(MH3A_E_CONFIG, "attention projection too wide");
    e->pre_hd = hd;
    e->pre_f = F;
    e->has_pre = true;
    return MH3A_OK;
}

bool enc_bx6(const mh3a_encoder* e, const ConvLayer& L) {
    return L.w6_off >= 0 && e->cfg.matrix_form != MH3A_MATRIX_FP32;
}
// ... in the fp16 form (two pieces, three products)
bool enc_h16(const mh3a_encoder* e, const ConvLayer& L) {
    return enc_bx6(e, L) && L.wh_off >= 0 && e->cfg.matrix_form == MH3A_MATRIX_SPLIT_F16;
}

// Per-item lengths: S' = frames * hop samples after the right pad; block i
// runs at L_i = S' / (r_0 ... r_{i-1}) positions.
int64_t enc_frames(const mh3a_encoder* e, int64_t samples) { return (samples + e->hop - 1) / e->hop; }

// Floats of one Snake output (per item) feeding conv L over l_out positions.
int64_t enc_snake_item_floats(const mh3a_encoder* e, const ConvLayer& L, int64_t l_out) {
    if (enc_bx6(e, L))
        return (int64_t)((L.c_in + kChunk - 1) / kChunk) * (enc_h16(e, L) ? kPiecesH : kPieces) * 4 * pk_lp(l_out);
    return (int64_t)L.c_in * l_out;
}

struct EncWs {
    int64_t x, r, p, partial;  // floats of each region (all items)
};

EncWs enc_ws_floats(const mh3a_encoder* e, int64_t batch, int64_t frames, bool inv, bool pre = false) {
    EncWs w{0, 0, 0, 0};
    int64_t len = frames * e->hop;
    auto part = [&](const ConvLayer& L, int64_t positions) {
        const bool bx6 = enc_bx6(e, L);
        const ConvPlan pl = plan_conv(e, L, (int)positions, (int)batch, false, inv, true, bx6);
        w.partial = std::max(w.partial, plan_partial_floats(L, (int)positions, (int)batch, pl, true));
    };
    w.x = (int64_t)e->cfg.encoder_dim * len;
    part(e->conv_in, len);
    for (int i = 0; i < e->cfg.num_blocks; ++i) {
        const int C = e->block_c[i], s = e->cfg.rates[i];
        w.x = std::max(w.x, (int64_t)C * len);
        for (int u = 0; u < 3; ++u) {
            const ConvLayer& k7 = e->unit_conv[(i * 3 + u) * 2];
            const ConvLayer& k1 = e->unit_conv[(i * 3 + u) * 2 + 1];
            w.p = std::max({w.p, enc_snake_item_floats(e, k7, len), enc_snake_item_floats(e, k1, len)});
            part(k7, len);
            part(k1, len);
        }
        w.p = std::max(w.p, enc_snake_item_floats(e, e->down[i], len / s + 1));
        part(e->down[i], len / s);
        len /= s;
        w.x = std::max(w.x, (int64_t)2 * C * len);
    }
    w.p = std::max(w.p, enc_snake_item_floats(e, e->conv_out, len));
    part(e->conv_out, len);
    w.r = w.x;
    if (pre) {
        // hidden -> R; its split form -> P; q/k/v -> X; the heads' outputs -> R
        const int64_t D = e->cfg.latent_dim;
        w.x = std::max(w.x, 3 * D * frames);
        w.r = std::max(w.r, D * frames);
        w.p = std::max(w.p, enc_snake_item_floats(e, e->qkv, frames));
        part(e->qkv, frames);
    }
    w.x = round_up(w.x * batch, 64);
    w.r = round_up(w.r * batch, 64);
    w.p = round_up(w.p * batch, 64);
    w.partial = round_up(w.partial, 64);
    return w;
}

int enc_check_args(const mh3a_encoder* e, int64_t batch, int64_t samples, uint32_t flags) {
    if (!e) return fail(MH3A_E_INVALID_ARG, "encoder is null");
    if (batch < 1 || batch > 4096) return fail(MH3A_E_INVALID_ARG, "batch must be in [1, 4096]");
    if (samples < 1) return fail(MH3A_E_INVALID_ARG, "samples must be >= 1");
    if (flags & ~MH3A_FLAG_BATCH_INVARIANT)
        return fail(MH3A_E_INVALID_ARG, "unsupported encode flags 0x%x", flags & ~MH3A_FLAG_BATCH_INVARIANT);
    const int64_t len = enc_frames(e, samples) * e->hop;
    // per-item tensors are addressed with 32-bit offsets in the kernels
    if (len > ((int64_t)1 << 30) || (int64_t)e->cfg.encoder_dim * 3 * (len + 2 * kPkPadR) >= ((int64_t)1 << 29))
        return fail(MH3A_E_INVALID_ARG, "samples too large for one item: %lld", (long long)samples);
    return MH3A_OK;
}

size_t enc_ws_bytes(const mh3a_encoder* e, int64_t batch, int64_t samples, uint32_t flags, bool pre = false) {
    const EncWs w = enc_ws_floats(e, batch, enc_frames(e, samples), (flags & MH3A_FLAG_BATCH_INVARIANT) != 0, pre);
    return (size_t)(w.x + w.r + w.p + w.partial) * sizeof(float);
}

// Snake of x (batch, c, l) rows into the input form of conv L (space-to-depth
// by s with shift p; l_out output positions).
hipError_t enc_run_snake(const mh3a_encoder* e, const SnakeLayer& S, const ConvLayer& L, const float* x, int l,
                         int s, int shift, int l_out, float* y, int batch, hipStream_t st) {
    SnakeArgs a;
    a.x = x;
    a.x_bstride = (int64_t)S.c * l;
    a.c = S.c;
    a.l = l;
    a.ab = reinterpret_cast<const float2*>(e->blob + S.ab_off);
    a.s = s;
    a.shift = shift;
    a.l_out = l_out;
    a.y = y;
    a.y_bstride = enc_snake_item_floats(e, L, l_out);
    a.lp = enc_bx6(e, L) ? (int)pk_lp(l_out) : 0;
    a.pieces = enc_h16(e, L) ? kPiecesH : kPieces;
    TimedLaunch tl(e, st, KIND_ENC_SNAKE);
    hipError_t err = launch_snake(a, batch, st);
    const double n_in = (double)batch * S.c * l, n_out = (double)batch * S.c * s * l_out;
    tl.done(KIND_ENC_SNAKE, 4.0 * n_in, 4.0 * n_in + (a.lp ? 2.0 * a.pieces : 4.0) * n_out);
    return err;
}

// conv L over its Snake input y (as enc_run_snake wrote it, l_in positions)
hipError_t enc_run_conv(const mh3a_encoder* e, const ConvLayer& L, const float* p, int l_in, int positions,
                        float* out, int batch, const float* res, bool inv, float* partial, hipStream_t st) {
    const bool bx6 = enc_bx6(e, L);
    return run_conv(e, L, p, enc_snake_item_floats(e, L, l_in), l_in, positions, out, (int64_t)L.c_out * positions,
                    batch, res, nullptr, 1.0f, false, inv, true, partial, st, bx6 ? (int)pk_lp(l_in) : 0, bx6,
                    enc_h16(e, L));
}

// hidden != null: the convolution stack into `hidden`; mean != null: the
// whole encode (stack, attention projection, mean_proj) into `mean`, the
// hidden state staying in the workspace.
int run_encode(mh3a_encoder* e, const float* wave, int64_t batch, int64_t samples, float* hidden, float* mean,
               void* ws, size_t ws_bytes, uint32_t flags, hipStream_t st) {
    int rc = enc_check_args(e, batch, samples, flags);
    if (rc) return rc;
    const bool pre = mean != nullptr;
    if (!wave || !(hidden || mean)) return fail(MH3A_E_INVALID_ARG, "null wave or output pointer");
    if (pre && !e->has_pre)
        return fail(MH3A_E_MISSING_TENSOR, "the encoder was built without the attention projection "
                    "(pre_block.attn.qkv.weight and the tensors that go with it)");
    if (!ws) return fail(MH3A_E_WORKSPACE, "workspace is null");
    if ((uintptr_t)ws % 256) return fail(MH3A_E_WORKSPACE, "workspace must be 256-byte aligned");
    const bool inv = (flags & MH3A_FLAG_BATCH_INVARIANT) != 0;
    const size_t need = enc_ws_bytes(e, batch, samples, flags, pre);
    if (ws_bytes < need) return fail(MH3A_E_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    const int64_t frames = enc_frames(e, samples);
    const EncWs w = enc_ws_floats(e, batch, frames, inv, pre);
    float* bufX = static_cast<float*>(ws);
    float* bufR = bufX + w.x;
    float* bufP = bufR + w.r;
    float* partial = bufP + w.p;
    const int B = (int)batch;
    HIP_TRY(hipSetDevice(e->device));

    int len = (int)(frames * e->hop);
    // first conv straight from the waveform: samples past S read as zeros,
    // which is the right pad to a whole number of hops
    HIP_TRY(run_conv(e, e->conv_in, wave, samples, (int)samples, len, bufX, (int64_t)e->cfg.encoder_dim * len, B,
                     nullptr, nullptr, 1.0f, false, inv, true, partial, st));
    size_t si = 0;
    for (int i = 0; i < e->cfg.num_blocks; ++i) {
        const int C = e->block_c[i], s = e->cfg.rates[i];
        for (int u = 0; u < 3; ++u) {
            const ConvLayer& k7 = e->unit_conv[(i * 3 + u) * 2];
            const ConvLayer& k1 = e->unit_conv[(i * 3 + u) * 2 + 1];
            HIP_TRY(enc_run_snake(e, e->snakes[si++], k7, bufX, len, 1, 0, len, bufP, B, st));
            HIP_TRY(enc_run_conv(e, k7, bufP, len, len, bufR, B, nullptr, inv, partial, st));
            HIP_TRY(enc_run_snake(e, e->snakes[si++], k1, bufR, len, 1, 0, len, bufP, B, st));
            // residual add in place: each output element is read and written by one thread
            HIP_TRY(enc_run_conv(e, k1, bufP, len, len, bufX, B, bufX, inv, partial, st));
        }
        const int lout = len / s;
        HIP_TRY(enc_run_snake(e, e->snakes[si++], e->down[i], bufX, len, s, (s + 1) / 2, lout + 1, bufP, B, st));
        (void)C;
        HIP_TRY(enc_run_conv(e, e->down[i], bufP, lout + 1, lout, bufX, B, nullptr, inv, partial, st));
        len = lout;
    }
    HIP_TRY(enc_run_snake(e, e->snakes[si++], e->conv_out, bufX, len, 1, 0, len, bufP, B, st));
    float* hid = pre ? bufR : hidden;
    HIP_TRY(enc_run_conv(e, e->conv_out, bufP, len, len, hid, B, nullptr, inv, partial, st));
    if (!pre) return ok();

    // attention projection: q/k/v (pointwise conv) -> X, heads -> R, then the tail -> mean
    const int D = e->cfg.latent_dim, F = (int)frames;
    const ConvLayer& Q = e->qkv;
    if (enc_bx6(e, Q)) {
        ActArgs sa;
        std::memset(&sa, 0, sizeof sa);
        sa.x = hid;
        sa.x_bstride = (int64_t)D * F;
        sa.y = bufP;
        sa.y_bstride = enc_snake_item_floats(e, Q, F);
        sa.c = D;
        sa.l = F;
        sa.lp = (int)pk_lp(F);
        sa.pieces = enc_h16(e, Q) ? kPiecesH : kPieces;
        TimedLaunch tl(e, st, KIND_ENC_SNAKE);
        HIP_TRY(launch_split(sa, B, st));
        tl.done(KIND_ENC_SNAKE, 0.0, (4.0 + 2.0 * sa.pieces) * B * (double)D * F);
        HIP_TRY(enc_run_conv(e, Q, bufP, F, F, bufX, B, nullptr, inv, partial, st));
    } else {
        HIP_TRY(run_conv(e, Q, hid, (int64_t)D * F, F, F, bufX, 3 * (int64_t)D * F, B, nullptr, nullptr, 1.0f, false,
                         inv, true, partial, st));
    }
    AttnArgs aa;
    aa.qkv = bufX;
    aa.qkv_bstride = 3 * (int64_t)D * F;
    aa.o = bufR;
    aa.o_bstride = (int64_t)D * F;
    aa.n = F;
    aa.dim = D;
    aa.heads = e->cfg.num_attention_heads;
    aa.hd = e->pre_hd;
    aa.inv_sqrt_hd = (float)(1.0 / std::sqrt((double)e->pre_hd));
    {
        TimedLaunch tl(e, st, KIND_ENC_ATTN);
        HIP_TRY(launch_attention(aa, B, st));
        // q.k and p.v over the causal triangle
        tl.done(KIND_ENC_ATTN, 4.0 * B * (double)D * F * (F + 1) / 2.0, 4.0 * B * (double)D * F * 4.0);
    }
    const int C = e->cfg.latent_channels;
    PreTailArgs ta;
    ta.o = bufR;
    ta.o_bstride = (int64_t)D * F;
    ta.n = F;
    ta.heads = e->cfg.num_attention_heads;
    ta.hd = e->pre_hd;
    ta.c = C;
    ta.f = e->pre_f;
    ta.lc = C;
    ta.wf = e->blob + e->wf_off;
    ta.bf = e->blob + e->bf_off;
    ta.w1 = e->blob + e->w1_off;
    ta.b1 = e->blob + e->b1_off;
    ta.w2 = e->blob + e->w2_off;
    ta.b2 = e->blob + e->b2_off;
    ta.wm = e->blob + e->wm_off;
    ta.bm = e->blob + e->bm_off;
    ta.y = mean;
    ta.y_bstride = (int64_t)C * F;
    TimedLaunch tl(e, st, KIND_ENC_TAIL);
    HIP_TRY(launch_pre_tail(ta, B, st));
    tl.done(KIND_ENC_TAIL, 2.0 * B * (double)F * (D + (double)C * e->pre_hd + 3.0 * C * e->pre_f + (double)C * C),
            4.0 * B * (double)F * (D + C));
    return ok();
}

}  // namespace

extern "C" {

void mh3a_encoder_config_default(mh3a_encoder_config* c) {
    if (!c) return;
    std::memset(c, 0, sizeof *c);
    c->encoder_dim = 64;
    c->num_blocks = 5;
    const int rates[5] = {2, 4, 4, 5, 5};
    for (int i = 0; i < 5; ++i) c->rates[i] = rates[i];
    c->latent_dim = 2048;
    c->latent_channels = 32;
    c->num_attention_heads = 8;
    c->matrix_form = MH3A_MATRIX_SPLIT_F16;
}

int mh3a_encoder_create(const mh3a_encoder_config* cfg, const mh3a_tensor* params, int n_params, int device,
                        mh3a_encoder** out) {
    if (!out) return fail(MH3A_E_INVALID_ARG, "out is null");
    *out = nullptr;
    if (!cfg) return fail(MH3A_E_INVALID_ARG, "config is null");
    if (n_params < 0 || (n_params > 0 && !params)) return fail(MH3A_E_INVALID_ARG, "bad parameter list");
    if (device < 0) return fail(MH3A_E_INVALID_ARG, "device must be >= 0");
    int rc = enc_check_config(cfg);
    if (rc) return rc;
    Table t;
    if ((rc = build_table(params, n_params, t))) return rc;

    mh3a_encoder* e = new (std::nothrow) mh3a_encoder();
    if (!e) return fail(MH3A_E_NOMEM, "out of host memory");
    std::unique_ptr<mh3a_encoder> guard(e);
    e->cfg = *cfg;
    e->device = device;
    Blob blob;
    int dim = cfg->encoder_dim;
    if ((rc = enc_conv(blob, t, "encoder.block.0", e->conv_in, dim, 1, 7, 1, 3, KIND_ENC_CONV, cfg->matrix_form)))
        return rc;
    e->hop = 1;
    for (int i = 0; i < cfg->num_blocks; ++i) {
        const std::string pre = "encoder.block." + std::to_string(i + 1);
        const int s = cfg->rates[i];
        e->block_c.push_back(dim);
        e->hop *= s;
        for (int u = 0; u < 3; ++u) {
            const std::string q = pre + ".block." + std::to_string(u);
            ConvLayer k7, k1;
            const int d = kEncDils[u];
            if ((rc = enc_snake_layer(blob, t, q + ".block.0.alpha", dim, e->snakes))) return rc;
            if ((rc = enc_conv(blob, t, q + ".block.1", k7, dim, dim, 7, d, 3 * d, KIND_ENC_UNIT_CONV,
                               cfg->matrix_form)))
                return rc;
            if ((rc = enc_snake_layer(blob, t, q + ".block.2.alpha", dim, e->snakes))) return rc;
            if ((rc = enc_conv(blob, t, q + ".block.3", k1, dim, dim, 1, 1, 0, KIND_ENC_CONV, cfg->matrix_form)))
                return rc;
            e->unit_conv.push_back(k7);
            e->unit_conv.push_back(k1);
        }
        if ((rc = enc_snake_layer(blob, t, pre + ".block.3.alpha", dim, e->snakes))) return rc;
        // strided conv (2 dim, dim, 2 s) regrouped as (2 dim, dim s, 2): [o][c s + r][j] = w[o][c][j s + r]
        std::vector<float> w;
        const float* bias = nullptr;
        const std::string dp = pre + ".block.4";
        if ((rc = fetch_weight(t, dp, 2 * dim, dim, 2 * s, w))) return rc;
        if ((rc = fetch_vector(t, dp + ".bias", 2 * dim, &bias))) return rc;
        std::vector<float> w2((size_t)2 * dim * dim * s * 2);
        for (int o = 0; o < 2 * dim; ++o)
            for (int c = 0; c < dim; ++c)
                for (int r = 0; r < s; ++r)
                    for (int j = 0; j < 2; ++j)
                        w2[(((size_t)o * dim + c) * s + r) * 2 + j] = w[((size_t)o * dim + c) * 2 * s + j * s + r];
        ConvLayer D;
        add_conv(blob, D, w2, bias, 2 * dim, dim * s, 2);
        D.alg_taps = 2;
        D.kind = KIND_ENC_CONV;
        if (enc_split_ok(D)) enc_pack_split(blob, D, w2, 2 * dim, dim * s, 2, cfg->matrix_form);
        e->down.push_back(D);
        dim *= 2;
    }
    const std::string fin = "encoder.block." + std::to_string(cfg->num_blocks + 1);
    if ((rc = enc_snake_layer(blob, t, fin + ".alpha", dim, e->snakes))) return rc;
    if ((rc = enc_conv(blob, t, "encoder.block." + std::to_string(cfg->num_blocks + 2), e->conv_out, cfg->latent_dim,
                       dim, 3, 1, 1, KIND_ENC_CONV, cfg->matrix_form)))
        return rc;
    if (t.get("pre_block.attn.qkv.weight") && (rc = enc_pre_block(blob, t, e))) return rc;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(MH3A_E_HIP, "no HIP device available");
    if (device >= ndev) return fail(MH3A_E_INVALID_ARG, "device %d out of range (%d devices)", device, ndev);
    HIP_TRY(hipSetDevice(device));
    HIP_TRY(hipDeviceGetAttribute(&e->num_cus, hipDeviceAttributeMultiprocessorCount, device));
    e->num_cus = std::max(1, e->num_cus);
    e->blob_floats = (int64_t)blob.h.size();
    HIP_TRY(hipMalloc((void**)&e->blob, sizeof(float) * blob.h.size()));
    HIP_TRY(hipMemcpy(e->blob, blob.h.data(), sizeof(float) * blob.h.size(), hipMemcpyHostToDevice));
    *out = guard.release();
    return ok();
}

void mh3a_encoder_destroy(mh3a_encoder* e) {
    if (!e) return;
    if (e->blob) {
        hipSetDevice(e->device);
        hipDeviceSynchronize();
        hipFree(e->blob);
        for (hipEvent_t ev : e->timing.evs) hipEventDestroy(ev);
    }
    delete e;
}

int mh3a_encode_frames(const mh3a_encoder* e, int64_t samples, int64_t* frames) {
    if (!e || !frames) return fail(MH3A_E_INVALID_ARG, "null argument");
    if (samples < 1) return fail(MH3A_E_INVALID_ARG, "samples must be >= 1");
    *frames = enc_frames(e, samples);
    return ok();
}

int mh3a_encode_workspace_size(const mh3a_encoder* e, int64_t batch, int64_t samples, uint32_t flags, size_t* bytes) {
    if (!bytes) return fail(MH3A_E_INVALID_ARG, "bytes is null");
    *bytes = 0;
    int rc = enc_check_args(e, batch, samples, flags);
    if (rc) return rc;
    *bytes = enc_ws_bytes(e, batch, samples, flags);
    return ok();
}

int mh3a_encode_hidden(mh3a_encoder* e, const float* wave, int64_t batch, int64_t samples, float* hidden,
                       void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!hidden) return fail(MH3A_E_INVALID_ARG, "hidden is null");
    return run_encode(e, wave, batch, samples, hidden, nullptr, workspace, workspace_bytes, flags,
                      static_cast<hipStream_t>(stream));
}

int mh3a_encode_mean_workspace_size(const mh3a_encoder* e, int64_t batch, int64_t samples, uint32_t flags,
                                    size_t* bytes) {
    if (!bytes) return fail(MH3A_E_INVALID_ARG, "bytes is null");
    *bytes = 0;
    int rc = enc_check_args(e, batch, samples, flags);
    if (rc) return rc;
    if (!e->has_pre) return fail(MH3A_E_MISSING_TENSOR, "the encoder was built without the attention projection");
    *bytes = enc_ws_bytes(e, batch, samples, flags, true);
    return ok();
}

int mh3a_encode_mean(mh3a_encoder* e, const float* wave, int64_t batch, int64_t samples, float* mean,
                     void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!mean) return fail(MH3A_E_INVALID_ARG, "mean is null");
    return run_encode(e, wave, batch, samples, nullptr, mean, workspace, workspace_bytes, flags,
                      static_cast<hipStream_t>(stream));
}

int mh3a_encoder_timing_enable(mh3a_encoder* e, int enable) { return timing_enable(e, enable); }
int mh3a_encoder_timing_read(mh3a_encoder* e, mh3a_kernel_stats* stats, int max_stats, int* n_stats) {
    return timing_read(e, stats, max_stats, n_stats);
}

}  // extern "C"
