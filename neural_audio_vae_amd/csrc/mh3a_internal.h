// Internal interface between the host orchestration (mh3a_host.cpp) and the
// gfx950 kernels (mh3a_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mh3a {

// Channels of one K-chunk of the implicit GEMM: each chunk stages CI input
// channels of the (activated) input window in LDS.
constexpr int kChunk = 8;
// Resampler filter length (2x up / 2x down low-pass).
constexpr int kTaps = 12;
constexpr int kMaxPhases = 8;

// Per-activation constants on the device: 12 up taps pre-multiplied by the
// upsampler gain 2 and split by output parity, 12 down taps, then per
// channel (alpha / pi, 0.5 / beta).
struct ActParams {
    const float* taps;  // [24]: even-parity up taps (6), odd-parity up taps (6), down taps (12)
    const float2* ab;   // [C]: (alpha / pi, 0.5 / beta)
};

// One implicit-GEMM convolution launch:
//   y[b, o, out_mul * pos + out_add[ph]] =
//       scale * (bias[o] + sum_{i, j} W_ph[o, i, j] * A[b, i, pos + in_off[ph] + j * dil]
//                + res[b, o, t] + sum_in[b, o, t])
// for pos in [0, positions). A is x itself or, with act, the anti-aliased
// SnakeBeta of x; A is zero outside [0, l_in) (zero padding).
struct ConvArgs {
    const float* x;
    int64_t x_bstride;  // floats between batch items
    int c_in;
    int l_in;
    const float* w;         // packed weights (see pack_conv_weights)
    const float* w16;       // the same for 16-row tiles (see pack_conv_weights16), or null
    const float* w6;        // bf16 pieces for split products (see pack_conv_weights6), or null
    int64_t w6_phase_stride; // floats between phases' split-product weights
    int64_t w_phase_stride; // floats between phases' packed weights
    const float* bias;      // [c_out] or null
    float* y;
    int64_t y_bstride;
    int c_out;
    int positions;
    int taps;
    int dil;
    int out_mul;
    int phases;
    int groups;           // batch * phases
    int in_off[kMaxPhases];
    int out_add[kMaxPhases];
    const float* res;     // residual, y's layout, or null
    const float* sum_in;  // running block sum, y's layout, or null
    float scale;
    ActParams act;        // act.taps == null: no activation
    int bf16;             // three-term bfloat16 split of the MFMA operands
    int ksplit;           // K ranges (divides the chunk count); > 1 uses `partial`
    float* partial;       // ksplit * tiles * tile_m * tile_n floats of raw sums
    int pk_lp;            // packed input (see below): padded row length; 0 = plain rows
    int bx6;              // packed input holds bf16 pieces; products split six ways (see below)
    int h16;              // (with bx6) the two-piece fp16 form instead (see kPiecesH); w6 then
                          // holds the fp16 weight pieces scaled by wscale = 2^e
    float wscale;         // 2^e (h16), applied to the bias the sums start from
    float out_scale;      // 2^-e (h16), applied to the sums
};

// Packed activated input of an AMP conv, written by the standalone
// activation and read by the conv without any arithmetic on the way to LDS:
// per batch item [chunk of 8 channels][hi = channel & 1][lp][p = (channel & 7) >> 1]
// with lp = l + kPkPadL + kPkPadR positions, position n at index
// kPkPadL + n, zeros in the pads and in channels past c. One chunk's window
// is then two contiguous runs of 16-byte groups, already in the matrix-core
// operand order. The pads cover the conv's zero padding and the overhang of
// the last output tile: pad <= kPkPadL and tile_n - 1 + (k - 1) d - pad <= kPkPadR.
constexpr int kPkPadL = 32;
constexpr int kPkPadR = 288;

// Split-product ("bx6") form of the packed input: every value v is split
// into bf16 pieces v0 = bf16(v), v1 = bf16(v - v0), v2 = bf16(v - v0 - v1)
// (round to nearest even), so v0 + v1 + v2 equals v to about 2^-27 relative.
// Per batch item: [chunk][piece][lp][8 bf16 of the chunk's channels], the
// same padding as above. A conv then sums the six piece products of order
// <= 2 (w0 x0, w0 x1, w1 x0, w0 x2, w1 x1, w2 x0) on bf16 matrix cores with
// fp32 accumulation, which keeps fp32-level accuracy (the dropped products
// are about 2^-27 of w x).
constexpr int kPieces = 3;
// Two-piece fp16 form: v0 = fp16(v), v1 = fp16(v - v0), so v0 + v1 equals v
// to about 2^-22 relative (|v| >= 2^-3; 2^-25 absolute below), |v| < 65504.
// Per item [chunk][piece][lp][8 fp16], the padding as above. With the
// weights split the same way after scaling by 2^e (e per layer, so that the
// largest |w| 2^e lies in [2^14, 2^15): no weight piece overflows and every
// weight's second piece stays in the normal range), a conv sums the three
// products w0 x0, w0 x1, w1 x0 on fp16 matrix cores with fp32 accumulation
// and scales the sums by 2^-e; the dropped w1 x1 is about 2^-22 of w x.
constexpr int kPiecesH = 2;
// Largest dilation the split-product conv has LDS planes for.
constexpr int kBx6MaxDil = 5;
// Dilation bound of the wider-plane instances (7 taps; the encoder's units).
constexpr int kBx6WideDil = 9;
// Chunks per pipeline item of a split-product conv with output tiles nwg
// wide: eight for up to 7 taps and four for more (2 to 28 instruction pairs
// per barrier), halved until the two item buffers fit 156 KB of LDS
// (256-wide tiles). Measured against two chunks per item for
// 3+ taps: about 1% faster. The chunks of a K range must be a multiple of it.
constexpr int bx6_cpi(int nwg, int taps, int dmax = kBx6MaxDil, int planes = kPieces) {
    int c = taps <= 7 ? 8 : 4;
    while (c > 2 && 2 * c * planes * (nwg + (taps - 1) * dmax) * 16 > 156 * 1024) c /= 2;
    return c;
}
// The largest item any tile uses for a tap count (eligibility: whole items).
constexpr int bx6_cpi_max(int taps) { return bx6_cpi(32, taps, 1); }
// (A matrix-core instruction of a split-product conv takes two consecutive
// (chunk, tap) slots, which for odd tap counts may lie in two chunks; see
// pack_conv_weights6.)

// Tile shapes of the conv kernel: four consumer waves arranged WM x WN,
// each computing MBW x NBW blocks of 32 x 32 outputs.
//          id            MBW NBW WM WN     workgroup tile (M x N)
#define MH3A_TILE_LIST                                              \
    MH3A_TILE(TILE_512x64, 4, 2, 4, 1)   /* 512 x  64 */           \
    MH3A_TILE(TILE_256x128, 2, 4, 4, 1)  /* 256 x 128 */           \
    MH3A_TILE(TILE_256x96, 2, 3, 4, 1)   /* 256 x  96 */           \
    MH3A_TILE(TILE_256x64, 2, 2, 4, 1)   /* 256 x  64 */           \
    MH3A_TILE(TILE_128x96, 1, 3, 4, 1)   /* 128 x  96 */           \
    MH3A_TILE(TILE_128x256, 2, 4, 2, 2)  /* 128 x 256 */           \
    MH3A_TILE(TILE_128x128, 2, 2, 2, 2)  /* 128 x 128 */           \
    MH3A_TILE(TILE_64x512, 2, 4, 1, 4)   /*  64 x 512 */           \
    MH3A_TILE(TILE_64x256, 2, 2, 1, 4)   /*  64 x 256 */           \
    MH3A_TILE(TILE_32x512, 1, 4, 1, 4)   /*  32 x 512 */           \
    MH3A_TILE(TILE_32x256, 1, 2, 1, 4)   /*  32 x 256 */           \
    MH3A_TILE(TILE_128x128R, 1, 4, 4, 1) /* 128 x 128, waves of 32 x 128 */ \
    MH3A_TILE(TILE_64x256R, 1, 4, 2, 2)  /*  64 x 256, waves of 32 x 128 */ \
    MH3A_TILE(TILE_128x160R, 1, 5, 4, 1) /* 128 x 160, waves of 32 x 160 */
// (the tiles from TILE_128x128R on serve AMP convs only: the general
// search of the planner skips them)
enum TileId {
#define MH3A_TILE(id, mbw, nbw, wm, wn) id,
    MH3A_TILE_LIST
#undef MH3A_TILE
    TILE_COUNT,
    // 16 x 256 on v_mfma_f32_16x16x4f32 (four waves of 16 x 64): AMP convs
    // of at most 16 output channels, fp32, compile-time taps, no K split.
    // Not part of the tile model's search.
    TILE_16x256 = TILE_COUNT
};
// Tiles with instances specialized for 3, 7 and 11 taps (the shapes the AMP
// convs use, with or without the fused activation); other shapes run those
// convs with a runtime tap count.
constexpr bool tile_has_act_taps(int t) {
    return t == TILE_256x96 || t == TILE_256x64 || t == TILE_128x96 || t == TILE_128x128 || t == TILE_64x256 ||
           t == TILE_32x256 || t == TILE_128x128R || t == TILE_64x256R || t == TILE_128x160R;
}
struct TileShape {
    int m, n;
};
TileShape tile_shape(TileId t);

// Number of packed floats for a conv weight of (c_out, c_in, taps).
int64_t packed_weight_floats(int c_out, int c_in, int taps);
// Pack w (c_out, c_in, taps), row-major, into the MFMA A-operand order.
void pack_conv_weights(const float* w, int c_out, int c_in, int taps, float* out);
// The same for 16-row tiles (v_mfma_f32_16x16x4f32 A-operand order).
int64_t packed_weight_floats16(int c_out, int c_in, int taps);
void pack_conv_weights16(const float* w, int c_out, int c_in, int taps, float* out);
// The same as bf16 pieces for v_mfma_f32_32x32x16_bf16 (see pack_conv_weights6).
int64_t packed_weight_floats6(int c_out, int c_in, int taps);
void pack_conv_weights6(const float* w, int c_out, int c_in, int taps, float* out);

hipError_t launch_conv(const ConvArgs& a, TileId tile, hipStream_t stream);

// What the planner needs of a conv layer.
struct ConvShape {
    int c_in, c_out, taps, dil, phases;
    bool act;  // activation fused into the operand staging
    bool amp;  // an AMP conv (tile table measured for them)
    bool m16;  // weights packed for 16-row tiles too
    bool bx6;  // packed input in the split-product form
};
// AMP activations of at least this many (batch x channel x position)
// elements run as their own pass (see amp_act_fused in mh3a_host.cpp).
constexpr int64_t kSeparateActMin = (int64_t)1 << 12;
// Tile shape and K split of one launch.
struct ConvPlan {
    TileId tile;
    int ksplit;
};
// Bound on a plan's partial sums (floats), which live in the workspace.
constexpr int64_t kMaxPartialFloats = (int64_t)32 << 20;
// Plan one conv launch of `batch` items over `positions` output positions
// per phase on a device with num_cus compute units, running next to
// ways - 1 launches of the same kind (1: alone).
ConvPlan plan_conv(const ConvShape& s, int positions, int batch, bool bf16, bool invariant, int num_cus,
                   int ways = 1);
// Floats of partial sums the plan needs (0 without a K split).
int64_t plan_partial_floats(const ConvShape& s, int positions, int groups, const ConvPlan& p);

// The anti-aliased SnakeBeta alone: y = act(x), x (B, c, l) rows, y packed
// (lp = l + kPkPadL + kPkPadR, pads written as zeros).
struct ActArgs {
    const float* x;
    int64_t x_bstride;
    float* y;
    int64_t y_bstride;  // ceil(c / 8) * 8 * lp
    int c;
    int l;
    int lp;
    int pieces;         // 0: fp32 packed layout; kPieces: bf16 pieces; kPiecesH: fp16 pieces
    ActParams act;
};
hipError_t launch_act(const ActArgs& a, int batch, hipStream_t stream);
// The same layout without the activation: y = x in the split-product form
// (a.act unused, a.pieces kPieces or kPiecesH).
hipError_t launch_split(const ActArgs& a, int batch, hipStream_t stream);

// One AMP residual unit in one launch, for narrow stages:
//   y = scale * (x + conv2(act2(conv1(act1(x)))) + sum_in)
// conv1 has k taps at dilation dil, conv2 k taps at dilation 1, both "same"
// padded with bias; x, y and sum_in are (B, c, l) rows; y must not alias x
// (workgroups read x around their own outputs); sum_in may alias y.
// Weights in the 16-row MFMA order (pack_conv_weights16).
struct UnitArgs {
    const float* x;
    float* y;
    const float* sum_in;  // or null
    float scale;
    int64_t bstride;      // floats between batch items (c * l)
    int c, l, taps, dil;
    const float* w1;
    const float* b1;
    ActParams act1;
    const float* w2;
    const float* b2;
    ActParams act2;
    int split;            // 0: fp32 matrix cores; 6 / 3: w1, w2 in the split-product unit order
                          // (pack_unit_weights6), six / three piece products on bf16 matrix cores;
                          // 2: fp16 pieces (pack_unit_weights_h), three products on fp16 matrix cores
    float wscale1, wscale2;  // (split 2) the 2^e each conv's weights were scaled by
};
// Shapes the unit kernel has instances for: c in {8, 16, 32}, taps in
// {3, 7, 11}, 1 <= dil <= kUnitMaxDil.
constexpr int kUnitMaxDil = 5;
bool unit_supported(int c, int taps, int dil);
hipError_t launch_unit(const UnitArgs& a, int batch, hipStream_t stream);
// Unit-kernel weights as bf16 pieces for v_mfma_f32_16x16x32_bf16.
int64_t unit_weight_floats6(int c, int taps);
void pack_unit_weights6(const float* w, int c, int taps, float* out);
// ... and as fp16 pieces of w 2^e for v_mfma_f32_16x16x32_f16 (kPiecesH).
int64_t unit_weight_floats_h(int c, int taps);
void pack_unit_weights_h(const float* w, int c, int taps, int e, float* out);

// Encoder Snake: y = snake(x) regrouped space-to-depth by s (s = 1: plain):
// output channel c * s + r at position t is snake(x[c, t * s + r - shift]),
// zero outside [0, l); t in [0, l_out). lp = 0: plain (B, c * s, l_out)
// rows; lp = l_out + kPkPadL + kPkPadR: the split-product packed form.
struct SnakeArgs {
    const float* x;
    int64_t x_bstride;
    int c, l;
    const float2* ab;    // [c]: (alpha / pi, 0.5 / (alpha + 1e-9))
    int s, shift, l_out;
    float* y;
    int64_t y_bstride;
    int lp;
    int pieces;          // (lp > 0) kPieces bf16 or kPiecesH fp16 pieces per value
};
hipError_t launch_snake(const SnakeArgs& a, int batch, hipStream_t stream);

// activation_post + conv_post (c -> 1, 7 taps, pad 3) + optional clamp.
struct FinalArgs {
    const float* x;
    int64_t x_bstride;
    int c;
    int l;
    ActParams act;
    const float* w;  // [c * 7] folded conv_post weight
    float bias;
    float* y;        // (B, 1, l)
    int clamp;
};
hipError_t launch_final(const FinalArgs& a, int batch, hipStream_t stream);

// ConvTranspose1d of a narrow stage on the vector ALU (fp32 fused
// multiply-adds, the polyphase form): y (B, co, r l) = convT(x (B, ci, l)),
// stride r, kernel k, padding (k - r) / 2, with bias. Supported shapes:
// ups_vec_supported.
struct UpsVecArgs {
    const float* x;     // (B, ci, l)
    float* y;           // (B, co, r l)
    const float* w;     // [ci][co][k], the folded transposed-conv weight as stored
    const float* bias;  // [co]
    int ci, co, r, k, l;
};
bool ups_vec_supported(int ci, int co, int r, int k);
hipError_t launch_ups_vec(const UpsVecArgs& a, int batch, hipStream_t stream);

// Static device scratch of mh3a_decode_noalloc (mh3a_noalloc.hip): its size,
// the once-per-device lookup of its device address (hipGetSymbolAddress
// with the device current; called from the decoder's create) and that
// address (null before the lookup).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;  // MH3A_NOALLOC_SCRATCH_BYTES
hipError_t noalloc_scratch_lookup(int device);
void* noalloc_scratch(int device);

// Causal multi-head attention of the encoder's attention projection:
// qkv (B, 3 dim, n) channel-major rows (q, k, v thirds, head h at features
// [h hd, (h + 1) hd) of each), o (B, dim, n) the heads' outputs side by side.
struct AttnArgs {
    const float* qkv;
    int64_t qkv_bstride;
    float* o;
    int64_t o_bstride;
    int n, dim, heads, hd;  // hd = dim / heads, one of attn_head_width_ok's
    float inv_sqrt_hd;
};
// Head widths the attention kernel has instances for: 8, 16, ..., 256.
bool attn_head_width_ok(int hd);
size_t attn_lds_bytes(int hd);
hipError_t launch_attention(const AttnArgs& a, int batch, hipStream_t stream);

// The rest of the attention projection and mean_proj, per token:
//   y = wf (sum_h o_h) + bf        (wf: the output projection with the head
//                                   mean and the average pooling folded in)
//   g = (w1_v y + b1_v) * GELU(w1_g y + b1_g)
//   z = w2 g + b2;   out = wm z + bm
struct PreTailArgs {
    const float* o;
    int64_t o_bstride;
    int n, heads, hd, c, f, lc;
    const float* wf;  // [c][hd]
    const float* bf;  // [c]
    const float* w1;  // [2 f][c] (value rows, then gate rows)
    const float* b1;  // [2 f]
    const float* w2;  // [c][f]
    const float* b2;  // [c]
    const float* wm;  // [lc][c]
    const float* bm;  // [lc]
    float* y;         // (B, lc, n)
    int64_t y_bstride;
};
size_t pre_tail_lds_bytes(int hd, int c, int f);
hipError_t launch_pre_tail(const PreTailArgs& a, int batch, hipStream_t stream);

}  // namespace mh3a
