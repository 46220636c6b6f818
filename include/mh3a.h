/*
 * mh3a -- MiniMax-H3 audio-VAE BigVGAN decoder on AMD MI355X (gfx950).
 *
 * C ABI of the decode path: de-normalized latents (B, latent_channels, N)
 * in, mono waveform (B, 1, hop * N) out, clamped to [-1, 1].
 *
 * Sources of what is computed (the decode contract and its layers):
 *   diffusers docs "AutoencoderKLMiniMaxH3Audio", section "decode": latents
 *     [batch, latent_channels, num_frames] -> waveform [batch, 1,
 *     num_frames * 800] clamped to [-1, 1]; stereo is two batch items.
 *   same page, class signature: the constructor defaults that
 *     mh3a_config_default() reproduces.
 *   FastVideo API docs "minimax_h3_audio_vae", MLXMiniMaxH3AudioVAE.decode:
 *     dec_in_proj (1x1) -> weight-normalized conv_pre (pad 3) -> per stage a
 *     weight-normalized ConvTranspose1d (stride r, padding (k - r) // 2) and
 *     the average of the AMP residual blocks -> activation_post ->
 *     weight-normalized conv_post (pad 3, optional bias) -> clip to [-1, 1].
 *   same page, module overview: AMP blocks with SnakeBeta behind alias-free
 *     Kaiser-window 2x up/down sampling; kaiser_sinc_filter1d designs the
 *     low-pass (released filter buffers take precedence when present).
 *   same page, mlx_h3_audio_vae_from_file: missing required tensors are an
 *     error (dec_in_proj.weight, decoder.conv_pre.weight_v,
 *     decoder.conv_post.weight_v).
 *
 * Conventions
 *   - All tensors are float32, C-contiguous, time fastest: (B, C, L).
 *   - Host pointers are read only during the call that receives them.
 *   - Device pointers are borrowed: the library never frees them.
 *   - Every entry point returns MH3A_OK (0) or a negative MH3A_E_* code and
 *     then sets a thread-local message readable with mh3a_last_error().
 *   - Argument, shape and configuration checks all run before the first
 *     HIP call, so they behave the same on a machine without a GPU.
 *   - mh3a_decode and the other device entry points only enqueue work on
 *     the given stream (hipStream_t passed as void*, NULL = the null
 *     stream); they never synchronize. A device fault surfaces at the
 *     caller's next synchronization of that stream.
 */
#ifndef MH3A_H_
#define MH3A_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MH3A_OK 0
#define MH3A_E_INVALID_ARG (-1)    /* null pointer, bad size, unknown flag     */
#define MH3A_E_MISSING_TENSOR (-2) /* a required parameter is absent           */
#define MH3A_E_SHAPE (-3)          /* a parameter has the wrong shape          */
#define MH3A_E_CONFIG (-4)         /* inconsistent architecture configuration  */
#define MH3A_E_WORKSPACE (-5)      /* workspace too small or misaligned        */
#define MH3A_E_HIP (-6)            /* a HIP runtime call failed                */
#define MH3A_E_NOMEM (-7)          /* host allocation failed                   */

/* ---- decode flags ---- */
/* Apply z * latents_std[c] + latents_mean[c] before dec_in_proj (the
 * per-channel convention of the diffusers "AutoencoderKLMiniMaxH3" page).
 * The affine map is folded into dec_in_proj at create time. */
#define MH3A_FLAG_DENORMALIZE 0x1u
/* Feed the AMP convs to the matrix cores as bfloat16 operands, each fp32
 * operand split into a bf16 head and a bf16 tail, summing head*head +
 * tail*head + head*tail with fp32 accumulation; storage stays fp32. */
#define MH3A_FLAG_BF16_MFMA 0x2u
/* Skip the final clamp (a test hook: most samples saturate under random
 * weights, so the unclamped signal is the sharper comparison). */
#define MH3A_FLAG_NO_CLAMP 0x4u
/* Plan every convolution from one batch item's shape alone, so that the
 * order in which each output's terms are summed, and hence every bit of an
 * item's result, is the same whatever batch the item is decoded in. By
 * default launches with few output tiles split the contraction into ranges
 * summed by a second pass, with the number of ranges chosen for the whole
 * batch (fastest, deterministic for a given batch, but a different batch
 * size may round differently). */
#define MH3A_FLAG_BATCH_INVARIANT 0x8u
#define MH3A_FLAG_ALL 0xFu

/* ---- matrix-core form of the convolutions (mh3a_config.matrix_form,
 * mh3a_encoder_config.matrix_form), fixed at create ---- */
/* Every conv with split-product weights runs on the bf16 matrix cores,
 * each fp32 operand split into three bf16 pieces and the six products of
 * order <= 2 summed in fp32 (about 2^-27 relative per product; the
 * encoder's default). */
#define MH3A_MATRIX_SPLIT 0
/* Every conv runs on the fp32 matrix cores (v_mfma_f32_32x32x2f32 /
 * 16x16x4f32): slower, kept as a second, independent form of the products. */
#define MH3A_MATRIX_FP32 1
/* The decoder's default: the wide convs (AMP convs of 64+ channels,
 * conv_pre, the transposed convs) split each operand into two fp16 pieces,
 * v0 = fp16(v), v1 = fp16(v - v0), the weights first scaled by a power of
 * two per layer, and sum the three products w0 x0, w0 x1, w1 x0 in fp32 on
 * the fp16 matrix cores (about 2^-22 relative per product). Every value
 * those convs read must stay below 65504 in magnitude (the fp16 range);
 * MH3A_MATRIX_SPLIT has no such bound. The narrow stages' fused unit
 * kernel and the bf16 flag keep bf16 pieces. Decoder only. */
#define MH3A_MATRIX_SPLIT_F16 2

/* ---- architecture limits ---- */
#define MH3A_MAX_STAGES 8
#define MH3A_MAX_RESBLOCKS 4
#define MH3A_MAX_DILATIONS 4

typedef struct mh3a_decoder mh3a_decoder; /* opaque, immutable after create */

/* One named host parameter array (float32, C-contiguous). */
typedef struct {
    const char* name;
    const float* data;
    int ndim;
    int64_t shape[3];
} mh3a_tensor;

/* Architecture constants. Defaults: diffusers "AutoencoderKLMiniMaxH3Audio"
 * constructor (latent_channels 32, latent_dim 2048, decoder_dim 1024,
 * decoder_rates (5,5,2,2,2,2,2), decoder_kernel_sizes (9,9,4,4,4,4,4),
 * resblock_kernel_sizes (3,7,11), dilations (1,3,5) for each block, hop
 * 800); the resampler filter is 12 taps, cutoff 0.25, half-width 0.3. */
typedef struct {
    int latent_channels;
    int latent_dim;
    int decoder_dim;
    int hop_length;                 /* product of rates must equal it */
    int num_ups;
    int rates[MH3A_MAX_STAGES];
    int kernels[MH3A_MAX_STAGES];
    int num_resblocks;
    int rb_kernels[MH3A_MAX_RESBLOCKS];
    int num_dilations;
    int rb_dilations[MH3A_MAX_RESBLOCKS][MH3A_MAX_DILATIONS];
    int filter_taps;                /* only 12 is supported */
    double filter_cutoff;
    double filter_half_width;
    int matrix_form;                /* MH3A_MATRIX_SPLIT_F16 (default), _SPLIT or _FP32 */
} mh3a_config;

/* Fill *cfg with the defaults above. */
void mh3a_config_default(mh3a_config* cfg);

/*
 * Build a decoder on GPU `device` from host parameters.
 *
 * params/n_params: named arrays. Required names (C_s = decoder_dim / 2^(s+1),
 * n = 3 s + j for stage s and block j, d = dilation index, m = 0..5):
 *   dec_in_proj.weight (latent_dim, latent_channels, 1), dec_in_proj.bias
 *   decoder.conv_pre.{weight_v (decoder_dim, latent_dim, 7), weight_g
 *     (decoder_dim, 1, 1), bias}
 *   decoder.ups.{s}.0.{weight_v (2 C_s, C_s, k_s), weight_g (2 C_s, 1, 1), bias}
 *   decoder.resblocks.{n}.convs1.{d}.{weight_v (C_s, C_s, k_j), weight_g, bias}
 *   decoder.resblocks.{n}.convs2.{d}.{...same...}
 *   decoder.resblocks.{n}.activations.{m}.act.{alpha, beta} (C_s)
 *   decoder.activation_post.act.{alpha, beta} (C_6)
 *   decoder.conv_post.{weight_v (1, C_6, 7), weight_g (1, 1, 1)} [, bias (1)]
 * Every weight_v/weight_g pair may instead be given as an already folded
 * `weight`. Optional filters: `<act>.upsample.filter` and
 * `<act>.downsample.lowpass.filter` (12 taps) replace the designed
 * Kaiser-sinc low-pass for that activation. conv_post.bias is optional
 * (absent means zero). Names not listed are ignored.
 *
 * Weight norm is folded once here: w = g * v / ||v||, the norm over every
 * axis but axis 0 (C_out for conv, C_in for the transposed conv).
 *
 * latents_mean / latents_std: host arrays of latent_channels floats used by
 * MH3A_FLAG_DENORMALIZE; NULL means 0 / 1.
 *
 * On success *out owns device copies of everything; the caller may free
 * its host arrays at once. Errors: MH3A_E_INVALID_ARG, MH3A_E_CONFIG,
 * MH3A_E_MISSING_TENSOR, MH3A_E_SHAPE, MH3A_E_HIP, MH3A_E_NOMEM; *out is
 * then NULL.
 */
int mh3a_decoder_create(const mh3a_config* cfg, const mh3a_tensor* params, int n_params,
                        const float* latents_mean, const float* latents_std, int device,
                        mh3a_decoder** out);

/* Release the decoder's device memory (waits for the device first). NULL is
 * a no-op. */
void mh3a_destroy(mh3a_decoder* dec);

/* Device workspace (bytes) that mh3a_decode needs for B items of N latents.
 * Errors: MH3A_E_INVALID_ARG (null, B < 1, N < 1, unknown flags). */
int mh3a_decode_workspace_size(const mh3a_decoder* dec, int64_t batch, int64_t frames, uint32_t flags,
                               size_t* bytes);

/*
 * Decode. latents: device (B, latent_channels, N); wave: device (B, 1, hop N).
 * workspace: device buffer of at least mh3a_decode_workspace_size bytes,
 * 256-byte aligned; it holds the intermediate activations and is clobbered.
 * The call enqueues every kernel on `stream` and returns; concurrent calls
 * on one decoder need distinct workspaces. Errors: MH3A_E_INVALID_ARG,
 * MH3A_E_WORKSPACE, MH3A_E_HIP.
 */
int mh3a_decode(mh3a_decoder* dec, const float* latents, int64_t batch, int64_t frames, float* wave,
                void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * mh3a_decode with no allocation and no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc). The intermediates live in a
 * static device array of MH3A_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from module load until the process ends; its
 * address is looked up once per device by mh3a_decoder_create. The call
 * allocates nothing and enqueues the same kernels as mh3a_decode.
 *
 * The scratch is shared by every call on one GPU (every decoder on it) and
 * keeps the last call's contents; nothing in it needs to start at zero.
 * Calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race on it: order them, or use mh3a_decode.
 * Errors: MH3A_E_INVALID_ARG (as mh3a_decode), MH3A_E_WORKSPACE when the
 * decode's workspace (mh3a_decode_workspace_size) exceeds the scratch,
 * MH3A_E_HIP.
 */
#define MH3A_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int mh3a_decode_noalloc(mh3a_decoder* dec, const float* latents, int64_t batch, int64_t frames, float* wave,
                        uint32_t flags, void* stream);

/*
 * The decode, stopped after layer `upto`, with that layer's output copied
 * to `out` (device). Layer numbering follows the decode order: 0 =
 * dec_in_proj (B, latent_dim, N), 1 = conv_pre (B, decoder_dim, N), then for
 * stage s: 2 + 2 s = its transposed conv, 3 + 2 s = its averaged AMP blocks
 * (both (B, C_s, N * r_0 ... r_s)). mh3a_decode_layer_shape reports the
 * shape. Same workspace as mh3a_decode. Used for per-layer checks.
 */
int mh3a_decode_layer_shape(const mh3a_decoder* dec, int64_t frames, int upto, int64_t* channels,
                            int64_t* length);
int mh3a_decode_partial(mh3a_decoder* dec, const float* latents, int64_t batch, int64_t frames, int upto,
                        float* out, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Time-chunked decode with bounded memory. No page prints this schedule; it
 * follows from the decoder being a stack of convolutions along time
 * (diffusers "AutoencoderKLMiniMaxH3Audio" overview; FastVideo
 * "minimax_h3_audio_vae" module overview: 1x1 projection, BigVGAN
 * upsamplers and AMP blocks, final conv), so an output sample depends only
 * on latents within a finite radius of it.
 *
 * mh3a_decode_margin reports that radius as a whole number of latents M
 * (an upper bound summed over every layer's one-sided reach, plus one).
 * mh3a_decode_chunked splits the N latents into chunks of chunk_frames
 * (the last may be shorter); chunk [n0, n1) is decoded from the window
 * [n0 - M, n1 + M) cut to [0, N) and samples [hop (n0 - w0), hop (n1 - w0))
 * of the window's waveform are written to wave[:, :, hop n0 : hop n1].
 * The result equals mh3a_decode's up to fp32 rounding order (each window
 * plans its own launches); chunk_frames >= N is mh3a_decode itself.
 *
 * latents: device (B, latent_channels, N); wave: device (B, 1, hop N).
 * workspace: device, 256-byte aligned, at least
 * mh3a_decode_chunked_workspace_size bytes; that size grows with B and
 * chunk_frames + 2 M, not with N (beyond N < chunk_frames + 2 M).
 * Chunks run one after another on `stream`. Errors: MH3A_E_INVALID_ARG
 * (null, chunk_frames < 1, batch or frames out of range, unknown flags),
 * MH3A_E_WORKSPACE, MH3A_E_HIP.
 */
int mh3a_decode_margin(const mh3a_decoder* dec, int64_t* margin);
int mh3a_decode_chunked_workspace_size(const mh3a_decoder* dec, int64_t batch, int64_t frames,
                                       int64_t chunk_frames, uint32_t flags, size_t* bytes);
int mh3a_decode_chunked(mh3a_decoder* dec, const float* latents, int64_t batch, int64_t frames,
                        int64_t chunk_frames, float* wave, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/*
 * One stage's AMP set alone (FastVideo "minimax_h3_audio_vae", decode: the
 * blocks of stage s run from the same input and are averaged): x device
 * (B, C_s, L) -> y device (B, C_s, L). Flags: MH3A_FLAG_BF16_MFMA and / or
 * MH3A_FLAG_BATCH_INVARIANT.
 * Workspace from mh3a_amp_stage_workspace_size.
 */
int mh3a_amp_stage_workspace_size(const mh3a_decoder* dec, int stage, int64_t batch, int64_t length,
                                  size_t* bytes);
int mh3a_amp_stage(mh3a_decoder* dec, int stage, const float* x, int64_t batch, int64_t length, float* y,
                   void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Kernel timing (a measurement aid). While enabled (MH3A_TIMING_ALL), every
 * launch a decode makes is bracketed by HIP events on the decode's stream
 * (MH3A_TIMING_AMP_CONV: only the AMP conv launches, which keeps the events'
 * own cost off the other launches) and tagged with
 * its kernel class and the algorithmic work it does: FLOPs of the dense
 * convolution (2 * C_out * C_in * k per output position, the transposed
 * conv counted at its k taps per input sample) and compulsory HBM bytes
 * (input, output, residual / running-sum reads, weights). mh3a_timing_read
 * waits for the recorded events, returns per-class totals in recording
 * order of first use and clears them. Enabling or disabling also clears.
 * Not thread-safe: one decode stream per decoder while enabled.
 */
typedef struct {
    char name[32];
    int64_t launches;
    double ms;
    double flops;
    double bytes;
} mh3a_kernel_stats;
#define MH3A_MAX_KERNEL_KINDS 16
#define MH3A_TIMING_OFF 0
#define MH3A_TIMING_ALL 1
#define MH3A_TIMING_AMP_CONV 2
/* enable: one of MH3A_TIMING_*; other values are MH3A_E_INVALID_ARG. */
int mh3a_timing_enable(mh3a_decoder* dec, int enable);
int mh3a_timing_read(mh3a_decoder* dec, mh3a_kernel_stats* stats, int max_stats, int* n_stats);

/*
 * Encoder convolution stack: waveform (B, 1, S) -> hidden (B, latent_dim,
 * F), F = ceil(S / hop), hop = product of the rates. Source: FastVideo API
 * docs "minimax_h3_audio_vae", the source of MLXMiniMaxH3AudioVAE.encode up
 * to the hidden state that feeds its attention projection (module overview:
 * a DAC-style encoder with plain-Snake residual units):
 *   right zero pad to F * hop samples; weight-normalized conv 1 -> dim, k7,
 *   pad 3; per rate s: three residual units (dilation 1, 3, 9) of
 *   x + conv_k1(snake(conv_k7_dil(snake(x)))) (k7 padded 3 * dilation),
 *   then snake and a conv dim -> 2 dim of kernel 2 s, stride s, padding
 *   ceil(s / 2); then snake and a conv -> latent_dim of kernel 3, pad 1.
 *   snake(x) = x + sin^2(alpha x) / (alpha + 1e-9), alpha per channel.
 * The page leaves the Snake form, the strided kernel (2 s), the unit's
 * second kernel (1) and the final kernel (3) implicit; those are the
 * readings taken here.
 *
 * Parameters (i = 1 .. num_blocks, u = 0 .. 2, dim_i = encoder_dim 2^(i-1)):
 *   encoder.block.0.{weight_v (dim, 1, 7), weight_g, bias}
 *   encoder.block.{i}.block.{u}.block.{0,2}.alpha (dim_i)
 *   encoder.block.{i}.block.{u}.block.1.{weight_v (dim_i, dim_i, 7), weight_g, bias}
 *   encoder.block.{i}.block.{u}.block.3.{weight_v (dim_i, dim_i, 1), weight_g, bias}
 *   encoder.block.{i}.block.3.alpha (dim_i)
 *   encoder.block.{i}.block.4.{weight_v (2 dim_i, dim_i, 2 s_i), weight_g, bias}
 *   encoder.block.{n+1}.alpha (encoder_dim 2^n), encoder.block.{n+2}.{weight_v
 *     (latent_dim, encoder_dim 2^n, 3), weight_g, bias}
 * (a folded `weight` may replace each weight_v / weight_g pair).
 *
 * Conventions as for the decoder: fp32 C-contiguous tensors, device
 * pointers borrowed, work only enqueued on `stream`, a 256-byte aligned
 * device workspace of at least mh3a_encode_workspace_size bytes (clobbered;
 * concurrent calls need distinct workspaces). Flags: 0 or
 * MH3A_FLAG_BATCH_INVARIANT. Errors: MH3A_E_INVALID_ARG (null, sizes,
 * flags), MH3A_E_CONFIG, MH3A_E_MISSING_TENSOR, MH3A_E_SHAPE,
 * MH3A_E_WORKSPACE, MH3A_E_HIP, MH3A_E_NOMEM.
 */
#define MH3A_MAX_ENC_BLOCKS 8
typedef struct mh3a_encoder mh3a_encoder; /* opaque, immutable after create */
typedef struct {
    int encoder_dim;                  /* channels after the first conv (64) */
    int num_blocks;                   /* strided blocks (5) */
    int rates[MH3A_MAX_ENC_BLOCKS];   /* their strides (2, 4, 4, 5, 5) */
    int latent_dim;                   /* hidden channels (2048) */
    int matrix_form;                  /* MH3A_MATRIX_SPLIT_F16 (default), _SPLIT or _FP32 */
    int latent_channels;              /* posterior width: mean_proj outputs (32) */
    int num_attention_heads;          /* heads of the attention projection (8) */
} mh3a_encoder_config;
void mh3a_encoder_config_default(mh3a_encoder_config* cfg);
int mh3a_encoder_create(const mh3a_encoder_config* cfg, const mh3a_tensor* params, int n_params, int device,
                        mh3a_encoder** out);
/* NULL is a no-op; waits for the device first. */
void mh3a_encoder_destroy(mh3a_encoder* enc);
/* F = ceil(samples / hop). */
int mh3a_encode_frames(const mh3a_encoder* enc, int64_t samples, int64_t* frames);
int mh3a_encode_workspace_size(const mh3a_encoder* enc, int64_t batch, int64_t samples, uint32_t flags,
                               size_t* bytes);
/* wave: device (B, 1, samples); hidden: device (B, latent_dim, F). */
int mh3a_encode_hidden(mh3a_encoder* enc, const float* wave, int64_t batch, int64_t samples, float* hidden,
                       void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * The whole encode: waveform -> posterior mean (the mode, the only part of
 * the posterior the MiniMax-H3 pipeline consumes: diffusers
 * "AutoencoderKLMiniMaxH3Audio", section "encode"; logs_proj is not
 * evaluated). The convolution stack, then the attention projection
 * `pre_block` and `mean_proj` (FastVideo "minimax_h3_audio_vae", module
 * overview, Encoder bullet, and the source of encode; the page gives the
 * block in prose only -- these are the readings taken):
 *   tokens are the F hidden frames; q, k, v = x W^T + (b_q, 0, b_v) with
 *     W = pre_block.attn.qkv.weight (3 latent_dim, latent_dim), b_q / b_v =
 *     pre_block.attn.q_bias / v_bias (or the q and v thirds of a fused
 *     pre_block.attn.qkv.bias; absent = 0); the k bias is zero whatever is
 *     stored;
 *   H = num_attention_heads heads of hd = latent_dim / H consecutive
 *     features (hd a power of two in [8, 256]); causal softmax attention
 *     (token t attends to u <= t), scores scaled by 1 / sqrt(hd);
 *   the head outputs averaged (a vector of hd per token), then average
 *     pooled into C = latent_channels streams of hd / C consecutive
 *     features;
 *   pre_block.attn.proj.{weight (C, C), bias}; then the GeGLU MLP:
 *     pre_block.mlp.fc1.{weight (2 F, C), bias} whose first F outputs are
 *     the value and last F the gate, value * GELU(gate) (exact erf form),
 *     pre_block.mlp.fc2.{weight (C, F), bias}; no residual, no norm;
 *   mean = mean_proj.{weight (C, C, 1), bias}, a 1x1 conv.
 * The encoder has these stages when its parameters hold
 * pre_block.attn.qkv.weight (then every tensor above but the q/v biases is
 * required). mean: device (B, latent_channels, F) with F = ceil(samples /
 * hop). Workspace: mh3a_encode_mean_workspace_size bytes, 256-byte aligned.
 * Errors as mh3a_encode_hidden, and MH3A_E_MISSING_TENSOR for an encoder
 * built without the attention projection.
 */
int mh3a_encode_mean_workspace_size(const mh3a_encoder* enc, int64_t batch, int64_t samples, uint32_t flags,
                                    size_t* bytes);
int mh3a_encode_mean(mh3a_encoder* enc, const float* wave, int64_t batch, int64_t samples, float* mean,
                     void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);
/* Kernel timing as mh3a_timing_enable / mh3a_timing_read (MH3A_TIMING_AMP_CONV
 * selects the residual units' k7 convs). */
int mh3a_encoder_timing_enable(mh3a_encoder* enc, int enable);
int mh3a_encoder_timing_read(mh3a_encoder* enc, mh3a_kernel_stats* stats, int max_stats, int* n_stats);

/* Message of the calling thread's last failure ("" if none). */
const char* mh3a_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MH3A_H_ */
