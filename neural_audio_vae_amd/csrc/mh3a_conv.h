// The persistent implicit-GEMM conv kernel (see conv_kernel below) and its
// launchers. Each tile shape is instantiated in a translation unit of its own
// (mh3a_conv_*.hip) so that the library builds in parallel.
#pragma once

#include "mh3a_device.h"
#include "mh3a_tiles.h"

namespace mh3a {

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
// matrix cores (packed input in the split-product form, see kPieces); 4 the
// two-piece fp16 form on fp16 matrix cores (three products w0 x0, w0 x1,
// w1 x0 with the weights scaled by 2^e, see kPiecesH); 3 the
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
    constexpr bool BX6 = PREC >= 2;            // bf16 / fp16 matrix cores on the pieces
    constexpr bool H16 = PREC == 4;            // fp16 pieces (two per value)
    constexpr int NPROD = PREC == 2 ? 6 : 3;   // piece products per pair
    constexpr int NPA = PREC == 2 ? kPieces : 2;  // weight / activation pieces used
    constexpr int NPL = H16 ? kPiecesH : kPieces; // planes per chunk of the packed input (and weight pieces)
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
    constexpr int CPI = BX6 ? bx6_cpi(NWG, TAPS, DMAX, NPL) : 1;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool producer = wave >= 4;
    const int W = NWG + (a.taps - 1) * a.dil;
    // one item's operand window: [CI][W] floats, or NPL planes of PS6 16-byte groups per chunk
    const int ABUF = BX6 ? CPI * NPL * PS6 * 4 : CI * W;
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
                                  0, act_xs_len(W));
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
        if constexpr (H16) {
            // the sums carry the weights' scale 2^e until the epilogue
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) bias_frag[mb] *= a.wscale;
        }
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
    typedef _Float16 v8h __attribute__((ext_vector_type(8)));
    const int G6 = nch * (TAPS > 0 ? TAPS : 1) / 2;  // weight groups (slot pairs) per 32-row block
    constexpr int NAW = BX6 ? NPL : 1;  // weight pieces per slot pair in the packing
    // weight ring: slot u % RING holds pair u, loaded RING - 1 pairs ahead
    // (at most an item's pairs ahead)
    constexpr int NPI6 = BX6 ? CPI * (TAPS > 0 ? TAPS : 1) / 2 : 2;
    // (three slots for the six-product form: its three weight pieces per
    // slot leave no registers for more)
    constexpr int RING_W = PREC == 2 ? 3 : kWeightRing;
    constexpr int RING = RING_W < NPI6 + 1 ? RING_W : NPI6 + 1;
    v4u A6r[RING][NAW][MBW];
    auto load_a6 = [&](v4u (&dst)[NAW][MBW], int mb_base, int ph, int g) {
        const v4u* wp = reinterpret_cast<const v4u*>(a.w6 + (int64_t)ph * a.w6_phase_stride) + (int64_t)g * NAW * 64 + lane;
#pragma unroll
        for (int p = 0; p < (BX6 ? NPA : 1); ++p)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                dst[p][mb] = wp[((int64_t)min(mb_base + mb, mb_tot - 1) * G6 * NAW + p) * 64];
    };
    // the six products of order <= 2 (the first three for PREC 3): (A piece, B piece),
    // measured 1-2% faster in this order
    auto mfma6 = [&](const v4u (&A)[NAW][MBW], const v4u (&B)[NAW][NBW]) {
        // by activation piece, so that only piece 0's LDS reads gate the first
        // products (PREC 3 and 4: the first three entries)
        constexpr int TA[6] = {0, 1, 0, 2, 1, 0}, TB[6] = {0, 0, 1, 0, 1, 2};
#pragma unroll
        for (int t = 0; t < NPROD; ++t)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    if constexpr (H16)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(v8h, A[TA[t]][mb]), __builtin_bit_cast(v8h, B[TB[t]][nb]), acc[mb][nb],
                            0, 0, 0);
                    else
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(v8bf, A[BX6 ? TA[t] : 0][mb]),
                            __builtin_bit_cast(v8bf, B[BX6 ? TB[t] : 0][nb]), acc[mb][nb], 0, 0, 0);
                }
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
            // (split products: the pieces' planes per chunk instead of two parities)
            constexpr int NPLI = BX6 ? NPL : 2;
            const int DS = BX6 ? PS6 : W;    // LDS plane stride (positions)
            const int pw = wave - 4;
            const int segs = (W + 63) >> 6;  // 64-position segments per plane
            // item c of tile t: chunks t.c0 + CPI c + cc, planes one after another
            auto dma = [&](const Tile& t, int c, float* dst) {
                const float* src = a.x + (int64_t)t.b * a.x_bstride +
                                   ((int64_t)(t.c0 + CPI * c) * NPLI * a.pk_lp + kPkPadL + t.n_lo) * 4;
                for (int q = pw; q < CPI * NPLI * segs; q += 4) {
                    const int hp = q / segs;  // plane within the item (chunk cc = hp / NPLI)
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
#pragma unroll
        for (int i = 0; i < RING - 1; ++i) load_a6(A6r[i], mb0, cur.ph, g0 + i);
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
            static_assert((CPI * TAPS) % 2 == 0 && NPI >= RING - 1, "whole slot pairs; the ring's lead within an item");
            const int q0 = (cur.c0 + CPI * cur_c) * TAPS / 2;
            const int nq0 = has_next ? (nxt.c0 + CPI * nxt_c) * TAPS / 2 : q0;
            const int nmb = has_next ? nmb_base : mb_base;
            const int nph6 = has_next ? nxt.ph : cur.ph;
            const float* bb_0 = cur_buf + colbase * 4;
            // B operand of pair u, piece p: one 16-byte LDS read per block
            auto read_b6 = [&](v4u (&dst)[NBW], int u, int p) {
                const int s0 = 2 * u, s1 = 2 * u + 1;
                const int off0 = (s0 / TAPS) * NPL * PS6 + (s0 % TAPS) * a.dil;
                const int off1 = (s1 / TAPS) * NPL * PS6 + (s1 % TAPS) * a.dil;
                const float* bq = bb_0 + (hi ? off1 : off0) * 4 + p * PS6 * 4;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) dst[nb] = *reinterpret_cast<const v4u*>(bq + nb * 32 * 4);
            };
            // the products (A piece ta) x (B piece of Bp) of every block
            auto mfma_piece = [&](const v4u (&A)[NAW][MBW], int ta, const v4u (&Bp)[NBW]) {
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        if constexpr (H16)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                __builtin_bit_cast(v8h, A[ta][mb]), __builtin_bit_cast(v8h, Bp[nb]), acc[mb][nb], 0, 0, 0);
                        else
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(v8bf, A[ta][mb]), __builtin_bit_cast(v8bf, Bp[nb]), acc[mb][nb], 0, 0, 0);
                    }
            };
            if constexpr (NPROD == 3) {
                // Three products (w0 x0, w1 x0, w0 x1): the LDS reads of pair
                // u + 1 go out behind pair u's products, piece 0 once
                // w0 x0 and w1 x0 have taken it, piece 1 once w0 x1 has, so
                // that only the item's first pair waits on LDS latency (and
                // no register is added). Slots 0 and 1 of the weight ring
                // hold pairs 0 and 1 on entry; pair u + 2 (or the next item's
                // pair u + 2 - NPI) loads while pair u multiplies.
                v4u B0[NBW], B1[NBW];
                read_b6(B0, 0, 0);
                read_b6(B1, 0, 1);
#pragma unroll
                for (int u = 0; u < NPI; ++u) {
                    v4u(&use)[NAW][MBW] = A6r[u % RING];
                    constexpr int LEAD = RING - 1;
                    if (u + LEAD < NPI) {
                        load_a6(A6r[(u + LEAD) % RING], mb_base, cur.ph, q0 + u + LEAD);
                    } else {
                        load_a6(A6r[(u + LEAD) % RING], nmb, nph6, nq0 + (u + LEAD - NPI));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_piece(use, 0, B0);
                    mfma_piece(use, 1, B0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (u + 1 < NPI) read_b6(B0, u + 1, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma_piece(use, 0, B1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (u + 1 < NPI) read_b6(B1, u + 1, 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // six products: pair u's reads go out right before its products
#pragma unroll
                for (int u = 0; u < NPI; ++u) {
                    v4u(&use)[NAW][MBW] = A6r[u % RING];
                    constexpr int LEAD = RING - 1;
                    if (u + LEAD < NPI) {
                        load_a6(A6r[(u + LEAD) % RING], mb_base, cur.ph, q0 + u + LEAD);
                    } else {
                        load_a6(A6r[(u + LEAD) % RING], nmb, nph6, nq0 + (u + LEAD - NPI));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    v4u Bv[NAW][NBW];
#pragma unroll
                    for (int p = 0; p < NPA; ++p) read_b6(Bv[p], u, p);
                    __builtin_amdgcn_sched_barrier(0);
                    mfma6(use, Bv);
                }
            }
            // the next item's pairs 0 .. RING - 2 sit in slots (NPI + i) % RING:
            // rotate them to slots i
            if constexpr (NPI % RING != 0) {
                v4u rot[RING][NAW][MBW];
#pragma unroll
                for (int i = 0; i < RING; ++i)
#pragma unroll
                    for (int p = 0; p < NAW; ++p)
#pragma unroll
                        for (int mb = 0; mb < MBW; ++mb) rot[i][p][mb] = A6r[(i + NPI) % RING][p][mb];
#pragma unroll
                for (int i = 0; i < RING; ++i)
#pragma unroll
                    for (int p = 0; p < NAW; ++p)
#pragma unroll
                        for (int mb = 0; mb < MBW; ++mb) A6r[i][p][mb] = rot[i][p][mb];
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
            if constexpr (H16) {
                // the sums carry 2^e (the weights' scale): back to the output's scale (exact)
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[mb][nb][r] *= a.out_scale;
            }
            // Whole tiles (every row and column inside the output, no K
            // split) take the buffer-instruction epilogue: one buffer
            // resource per array over the batch item's slice, the lane's
            // column in the vector offset and each register's row and block
            // in the scalar offset, so no output costs an address computation
            // or an exec-mask branch. Block k + 1's residual and running-sum
            // loads go out before block k's stores (exact for in-place
            // updates: they read other outputs than block k writes).
            const bool whole = a.ksplit == 1 && (mb_base + MBW) * 32 <= a.c_out &&
                               cur.p0 + NWG <= a.positions && a.y_bstride <= kEpiMaxSlice &&
                               a.y_bstride >= (int64_t)a.c_out * a.out_mul * a.positions;
            auto epilogue_whole = [&](auto has_res, auto has_sum) {
                constexpr bool HR = decltype(has_res)::value, HS = decltype(has_sum)::value;
                constexpr int NB = MBW * NBW;
                const int64_t ybase = (int64_t)cur.b * a.y_bstride;
                const int nbytes = (int)(a.y_bstride * 4);
                const auto ry = __builtin_amdgcn_make_buffer_rsrc(a.y + ybase, (short)0, nbytes, kBufferWord3);
                const auto rr = __builtin_amdgcn_make_buffer_rsrc((void*)(HR ? a.res + ybase : a.y + ybase), (short)0,
                                                                  nbytes, kBufferWord3);
                const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(HS ? a.sum_in + ybase : a.y + ybase),
                                                                  (short)0, nbytes, kBufferWord3);
                const int ost = a.out_mul * a.positions;
                const int vlane = ((mb_base * 32 + 4 * hi) * ost + a.out_mul * (cur.p0 + colbase) + a.out_add[cur.ph]) * 4;
                auto soff = [&](int k, int r) {
                    return ((k / NBW * 32 + 8 * (r >> 2) + (r & 3)) * ost + a.out_mul * (k % NBW) * 32) * 4;
                };
                float rv[2][16], sv[2][16];
                auto load = [&](int k) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if constexpr (HR)
                            rv[k & 1][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, vlane, soff(k, r), 0));
                        if constexpr (HS)
                            sv[k & 1][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vlane, soff(k, r), 0));
                    }
                };
                if constexpr (HR || HS) load(0);
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    if constexpr (HR || HS)
                        if (k + 1 < NB) load(k + 1);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float v = acc[k / NBW][k % NBW][r];
                        if constexpr (HR) v += rv[k & 1][r];
                        if constexpr (HS) v += sv[k & 1][r];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v * a.scale), ry, vlane, soff(k, r), 0);
                    }
                }
            };
            using T_ = std::true_type;
            using F_ = std::false_type;
            if (whole) {
                if (a.res && a.sum_in) epilogue_whole(T_{}, T_{});
                else if (a.res) epilogue_whole(T_{}, F_{});
                else if (a.sum_in) epilogue_whole(F_{}, T_{});
                else epilogue_whole(F_{}, F_{});
            } else if (a.ksplit > 1) {
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
                if (a.h16) {
                    // two fp16 pieces, three products (AMP convs, conv_pre, transposed convs,
                    // the encoder's convs)
                    if (a.dil > kBx6MaxDil) {
                        // wider planes: 7 taps up to dilation kBx6WideDil (encoder units)
                        if (a.taps != 7 || a.dil > kBx6WideDil || a.bf16 ||
                            (((a.c_in + kChunk - 1) / kChunk) / a.ksplit) % bx6_cpi(NWG, 7, kBx6WideDil, kPiecesH))
                            return hipErrorInvalidValue;
                        return launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 4, 7, 32, kBx6WideDil>, a, tiles,
                                                 sizeof(float) * (size_t)conv_lds_floats6(NWG, 7, kBx6WideDil, kPiecesH),
                                                 stream);
                    }
                    if (a.bf16 || a.dil > kBx6MaxDil ||
                        (((a.c_in + kChunk - 1) / kChunk) / a.ksplit) % bx6_cpi(NWG, a.taps, kBx6MaxDil, kPiecesH))
                        return hipErrorInvalidValue;
#define MH3A_TAPSH(T)                                                                                          \
    if (a.taps == T)                                                                                          \
        return launch_persistent(conv_kernel<MBW, NBW, WM, WN, false, 4, T>, a, tiles,                        \
                                 sizeof(float) * (size_t)conv_lds_floats6(NWG, T, kBx6MaxDil, kPiecesH), stream);
                    MH3A_TAPSH(1)
                    MH3A_TAPSH(2)
                    MH3A_TAPSH(3)
                    MH3A_TAPSH(7)
                    MH3A_TAPSH(11)
#undef MH3A_TAPSH
                    return hipErrorInvalidValue;
                }
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

// The launcher of one tile shape, for its translation unit.
#define MH3A_DEFINE_TILE_LAUNCHER(ID, MBW, NBW, WM, WN)                                   \
    template <>                                                                          \
    hipError_t launch_tile_of<ID>(const ConvArgs& a, hipStream_t stream) {               \
        return launch_tile<MBW, NBW, WM, WN, tile_has_act_taps(ID)>(a, stream);          \
    }

}  // namespace mh3a
