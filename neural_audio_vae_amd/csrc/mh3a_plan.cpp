// Launch planning for the conv kernel: tile shape and K split per launch.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include "mh3a_internal.h"

namespace mh3a {

int64_t plan_partial_floats(const ConvShape& L, int positions, int groups, const ConvPlan& p) {
    if (p.ksplit <= 1) return 0;
    const TileShape s = tile_shape(p.tile);
    return (int64_t)p.ksplit * ((L.c_out + s.m - 1) / s.m) * ((positions + s.n - 1) / s.n) * groups * s.m * s.n;
}

namespace {

// ---------------------------------------------------------------------------
// Tile choice: a cycle model of the wave-specialized conv kernel, fitted to
// measured stage times. Per K-chunk of 8 channels a consumer wave issues
// taps * 4 * MBW * NBW fp32 MFMAs of 64 cycles; the producer waves stage
// the window (act: ~12 cycles per window position, plain copy: ~2). Wave
// tiles of at most 64 x 64 outputs leave room for two workgroups per CU,
// which hide each other's stalls (measured ~65% of MFMA peak, ~58% with
// one workgroup per CU). A launch takes ceil(workgroups / slots) rounds.
// ---------------------------------------------------------------------------
struct TileGeom {
    int mbw, nbw, wm, wn;
};

TileGeom tile_geom(TileId t) {
    switch (t) {
#define MH3A_TILE(id, mbw, nbw, wm, wn) \
    case id: return {mbw, nbw, wm, wn};
        MH3A_TILE_LIST
#undef MH3A_TILE
        default: return {1, 1, 1, 4};
    }
}

// With a K split of S ranges the launch has S times the workgroups, each
// walking nch / S chunks, plus a reduce pass over the S partial tiles.
double tile_cost(const ConvShape& L, TileId id, int positions, int groups, bool bf16, int ksplit, int num_cus) {
    const TileShape s = tile_shape(id);
    const TileGeom g = tile_geom(id);
    const bool act = L.act;
    const int nch = (L.c_in + kChunk - 1) / kChunk;
    const int W = s.n + (L.taps - 1) * L.dil;
    const double mt = (L.c_out + s.m - 1) / s.m;
    const double nt = (positions + s.n - 1) / s.n;
    const double wgs = mt * nt * groups * ksplit;
    const int occ = (g.mbw * g.nbw <= 4) ? 2 : 1;
    const double rounds = std::ceil(wgs / ((double)num_cus * occ));
    const double shared = std::min<double>(occ, std::ceil(wgs / num_cus));  // workgroups sharing a CU
    const double eff = occ == 2 ? 0.65 : 0.58;
    const double t_cons = (double)L.taps * 4 * g.mbw * g.nbw * 64 * (act && bf16 ? 3 : 1) / eff;
    const double t_prod = (act ? 12.0 : 2.0) * W + 400;
    const double t_chunk = std::max(t_cons, t_prod) + 200;
    const double t_epi = 16.0 * g.mbw * g.nbw * 40 + 2000;
    double cost = rounds * shared * ((double)(nch / ksplit) * t_chunk + t_epi);
    if (ksplit > 1) {
        // one more launch (~3 us) streaming S partials in and the output out
        const double outs = mt * s.m * nt * s.n * groups;
        cost += 8000.0 + (ksplit + 2.0) * outs * 4.0 / 1700.0;
    }
    return cost;
}

// Build-time option -DMH3A_FORCE_TILE=<index into MH3A_TILE_LIST> forces one
// tile shape for every conv launch whose LDS it fits (a tuning aid).
constexpr int forced_tile() {
#ifdef MH3A_FORCE_TILE
    return (MH3A_FORCE_TILE >= 0 && MH3A_FORCE_TILE < TILE_COUNT) ? MH3A_FORCE_TILE : -1;
#else
    return -1;
#endif
}

TileId choose_tile(const ConvShape& L, int positions, int groups, bool bf16, int ksplit, int num_cus) {
    // split products on a packed input (conv_pre, transposed convs): the
    // compile-time-tap shapes, by output width
    // fp32 transposed convs of at most 16 outputs (the two narrowest stages):
    // 32 x 256 tiles (measured 7% faster than the model's pick, 32 x 512)
    if (!L.bx6 && !L.amp && L.phases > 1 && L.c_out <= 16 && forced_tile() < 0) return TILE_32x256;
    if (L.bx6 && !L.amp && forced_tile() < 0) {
        // pointwise convs of 64-127 outputs: one row block per wave (its
        // batched epilogue; measured 18% faster on the HBM-bound 64-channel case)
        if (L.taps == 1 && L.c_out >= 64 && L.c_out < 128) return TILE_64x256R;
        // (128 x 160 tiles from 128 outputs: measured 1.3% faster on the
        // encoder than 128 x 128, even on the decoder's conv_pre and
        // transposed convs)
        return L.c_out >= 128 ? TILE_128x160R : (L.c_out >= 64 ? TILE_64x256 : TILE_32x256);
    }
    if (forced_tile() >= 0) {
        const TileShape s = tile_shape((TileId)forced_tile());
        const int W = s.n + (L.taps - 1) * L.dil;
        const int lds_floats = 2 * kChunk * W + (L.act ? kChunk * (3 * W + 32) : 0);
        if (lds_floats * 4 <= 160 * 1024) return (TileId)forced_tile();
    }
    double best = 1e300;
    TileId pick = TILE_32x256;
    const bool act = L.act;
    const int mpad = ((L.c_out + 31) / 32) * 32;
    // The act-fused AMP convs use the shapes measured fastest per width in a
    // tile sweep of every stage (one-workgroup-per-CU shapes only pay off at
    // 512 channels, where they fill the 256 CUs in one round).
    if (L.amp) {
        // split products at 128 to 256 channels: waves of 32 x 160 (a fifth
        // fewer weight fetches per product than 32 x 128 and half of 64 x 64
        // waves; measured 2% faster than 32 x 128 at 256 channels, 0.9% on the
        // whole decode at 128)
        if (L.bx6 && L.c_out >= 128 && L.c_out < 512) return TILE_128x160R;
        // (64 channels on split products: waves of 32 x 128 measured 6% faster
        // than 64 x 128 waves on that stage in the fp16 form)
        if (L.bx6 && L.c_out >= 64 && L.c_out < 128) return TILE_64x256R;
        if (L.c_out >= 512) return TILE_256x96;
        if (L.c_out >= 256) return TILE_256x64;
        if (L.c_out >= 128) return TILE_128x128;
        if (L.c_out >= 64) return TILE_64x256;
        return TILE_32x256;
    }
    for (int id = 0; id < TILE_128x128R; ++id) {
        const TileShape s = tile_shape((TileId)id);
        if (s.m > mpad && s.m > 32) continue;  // consumer waves would idle
        const int W = s.n + (L.taps - 1) * L.dil;
        const int lds_floats = 2 * kChunk * W + (act ? kChunk * (3 * W + 32) : 0);
        if (lds_floats * 4 > 160 * 1024) continue;
        const double cost = tile_cost(L, (TileId)id, positions, groups, bf16, ksplit, num_cus);
        if (cost < best) {
            best = cost;
            pick = (TileId)id;
        }
    }
    return pick;
}

// Launch plan of one conv: tile shape and K split. Splits are powers of two
// dividing the chunk count, picked by the cost model for the batch's
// geometry, or with `invariant` for one item's (groups = phases), so that
// the order in which an output's terms are summed does not depend on the
// batch size. The tile shape never changes that order. The bound on the
// partial sums keeps the workspace modest.

}  // namespace

ConvPlan plan_conv(const ConvShape& L, int positions, int batch, bool bf16, bool invariant, int num_cus,
                   int ways) {
    // AMP convs of <= 16 output channels: 16-row tiles (a 32-row block would
    // be half or three quarters padding); they never split (1-2 chunks).
    if (L.amp && L.m16 && !bf16 && !L.bx6 && forced_tile() < 0) return {TILE_16x256, 1};
    const int nch = (L.c_in + kChunk - 1) / kChunk;
    const int item_groups = invariant ? L.phases : batch * L.phases;
    // Launches that run next to ways - 1 others (the concurrent residual
    // blocks) take no K split once their tiles together cover half the
    // compute units: the split's partial sums and reduce pass then cost more
    // than the idle units they would fill (measured on B=2 x N=200).
    if (ways > 1 && !invariant) {
        const TileId t1 = choose_tile(L, positions, batch * L.phases, bf16, 1, num_cus);
        const TileShape s1 = tile_shape(t1);
        const int64_t tiles = (int64_t)((L.c_out + s1.m - 1) / s1.m) * ((positions + s1.n - 1) / s1.n) * batch *
                              L.phases;
        if (tiles * ways >= num_cus / 2) return {t1, 1};
    }
    int best_s = 1;
    double best = 1e300;
    for (int S = 1; S <= 64 && S <= nch; S *= 2) {
        if (nch % S) continue;
        if (L.bx6 && (nch / S) % bx6_cpi_max(L.taps)) continue;  // whole split-product items (<= 8 chunks)
        const TileId t = choose_tile(L, positions, item_groups, bf16, S, num_cus);
        // the batch's own tile must keep the partials bounded too
        const TileId tb = choose_tile(L, positions, batch * L.phases, bf16, S, num_cus);
        if (S > 1 && plan_partial_floats(L, positions, batch * L.phases, {tb, S}) > kMaxPartialFloats) break;
        const double c = tile_cost(L, t, positions, item_groups, bf16, S, num_cus);
        if (c < 0.97 * best) {
            best = c;
            best_s = S;
        }
    }
    return {choose_tile(L, positions, batch * L.phases, bf16, best_s, num_cus), best_s};
}

}  // namespace mh3a
