#include "plan.hpp"

#include <algorithm>

namespace chol {

// The trailing update is deferred so that most of it contracts over DEFER
// panels at once (a product DEFER*nb deep reads and writes the trailing
// triangle once where DEFER products nb deep would each do so).  Panel j is
// L[rows below tile j, tile column j]; consecutive panels sit side by side in
// L, so a run of them is one wide operand.  The steps form groups of DEFER;
// at step k = g + j of the group starting at g (tile column k factored on the
// chain stream, its panel solved on the wide stream):
//   j = 0:  tile columns k+1 .. k+DEFER receive the DEFER panels they lack
//           (those of the previous group; panel 0 alone at k = 0), in one
//           launch;
//   j > 0:  tile columns k+1 .. g+DEFER receive panel k;
//   then the chain stream factors tile column k+1 while the wide stream
//   updates part j of DEFER of the group's far triangle (right of tile column
//   g+DEFER) with the same panels as step g; where that part is empty, the
//   wide stream factors tile column k+1 itself, after the narrow update,
//   and the two joins around the factor are left out.
// The far triangle's tiles are taken by `slots` persistent blocks, each tile
// the same long product (DEFER*nb deep), so a launch lasts a whole number of
// rounds of tiles however few tiles its last round holds.  The parts are
// therefore cut at multiples of `slots` tiles: the group's rounds are shared
// out among its DEFER launches and only one launch ends in a partly filled
// round (slots <= 0: equal parts).
// The diagonal tiles' inverses alternate between two slots: the panel solve
// of tile column k reads slot k % 2 while tile column k+1 is factored into
// the other one.
// With A apart from L, only the tile columns left of the first group's far
// triangle are copied from A into L: that triangle's tiles receive their
// first update from the first group's far-triangle parts, which read them
// from A and write them to L (copy and update in one pass).
std::vector<FwdOp> forward_plan(int64_t n, int nb, bool copy, int slots)
{
    std::vector<FwdOp> ops;
    if (n <= 0 || nb <= 0)
        return ops;
    auto op = [&](int kind, int stream) -> FwdOp & {
        ops.push_back(FwdOp{kind, stream, 0, 0, 0, 0, 0, 0, 0, -1});
        return ops.back();
    };
    const int64_t K = (n + nb - 1) / nb;
    auto diag = [&](int64_t k, int stream) {
        FwdOp &o = op(FWD_DIAG, stream);
        o.k = k;
        o.slot = (k * nb + std::min<int64_t>(nb, n - k * nb) < n) ? (int)(k & 1) : -1;
    };
    auto tri_tiles = [&](int64_t c) -> int {
        const int64_t TI = (n - c + 127) / 128;
        return (int)(TI * (TI + 1) / 2);
    };
    if (copy) {
        // columns left of the first group's far triangle (all of them when
        // the matrix has no such triangle)
        const int64_t first_far = std::min<int64_t>(nb, n) + (int64_t)FWD_DEFER * nb;
        op(FWD_COPY, FWD_CHAIN).w = first_far < n ? first_far : n;
    }
    diag(0, FWD_CHAIN);
    // the far triangle of the current group: first column, panels, tile count,
    // whether its tiles are read from A (the first group's, when copying)
    int64_t fcol = -1, ff = 0;
    int fnp = 0, ftiles = 0;
    bool ffrom_a = false;
    bool diag_wide = false;   // the last diagonal tile was factored on the wide stream
    for (int64_t k = 0; k < K; ++k) {
        const int64_t k0 = k * nb;
        const int64_t r0 = k0 + std::min<int64_t>(nb, n - k0), m = n - r0;
        if (m == 0)
            break;
        if (!diag_wide)
            op(FWD_JOIN, FWD_WIDE).slot = 0;
        {
            FwdOp &o = op(FWD_PANEL, FWD_WIDE);
            o.k = k;
            o.slot = (int)(k & 1);
        }
        const int j = (int)(k % FWD_DEFER);
        const int np = j == 0 ? (k == 0 ? 1 : FWD_DEFER) : 1;
        const int64_t f = k + 1 - np;
        {
            FwdOp &o = op(FWD_UPDATE, FWD_WIDE);
            o.c = r0;
            o.w = std::min<int64_t>((int64_t)(j == 0 ? FWD_DEFER : FWD_DEFER - j) * nb, m);
            o.f = f;
            o.np = np;
        }
        if (j == 0) {
            fcol = r0 + (int64_t)FWD_DEFER * nb;
            if (fcol < n) {
                ff = f;
                fnp = np;
                ftiles = tri_tiles(fcol);
                ffrom_a = copy && k == 0;
            } else {
                fcol = -1;
            }
        }
        int t0 = 0, t1 = 0;
        if (fcol >= 0) {
            auto cut = [&](int q) -> int {
                if (slots <= 0)
                    return (int)((int64_t)ftiles * q / FWD_DEFER);
                const int64_t rounds = ((int64_t)ftiles + slots - 1) / slots;
                return (int)std::min<int64_t>(ftiles, rounds * q / FWD_DEFER * slots);
            };
            t0 = cut(j);
            t1 = cut(j + 1);
        }
        if (t1 > t0) {
            op(FWD_JOIN, FWD_CHAIN).slot = 1;
            diag(k + 1, FWD_CHAIN);
            FwdOp &o = op(FWD_TRI, FWD_WIDE);
            o.c = fcol;
            o.f = ff;
            o.np = fnp;
            o.t0 = t0;
            o.tn = t1 - t0;
            o.slot = ffrom_a ? 1 : -1;
            diag_wide = false;
        } else {
            // nothing to run beside the diagonal factor: it follows the
            // narrow update on the wide stream, with no join either way
            diag(k + 1, FWD_WIDE);
            diag_wide = true;
        }
        if (fcol >= 0 && j == FWD_DEFER - 1)
            fcol = -1;
    }
    op(FWD_JOIN, FWD_CHAIN).slot = 1;
    op(FWD_ZERO_UPPER, FWD_CHAIN);
    return ops;
}

} // namespace chol
