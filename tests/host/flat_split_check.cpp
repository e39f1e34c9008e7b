// Host-side check of the row pass's split of a position's tiles over its
// workgroups (row_grid / flat_begin / flat_owner / unit_records in
// sv_device.h): for many class mixes, tile counts and grids, the number of
// workgroups taking part (at least kRowMinTiles tiles each unless every unit
// is untruncated; with long pieces a multiple of the unit count, each
// workgroup inside one unit, when that keeps 5/8 of them), every one of them owning a contiguous, non-empty range,
// the ranges tiling the concatenation in order, the owner of every tile
// being the workgroup whose range holds it, every unit's records being
// exactly the pieces that cover it, and the record slots u + w unique and
// below n + G.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "sv_device.h"

using namespace sv;

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static unsigned next_u32() {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (unsigned)(rng_state >> 33);
}

static int n_aligned = 0;  // cases that took the unit-aligned split

static int check(const PosDesc& P, int ntiles, int G0) {
    const int n = pos_units(P);
    const int64_t T = (int64_t)n * ntiles;
    const int G = row_grid(P, T, G0);  // the workgroups the row pass lets take part
    const bool all_full = P.n_cls[CLS_FULL] == n;
    const int64_t want = all_full ? T : (T + kRowMinTiles - 1) / kRowMinTiles;
    const int Gm = (int)(want < G0 ? want : G0);
    // a multiple of the unit count (same pieces per unit) when that keeps 5/8
    // of the workgroups and pieces of kRowMinTiles tiles, else Gm
    int Gw = Gm;
    if (!all_full && n <= G0 && T >= (int64_t)Gm * 2 * kRowMinTiles) {
        for (int per = G0 / n; per >= 1; per--) {
            if (per * kRowMinTiles > ntiles) continue;
            if ((int64_t)n * per * 8 >= (int64_t)Gm * 5) Gw = n * per;
            break;
        }
    }
    if (G != Gw) return 1;
    const bool aligned = G % n == 0 && !all_full && G != Gm;
    if (aligned) n_aligned++;
    const int Ga = flat_active(T, G);
    if (flat_begin(T, G, 0) != 0 || flat_begin(T, G, G) != T) return 2;
    std::vector<int> owner(T, -1);
    for (int w = 0; w < G; w++) {
        const int64_t a = flat_begin(T, G, w), b = flat_begin(T, G, w + 1);
        if (b < a) return 3;
        if (w < Ga && b == a) return 4;  // a workgroup taking part without a tile
        if (w >= Ga && b != a) return 5;
        // an aligned split never puts two units into one workgroup
        if (aligned && b > a && a / ntiles != (b - 1) / ntiles) return 10;
        for (int64_t t = a; t < b; t++) owner[t] = w;
    }
    for (int64_t t = 0; t < T; t++)
        if (owner[t] < 0 || flat_owner(t, T, G) != owner[t]) return 6;
    std::vector<char> used(n + G, 0);
    for (int li = 0; li < n; li++) {
        const RecRange r = unit_records(P, li, ntiles, G0);
        const int w0 = owner[(int64_t)li * ntiles], w1 = owner[(int64_t)(li + 1) * ntiles - 1];
        if (r.first != li + w0 || r.count != w1 - w0 + 1) return 7;
        for (int w = w0; w <= w1; w++) {  // each of them streams part of unit li
            const int64_t a = flat_begin(T, G, w), b = flat_begin(T, G, w + 1);
            if (b <= (int64_t)li * ntiles || a >= (int64_t)(li + 1) * ntiles) return 8;
            const int slot = li + w;
            if (slot >= n + G || used[slot]) return 9;
            used[slot] = 1;
        }
    }
    return 0;
}

int main() {
    int cases = 0;
    const int grids[] = {1, 3, 256, 768, 1024};
    const int tiles[] = {1, 2, 5, 37, 61};
    for (int iter = 0; iter < 3000; iter++) {
        PosDesc P = {};
        const int scale = (iter % 3 == 0) ? 4 : (iter % 3 == 1 ? 64 : 700);
        for (int c = 0; c < kNumCls; c++)
            P.n_cls[c] = (next_u32() % 4 == 0) ? 0 : (int)(next_u32() % (unsigned)scale);
        if (iter % 5 == 0)  // untruncated units only
            for (int c = 0; c < kNumCls; c++)
                if (c != CLS_FULL) P.n_cls[c] = 0;
        if (pos_units(P) == 0) P.n_cls[next_u32() % kNumCls] = 1;
        const int G = grids[next_u32() % 5], nt = tiles[next_u32() % 5];
        const int rc = check(P, nt, G);
        if (rc) {
            printf("FAIL rc=%d n_cls=%d,%d,%d,%d ntiles=%d G=%d\n", rc, P.n_cls[0], P.n_cls[1],
                   P.n_cls[2], P.n_cls[3], nt, G);
            return 1;
        }
        cases++;
    }
    if (n_aligned == 0) {
        printf("FAIL no case took the unit-aligned split\n");
        return 1;
    }
    printf("ok %d cases (%d unit-aligned)\n", cases, n_aligned);
    return 0;
}
