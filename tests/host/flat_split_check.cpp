// Host-side check of the row pass's split of a position's tiles over its
// workgroups (flat_begin / flat_owner / unit_records in sv_device.h): for
// many unit counts, tile counts and grids, every workgroup taking part owns a
// contiguous, non-empty range, the ranges tile the concatenation in order,
// the owner of every tile is the workgroup whose range holds it, every unit's
// records are exactly the pieces that cover it, and the record slots u + w
// are unique and below n + G.
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

static int check(int n, int ntiles, int G) {
    const int64_t T = (int64_t)n * ntiles;
    const int Ga = flat_active(T, G);
    if (flat_begin(T, G, 0) != 0 || flat_begin(T, G, G) != T) return 2;
    std::vector<int> owner(T, -1);
    for (int w = 0; w < G; w++) {
        const int64_t a = flat_begin(T, G, w), b = flat_begin(T, G, w + 1);
        if (b < a) return 3;
        if (w < Ga && b == a) return 4;  // a workgroup taking part without a tile
        if (w >= Ga && b != a) return 5;
        for (int64_t t = a; t < b; t++) owner[t] = w;
    }
    for (int64_t t = 0; t < T; t++)
        if (owner[t] < 0 || flat_owner(t, T, G) != owner[t]) return 6;
    std::vector<char> used(n + G, 0);
    for (int li = 0; li < n; li++) {
        const RecRange r = unit_records(li, n, ntiles, G);
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
        const int scale = (iter % 3 == 0) ? 4 : (iter % 3 == 1 ? 64 : 2800);
        const int n = 1 + (int)(next_u32() % (unsigned)scale);
        const int G = grids[next_u32() % 5], nt = tiles[next_u32() % 5];
        const int rc = check(n, nt, G);
        if (rc) {
            printf("FAIL rc=%d n=%d ntiles=%d G=%d\n", rc, n, nt, G);
            return 1;
        }
        cases++;
    }
    printf("ok %d cases\n", cases);
    return 0;
}
