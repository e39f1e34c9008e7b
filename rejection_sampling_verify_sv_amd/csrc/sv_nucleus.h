// sv_nucleus.h — the top_p cut over the whole vocabulary (top_k off).
//
// deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…", section
// "Kesme her iki tarafta eşleşmek zorunda": both distributions are cut to the
// smallest head of the ranking whose preceding mass stays below top_p.  With
// top_k disabled that head can hold tens of thousands of tokens, so the cut is
// located by mass instead of by sorting the row.  Weights and buckets are
// those of the anchor window (sv_device.h).
//
// The row pass leaves each nucleus unit's mass histogram, one per piece.
// Then cut_decide_kernel finishes the cut, one workgroup per unit, or several when the
// units are few:
//   hist     the unit's histogram in LDS: the sum of its pieces, or, when a
//            piece saw a token above the window, the row again, anchored at
//            the row max;
//   select   Z = total mass; the boundary bucket is the last non-empty bucket
//            whose preceding mass is below top_p Z, with its exact logit
//            range [l_lo, l_hi];
//   collect  the row once more (a slice of it per workgroup of a split
//            unit), keeping the keys of the boundary bucket's tokens; a split
//            unit's workgroups publish theirs to global memory and the last
//            to arrive goes on with all of them (a bucket too large for LDS
//            is instead narrowed by a radix select over its keys, see
//            resolve_wide);
//   resolve  a token of the boundary bucket is kept when the mass before the
//            bucket plus the mass of the bucket's tokens ranked ahead of it
//            (logit desc, id asc) is below top_p Z.  The cut key tau (last
//            kept token) and the kept mass S define the distribution
//            p(i) = [key_i >= tau] exp(t_i / 64) / S.
// Within a bucket the masses are exact fixed-point integers; across buckets
// they are combined in fp64 in one fixed order, so the cut is deterministic
// (the workgroups of a split unit find the same boundary).  One launch per
// position replaces grid-wide passes and the launches between them: a few
// hundred workgroups reading rows on their own saturate HBM, and a few
// dozen units are split so that their rows are still read by many compute
// units.
#pragma once

#include "sv_decide.h"

namespace sv {

// Smallest ranking image o in [-inf, +inf] with nuc_gbin(o) >= beta (that of
// +inf is kNW, so one exists); the logits of bucket beta are exactly those
// from ord_float(first(beta)) to ord_float(first(beta + 1) - 1).  Wave-wide: every lane calls it and gets the
// result; each round probes 64 evenly spaced images and keeps the gap where
// the predicate turns true, so six rounds cover the 32-bit range.
__device__ inline uint32_t nuc_first_image(int beta, float la, float cb) {
    uint32_t lo = 0x007FFFFFu, hi = 0xFF800000u;
    const int lane = lane_id();
    while (lo < hi) {
        const uint64_t span = hi - lo;
        const uint32_t p = lo + (uint32_t)((span * (uint64_t)(lane + 1)) / (kWave + 1));
        const uint64_t m = __ballot(nuc_gbin(ord_float(p), la, cb) >= beta);
        const int f = m ? __ffsll((unsigned long long)m) - 1 : kWave;
        // f is the same in every lane: scalar reads of lanes f - 1 and f
        const uint32_t nlo =
            f == 0 ? lo : (uint32_t)__builtin_amdgcn_readlane((int)p, f - 1) + 1u;
        const uint32_t nhi = f == kWave ? hi : (uint32_t)__builtin_amdgcn_readlane((int)p, f);
        lo = nlo;
        hi = nhi;
    }
    return lo;
}
// Max over the row-pass pieces of one unit (keys[0] holds each piece's max as
// float bits); every thread of the block gets it.  Contains barriers.
__device__ inline float unit_piece_max(const PartSlot* parts, RecRange r, uint64_t* tmp) {
    float m = -INFINITY;
    for (int i = threadIdx.x; i < r.count; i += kThreads)
        m = fmaxf(m, __uint_as_float((uint32_t)parts[r.first + i].keys[0]));
    return block_max_f32(m, tmp);
}

constexpr int kSub = 256;
static_assert(kSub == kThreads, "one sub-bucket per thread");

// Boundary buckets of more than kCollectCap tokens (nearly flat rows, high
// temperatures) are resolved by the unit's workgroup alone, re-reading the
// row once per step of a radix select over the bucket's keys:
//   range  the bucket's keys form one interval [lo, hi] of the key order
//          (the bucket index never rises as the logit falls, and equal
//          logits share a bucket); one pass finds it;
//   level  the interval is cut into at most kBins bins of 2^s consecutive
//          keys; one pass adds every token's fixed-point weight and a count
//          into its bin; the boundary bin is chosen as the boundary bucket
//          was (last bin with mass whose preceding mass is below top_p Z),
//          the mass of the bins ahead of it joins the mass before the
//          interval, and the interval shrinks to that bin;
//   rank   once the interval holds at most kThreads tokens (with 2^s = 1 it
//          holds one, as keys are distinct), they are ranked one per thread
//          like the boundary sub-bucket of the narrow path.
// The first token of every chosen bin is kept, so tau stays in the interval.
// `pre` counts the bucket's mass ranked ahead of the interval (exact), the
// preceding mass of a token is A + sc * (pre + ...).  Returns the cut key and
// the kept mass through fu.  Contains barriers; every thread of the block
// calls it.
constexpr int kBins = 2048;

template <int DT, bool kAligned>
__device__ void resolve_wide(const void* row, int64_t V, FnUnit* fu, float la, float cb,
                             float l_lo, float l_hi, double A, double sc, double target,
                             uint64_t* s_mass /* kBins */,
                             uint32_t* s_cnt /* kBins */, uint64_t* s_key /* kThreads */,
                             uint64_t* s_w /* kThreads */, uint64_t* s_tmp /* kWaves */) {
    using TS = TileShape<DT>;
    constexpr int kPer = kBins / kThreads;  // bins per thread, in descending key order
    __shared__ unsigned long long s_lo, s_hi, s_tau, s_kept;
    __shared__ uint64_t s_pre;
    __shared__ int s_star, s_n;
    __shared__ uint32_t s_bincnt;
    static_assert(kBins == 2048, "11-bit bins");
    if (threadIdx.x == 0) {
        s_lo = ~0ull;
        s_hi = 0ull;
    }
    __syncthreads();
    {
        uint64_t lo = ~0ull, hi = 0ull;
        stream_range<DT, kAligned>(row, 0, V, [&](float (&v)[TS::kE], int64_t t0, bool)
                                                  __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                if (v[i] >= l_lo && v[i] <= l_hi) {
                    const uint64_t key = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
                    lo = key < lo ? key : lo;
                    hi = key > hi ? key : hi;
                }
            }
        });
        if (lo <= hi) {
            atomicMin(&s_lo, (unsigned long long)lo);
            atomicMax(&s_hi, (unsigned long long)hi);
        }
    }
    __syncthreads();
    uint64_t rlo = s_lo, rhi = s_hi;
    uint64_t pre = 0ull;
    for (;;) {
        // bin width 2^s with (rhi - rlo) >> s < kBins
        const uint64_t span = rhi - rlo;
        const int bits = span == 0ull ? 0 : 64 - __clzll((long long)span);
        const int s = bits > 11 ? bits - 11 : 0;
        for (int i = threadIdx.x; i < kBins; i += kThreads) {
            s_mass[i] = 0ull;
            s_cnt[i] = 0u;
        }
        if (threadIdx.x == 0) s_star = -1;
        __syncthreads();
        stream_range<DT, kAligned>(row, 0, V, [&](float (&v)[TS::kE], int64_t t0, bool)
                                                  __attribute__((always_inline)) {
            // the bucket's logits first, as one bit mask per lane (its keys
            // form [lo, hi] inside them): keys are built for those tokens only
            uint32_t bits = 0u;
#pragma unroll
            for (int i = TS::kE - 1; i >= 0; i--)
                bits = (bits << 1) | ((v[i] >= l_lo && v[i] <= l_hi) ? 1u : 0u);
            while (bits != 0u) {
                const int i = __builtin_ctz(bits);
                bits &= bits - 1u;
                const float vi = pick_elem(v, i);
                const uint64_t key = make_key(vi, (uint32_t)elem_id<DT>(t0, i));
                if (key >= rlo && key <= rhi) {  // in the bucket (its keys form [lo, hi])
                    const int bin = (int)((key - rlo) >> s);
                    int bk;
                    const uint64_t w = nuc_wfix_t(nuc_t(vi, la, cb), &bk);
                    atomicAdd((unsigned long long*)&s_mass[bin], (unsigned long long)w);
                    atomicAdd(&s_cnt[bin], 1u);
                }
            }
        });
        __syncthreads();
        uint64_t mass[kPer];
        uint64_t mine = 0ull;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            mass[q] = s_mass[kBins - 1 - (threadIdx.x * kPer + q)];
            mine += mass[q];
        }
        uint64_t tot;
        uint64_t run = pre + block_exclusive_scan(mine, s_tmp, &tot);
        int cand = -1;
        uint64_t cand_before = 0ull;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            if (mass[q] != 0ull && A + sc * (double)run < target) {
                cand = threadIdx.x * kPer + q;
                cand_before = run;
            }
            run += mass[q];
        }
        if (cand >= 0) atomicMax(&s_star, cand);
        __syncthreads();
        const int star = s_star;
        if (star < 0) {  // cannot happen: the interval's first token qualifies
            if (threadIdx.x == 0) fn_put_status(fu, 1);
            __syncthreads();
            return;
        }
        if (cand == star) {
            s_pre = cand_before;
            s_bincnt = s_cnt[kBins - 1 - star];
        }
        __syncthreads();
        pre = s_pre;
        const uint32_t nbin = s_bincnt;
        const uint64_t j = (uint64_t)(kBins - 1 - star);
        rlo = rlo + (j << s);
        const uint64_t top = rlo + ((1ull << s) - 1ull);
        rhi = top < rhi ? top : rhi;
        __syncthreads();  // s_tmp, s_mass and s_cnt are reused
        if (nbin <= (uint32_t)kThreads || s == 0) break;
    }
    if (threadIdx.x == 0) {
        s_n = 0;
        s_tau = ~0ull;
        s_kept = 0ull;
    }
    __syncthreads();
    stream_range<DT, kAligned>(row, 0, V, [&](float (&v)[TS::kE], int64_t t0, bool)
                                              __attribute__((always_inline)) {
        uint32_t bits = 0u;
#pragma unroll
        for (int i = TS::kE - 1; i >= 0; i--)
            bits = (bits << 1) | ((v[i] >= l_lo && v[i] <= l_hi) ? 1u : 0u);
        while (bits != 0u) {
            const int i = __builtin_ctz(bits);
            bits &= bits - 1u;
            const float vi = pick_elem(v, i);
            const uint64_t key = make_key(vi, (uint32_t)elem_id<DT>(t0, i));
            if (key >= rlo && key <= rhi) {
                const int slot = atomicAdd(&s_n, 1);
                if (slot < kThreads) {
                    int bk;
                    s_key[slot] = key;
                    s_w[slot] = nuc_wfix_t(nuc_t(vi, la, cb), &bk);
                }
            }
        }
    });
    __syncthreads();
    const int n = s_n < kThreads ? s_n : kThreads;
    if ((int)threadIdx.x < n) {
        const uint64_t key = s_key[threadIdx.x];
        uint64_t p = pre;
        for (int j = 0; j < n; j++) p += s_key[j] > key ? s_w[j] : 0ull;
        if (A + sc * (double)p < target) {
            atomicMin(&s_tau, (unsigned long long)key);
            atomicAdd(&s_kept, (unsigned long long)s_w[threadIdx.x]);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        fn_put_cut(fu, s_tau, A + sc * (double)(pre + s_kept));
    }
    __syncthreads();
}

// The boundary of the cut from the unit's histogram in s_h (kNW buckets,
// fixed point): Z, the boundary bucket (the last non-empty bucket whose
// preceding mass is below top_p Z), the mass A before it and its logit range.
// Every thread calls it (barriers inside); o->beta = -1 when there is no mass.
struct SelOut {
    double Z, A;
    float l_lo, l_hi;
    int beta;
};

__device__ inline void select_boundary(const uint64_t* s_h, float top_p, float la, float cb,
                                       double* s_tmp /* kWaves */, int* s_star, SelOut* o) {
    constexpr int kPer = kNW / kThreads;  // buckets per thread, taken in descending order
    // this thread's lowest bucket; opaque, so that the scales below are
    // loaded here rather than hoisted and held across the caller's loop
    const int j0 = kNW - kPer * (tid_opaque() + 1);
    double m[kPer];  // bucket masses, highest bucket first
    double mine = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; q++) {
        const int j = j0 + kPer - 1 - q;
        m[q] = nuc_scale(j) * ((double)s_h[j] * kUnfix);
        mine += m[q];
    }
    double Z;
    const double excl0 = block_exclusive_scan(mine, s_tmp, &Z);
    const double target = (double)top_p * Z;
    if (threadIdx.x == 0) *s_star = -1;
    __syncthreads();
    double run = excl0;
    int best = -1;
    double best_before = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; q++) {
        if (m[q] != 0.0 && run < target) {  // a bucket's mass is 0 iff it holds no weight
            best = (int)threadIdx.x * kPer + q;
            best_before = run;
        }
        run += m[q];
    }
    if (best >= 0) atomicMax(s_star, best);
    __syncthreads();
    const int star = *s_star;
    if (star >= 0 && best == star) {
        o->Z = Z;
        o->A = best_before;
        o->beta = kNW - 1 - star;
    }
    if (star < 0 && threadIdx.x == 0) o->beta = -1;
    if (star >= 0 && wave_id() < 2) {  // wave 0: the range's low end, wave 1: its high end
        const uint32_t im = nuc_first_image(kNW - 1 - star + wave_id(), la, cb);
        if (lane_id() == 0) {
            if (wave_id() == 0)
                o->l_lo = ord_float(im);
            else
                o->l_hi = ord_float(im - 1u);
        }
    }
    __syncthreads();
}

// Workgroups per unit in the cut.  One workgroup alone collects a row at
// about 40 GB/s, far below its share of HBM, so when the units are few each
// gets several, up to one per compute unit in all (the grid holds two per
// compute unit; two on one compute unit slow each other down), at most
// kMaxSplit and one per tile of the row.  A split unit's index in the nucleus
// list is below gridDim.x / 4 here, and below kThreads with the split by
// density in the kernel: either way below kGrid / 2, the rows of fn_sync and
// fn_keys.
constexpr int kMaxSplit = 8;
constexpr int kDenseSplit = 3;   // workgroups of a unit expected to keep many boundary keys
constexpr int kDenseKeys = 128;  // boundary keys from which a collect counts as such
__host__ __device__ inline int fn_split(int n_units, int grid, int ntiles) {
    if (n_units <= 0) return 1;
    int s = (grid / 2) / n_units;
    s = s < kMaxSplit ? s : kMaxSplit;
    s = s < ntiles ? s : ntiles;
    return s > 1 ? s : 1;
}

// Position k after its row pass: the cut of every nucleus unit, one or (few
// units) several workgroups each (histogram, boundary bucket, its keys and
// the exact cut, see the top of this file), and the decision of every live
// row (sv_decide.h).
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void cut_decide_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    static_assert(TS::kE <= 32, "hit mask is 32 bits");
    constexpr int kOwn = 4;  // boundary tokens a thread ranks per pass
    constexpr int kSortSel = 512;  // above: the boundary sub-bucket is ranked by a sort
    constexpr int kRing = DT == SV_BF16 ? 3 : 4;  // tiles in flight while collecting a slice
    constexpr int kWaveCap = kCollectCap / kWaves;  // boundary keys a wave can hold
    static_assert(kNW <= kCollectCap && kBins <= kCollectCap && kBins + kThreads <= kCollectCap,
                  "LDS arrays are shared between the steps");
    __shared__ uint64_t s_h[kCollectCap];    // histogram, then the boundary tokens' weights
    __shared__ uint64_t s_key[kCollectCap];  // boundary-bucket keys
    __shared__ uint16_t s_sel[kCollectCap];
    __shared__ uint8_t s_sb[kCollectCap];
    __shared__ uint64_t s_sub[kSub];
    __shared__ uint64_t s_tmp[kWaves], s_red[kWaves];
    __shared__ double s_tmpd[kWaves];
    __shared__ SelOut s_so;
    __shared__ unsigned long long s_tau, s_kept;
    __shared__ int s_star, s_nsel, s_wcnt[kWaves], s_base, s_last;
    __shared__ uint64_t s_before;
    __shared__ DecideIntent s_it[kWaves];
    __shared__ int s_dbase[kNumCls + 3];
    constexpr int kPend = 32;  // completed nucleus rows awaiting their decision
    __shared__ int s_pend[kPend], s_npend;
    __shared__ PosDesc s_P;  // this launch's lists, for the decisions
    static_assert(sizeof(TopkScratch) * kWaves <= sizeof(uint64_t) * kCollectCap,
                  "the decisions' scratch lies over s_key");
    const PosDesc P = a.pos[k];
    if (threadIdx.x == 0) s_P = P;  // read after the barriers below
    const int n_units = P.n_cls[CLS_NUCLEUS];
    const int32_t* list = nuc_list(a, k);
    // Few units: each is split over S workgroups, which all find the same
    // boundary from the same histogram and collect the keys of one slice of
    // the row each; the last of them to finish ranks the keys.  Many units:
    // one workgroup per unit.
    const int S = fn_split(n_units, (int)gridDim.x, a.ntiles);
    int n_work = n_units * S;
    // A unit whose row kept many boundary keys at its last cut (a bit per
    // side in RowInfo.pad) will likely do so again, and such a collect is
    // bound by its workgroup's instruction issue.  When the even split gives
    // one workgroup per unit, those units get up to kDenseSplit workgroups
    // each, as many as keep all work items one per compute unit; s_wpre[li]
    // is then the first work item of unit li.
    __shared__ uint16_t s_wpre[kThreads + 1];
    bool var = false;
    if (S == 1 && n_units > 0 && n_units <= kThreads && !a.stats) {
        uint64_t dn = 0;
        if ((int)threadIdx.x < n_units) {
            const int b = unit_b(a, list[threadIdx.x], k);
            dn = (a.rows[b].pad & 3) ? 1ull : 0ull;
        }
        uint64_t nd;
        const uint64_t ex = block_exclusive_scan(dn, s_tmp, &nd);  // barriers
        int sd = min(kDenseSplit, a.ntiles);
        while (sd > 1 && n_units + (sd - 1) * (int)nd > (int)gridDim.x / 2) sd--;
        var = nd > 0 && sd > 1;
        if (var) {
            if ((int)threadIdx.x < n_units)
                s_wpre[threadIdx.x] = (uint16_t)(threadIdx.x + (sd - 1) * (int)ex);
            if (threadIdx.x == 0) s_wpre[n_units] = (uint16_t)(n_units + (sd - 1) * (int)nd);
            n_work = n_units + (sd - 1) * (int)nd;
        }
        __syncthreads();
    }
    // one unit, or one slice of a unit split over Su workgroups; true for the
    // workgroup that completes the unit's cut
    auto cut_unit = [&](int li, int sl, int Su) -> bool {
        const int u = list[li];
        const int b = unit_b(a, u, k), side = u & 1;
        const RowInfo& ri = a.rows[b];
        FnUnit* fu = a.fn_unit + u;
        const void* row = unit_row<DT>(a, b, side, unit_rowidx(a, u, b, k));
        const float cb = bucket_coef(ri.T);
        const RecRange rr =
            unit_records(P, unit_index(P, CLS_NUCLEUS, li), a.ntiles, a.g_row);
        const bool re = fu->rehist != 0;
        // 1. the unit's histogram in LDS
        float la;
        if (re) {
            for (int j = threadIdx.x; j < kNW; j += kThreads) s_h[j] = 0ull;
            la = unit_piece_max(a.parts, rr, s_red);  // barriers
            stream_range<DT, kAligned>(row, 0, a.V, [&](float (&v)[TS::kE], int64_t, bool)
                                                        __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < TS::kE; i++) {
                    const float t = nuc_t(v[i], la, cb);
                    int bin;
                    const uint64_t w = nuc_wfix_t(t, &bin);
                    if (nuc_in(t)) atomicAdd((unsigned long long*)&s_h[bin], (unsigned long long)w);
                }
            });
        } else {
            // thread t sums buckets t + q kThreads over the pieces in
            // registers; a piece's slot holds its buckets [lo, hi] from the
            // slot's start (every load is clamped into the slot and the
            // buckets outside the range masked off)
            constexpr int kPer = kNW / kThreads;
            la = fu->la;
            uint64_t acc[kPer];
#pragma unroll
            for (int q = 0; q < kPer; q++) acc[q] = 0ull;
            for (int p = 0; p < rr.count; p++) {
                const uint64_t rg = a.parts[rr.first + p].keys[1];
                const uint64_t* h = a.hist + (int64_t)(rr.first + p) * kHistSlot;
                const int lo = (int)(uint32_t)(rg >> 32), hi = (int)(uint32_t)rg;
                uint64_t x[kPer];
#pragma unroll
                for (int q = 0; q < kPer; q++) {
                    int i = q * kThreads + (int)threadIdx.x - lo;
                    i = i < 0 ? 0 : (i > kHistSlot - 1 ? kHistSlot - 1 : i);
                    x[q] = h[i];
                }
#pragma unroll
                for (int q = 0; q < kPer; q++) {
                    const int j = q * kThreads + (int)threadIdx.x;
                    acc[q] += (j >= lo && j <= hi) ? x[q] : 0ull;
                }
            }
#pragma unroll
            for (int q = 0; q < kPer; q++) s_h[q * kThreads + threadIdx.x] = acc[q];
        }
        __syncthreads();
        // 2. the boundary bucket
        select_boundary(s_h, ri.top_p, la, cb, s_tmpd, &s_star, &s_so);  // barriers
        const SelOut so = s_so;
        if (threadIdx.x == 0) fn_put_status(fu, so.beta < 0 ? 2 : 0);  // 2: no finite logit
        if (so.beta < 0) {
            __syncthreads();
            return sl == 0;
        }
        // 3. the boundary bucket's keys in this workgroup's slice of the row,
        //    appended by each wave to its own quarter of s_h (free once the
        //    boundary is known) with a wave-uniform count: no atomics and no
        //    scans on the way
        const float l_lo = so.l_lo, l_hi = so.l_hi;
        const int64_t e_lo = ((int64_t)sl * a.ntiles / Su) * TS::kTile;
        const int64_t e_hi = min(((int64_t)(sl + 1) * a.ntiles / Su) * TS::kTile, (int64_t)a.V);
        uint64_t* const s_mine = s_h + wave_id() * kWaveCap;
        int filled = 0;  // wave-uniform
        auto cbody = [&](float (&v)[TS::kE], int64_t t0, bool)
                                      __attribute__((always_inline)) {
            // v lies in [l_lo, l_hi] iff clamping it to that range leaves it
            // unchanged (never for -inf past `end`); the lane's bits are
            // formed on every tile (a compare and a select per element),
            // which the tiles with hits then use as they are
            uint32_t hit = 0u;
#pragma unroll
            for (int i = 0; i < TS::kE; i++)
                hit |= (__builtin_amdgcn_fmed3f(v[i], l_lo, l_hi) == v[i] ? 1u : 0u) << i;
            if (__ballot(hit != 0u) == 0ull) return;
            uint32_t id0 = (uint32_t)elem_id<DT>(t0, 0);
            asm volatile("" : "+v"(id0));
            // round r stores the r-th hit of every lane that has one; the
            // lane's slot is its rank among those lanes
            for (;;) {
                const uint64_t m = __ballot(hit != 0u);
                if (m == 0ull) break;
                if (hit != 0u) {
                    constexpr int kVec = Elt<DT>::kVec;
                    const int i = __builtin_ctz(hit);
                    hit &= hit - 1u;
                    const int slot = filled + (int)__builtin_amdgcn_mbcnt_hi(
                                                  (uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    const uint32_t id = id0 + (uint32_t)((i / kVec) * kThreads * kVec + i % kVec);
                    if (slot < kWaveCap) s_mine[slot] = make_key(pick_elem(v, i), id);
                }
                filled += __popcll(m);
            }
        };
        // kRing tiles in flight: the cuts run at two workgroups per compute
        // unit at most (registers, LDS), often fewer, and the double buffer
        // of the row pass left the re-read latency-bound (about 4 TB/s over
        // a few hundred units on the 1024-row mix)
        {
            TileRing<DT, kAligned, kRing> ring;
            ring.start(row, e_lo, e_hi);
            ring.run(row, e_lo, e_hi, cbody);
        }
        if (lane_id() == 0) s_wcnt[wave_id()] = filled;
        __syncthreads();
        int n = 0;
        bool over = false;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            n += s_wcnt[w];
            over |= s_wcnt[w] > kWaveCap;
        }
        if (!over) {  // the waves' lists, end to end, into s_key
            for (int i = threadIdx.x; i < n; i += kThreads) {
                int w = 0, off = 0;
#pragma unroll
                for (int q = 0; q < kWaves - 1; q++) {
                    const bool past = i >= off + s_wcnt[w];
                    off += past ? s_wcnt[w] : 0;
                    w += past ? 1 : 0;
                }
                s_key[i] = s_h[w * kWaveCap + (i - off)];
            }
        }
        if (Su > 1) {
            // Publish the slice's keys (device-scope stores, see dev_store);
            // only the unit's last workgroup goes on, and reads them all.
            int32_t* const sync = a.fn_sync + 2 * li;  // [0] arrived, [1] keys reserved
            uint64_t* const gk = a.fn_keys + (int64_t)li * kCollectCap;
            __syncthreads();
            if (threadIdx.x == 0) s_base = atomicAdd(&sync[1], over ? kCollectCap + 1 : n);
            __syncthreads();
            const int base = s_base;
            if (!over)
                for (int i = threadIdx.x; i < n && base + i < kCollectCap; i += kThreads)
                    dev_store(gk + base + i, s_key[i]);
            dev_stores_done();  // every wave's keys, before the arrival below
            __syncthreads();
            if (threadIdx.x == 0)
                s_last = __hip_atomic_fetch_add(&sync[0], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == Su - 1;
            __syncthreads();
            if (!s_last) return false;
            n = dev_load(&sync[1]);
            over = n > kCollectCap;
            if (!over)
                for (int i = threadIdx.x; i < n; i += kThreads)
                    s_key[i] = dev_load(gk + i);
            __syncthreads();
            if (threadIdx.x == 0) {  // ready for the next position's launch
                sync[0] = 0;
                sync[1] = 0;
            }
        }
        __syncthreads();
        if (over) n = kCollectCap + 1;
        if (threadIdx.x == 0) {  // the hint for the row's next cut
            const int bit = 1 << side;
            if (n > kDenseKeys)
                atomicOr(&a.rows[b].pad, bit);
            else
                atomicAnd(&a.rows[b].pad, ~bit);
        }
        const double target = (double)ri.top_p * so.Z;
        const double sc = nuc_scale(so.beta) * kUnfix;
        const double A = so.A;
        if (n < 1 || n > kCollectCap) {
            if (n < 1) {  // cannot happen: the boundary bucket has mass
                if (threadIdx.x == 0) fn_put_status(fu, 1);
                __syncthreads();
                return true;
            }
            if (threadIdx.x == 0) fn_put_la(fu, la);
            resolve_wide<DT, kAligned>(row, a.V, fu, la, cb, so.l_lo, so.l_hi, A, sc, target, s_h,
                                       reinterpret_cast<uint32_t*>(s_key), s_h + kBins,
                                       s_key + kBins, s_tmp);  // tau and S (barriers)
            return true;
        }
        // 4. the cut inside the boundary bucket
        s_sub[threadIdx.x] = 0ull;
        if (threadIdx.x == 0) {
            s_tau = ~0ull;
            s_kept = 0ull;
            s_star = -1;
            s_nsel = 0;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kThreads) {
            const uint64_t key = s_key[i];
            const float t = nuc_t(key_logit(key), la, cb);
            const float fr = t - floorf(t);
            // sub-buckets in ranking order: a larger fraction is a larger logit
            int sb = kSub - 1 - (int)(fr * (float)kSub);
            sb = sb < 0 ? 0 : (sb >= kSub ? kSub - 1 : sb);
            const uint64_t w = nuc_wrel(fr);
            s_h[i] = w;
            s_sb[i] = (uint8_t)sb;
            atomicAdd((unsigned long long*)&s_sub[sb], (unsigned long long)w);
        }
        __syncthreads();
        {
            const uint64_t mine = s_sub[threadIdx.x];
            uint64_t tot;
            const uint64_t before = block_exclusive_scan(mine, s_tmp, &tot);
            const bool cand = mine != 0ull && A + sc * (double)before < target;
            if (cand) atomicMax(&s_star, (int)threadIdx.x);
            __syncthreads();
            if ((int)threadIdx.x == s_star) s_before = before;
        }
        __syncthreads();
        const int star = s_star;
        if (star < 0) {  // cannot happen: the bucket's first token qualifies
            if (threadIdx.x == 0) fn_put_status(fu, 1);
            __syncthreads();
            return true;
        }
        for (int i = threadIdx.x; i < n; i += kThreads)
            if (s_sb[i] == star) s_sel[atomicAdd(&s_nsel, 1)] = (uint16_t)i;
        __syncthreads();
        const int nsel = s_nsel;
        const uint64_t before = s_before;
        // Many tokens in the boundary sub-bucket: rounded logits (bf16) put
        // every token of one value there, and counting, for each token, the
        // mass of those ranked ahead of it costs nsel^2.
        bool one_value = false;
        if (nsel > kSortSel) {
            // all of one logit?  (the high halves of their keys)
            uint64_t hi = 0ull, nlo = 0ull;
            for (int i = threadIdx.x; i < nsel; i += kThreads) {
                const uint64_t h = s_key[s_sel[i]] >> 32;
                hi = h > hi ? h : hi;
                nlo = (~h & 0xFFFFFFFFull) > nlo ? (~h & 0xFFFFFFFFull) : nlo;
            }
            hi = block_max_u64(hi, s_red);    // barriers
            nlo = block_max_u64(nlo, s_red);  // barriers
            one_value = hi == (~nlo & 0xFFFFFFFFull);
        }
        if (one_value) {
            // One value, one weight w: the token of rank r (ascending id)
            // has r w ahead of it, so the kept ones are the m smallest ids
            // with m the count of r where A + sc (before + r w) < target
            // (the per-token test, monotone in r), and tau is the key of the
            // m-th smallest id, found by a radix select over the ids.
            const uint64_t key0 = s_key[s_sel[0]];
            const float l0 = key_logit(key0);
            const float t0 = nuc_t(l0, la, cb);
            const uint64_t w = nuc_wrel(t0 - floorf(t0));
            if (threadIdx.x == 0) {
                int lo = 0, hi = nsel;  // kept(r) holds for r < m
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (A + sc * (double)(before + (uint64_t)mid * w) < target)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                s_nsel = lo;  // m (>= 1: the sub-bucket's first token qualifies)
            }
            __syncthreads();
            const int m = s_nsel;
            // the (m - 1)-th smallest id, 8 bits at a time from the top (none
            // kept, m = 0, leaves tau and the kept mass as they are)
            uint32_t prefix = 0u;
            int rank = m - 1;
            uint32_t* const s_cnt = reinterpret_cast<uint32_t*>(s_sub);  // kSub words, free now
            for (int shift = 24; m > 0 && shift >= 0; shift -= 8) {
                s_cnt[threadIdx.x] = 0u;
                __syncthreads();
                const uint32_t mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
                for (int i = threadIdx.x; i < nsel; i += kThreads) {
                    const uint32_t id = key_id(s_key[s_sel[i]]);
                    if ((id & mask) == prefix) atomicAdd(&s_cnt[(id >> shift) & 0xFFu], 1u);
                }
                __syncthreads();
                uint64_t tot;
                const uint64_t c = s_cnt[threadIdx.x];
                const uint64_t ex = block_exclusive_scan(c, s_tmp, &tot);  // barriers
                if ((uint64_t)rank >= ex && (uint64_t)rank < ex + c) {
                    s_star = (int)threadIdx.x;
                    s_before = ex;
                }
                __syncthreads();
                prefix |= (uint32_t)s_star << shift;
                rank -= (int)s_before;
                __syncthreads();
            }
            if (threadIdx.x == 0 && m > 0) {
                s_tau = make_key(l0, prefix);
                s_kept = (unsigned long long)m * w;
            }
        } else if (nsel > kSortSel) {
            // Sorted (descending keys) instead, the mass ahead of a token is
            // the prefix before it: the same integers, so the same cut.
            int np = kThreads;
            while (np < nsel) np <<= 1;  // <= kCollectCap: nsel <= n
            for (int i = threadIdx.x; i < np; i += kThreads)
                s_h[i] = i < nsel ? s_key[s_sel[i]] : 0ull;  // key 0: below every token
            __syncthreads();
            block_sort_desc(s_h, np);  // barriers
            // a token's weight, as the sub-buckets above computed it
            auto wkey = [&](uint64_t key) __attribute__((always_inline)) {
                const float t = nuc_t(key_logit(key), la, cb);
                return nuc_wrel(t - floorf(t));
            };
            constexpr int kPerT = kCollectCap / kThreads;
            const int per = np / kThreads, i0 = (int)threadIdx.x * per;
            uint64_t mine = 0ull;
#pragma unroll
            for (int q = 0; q < kPerT; q++)
                if (q < per && i0 + q < nsel) mine += wkey(s_h[i0 + q]);
            uint64_t tot;
            uint64_t pre = before + block_exclusive_scan(mine, s_tmp, &tot);  // barriers
#pragma unroll
            for (int q = 0; q < kPerT; q++) {
                if (q < per && i0 + q < nsel) {
                    const uint64_t key = s_h[i0 + q], w = wkey(key);
                    if (A + sc * (double)pre < target) {
                        atomicMin(&s_tau, (unsigned long long)key);
                        atomicAdd(&s_kept, (unsigned long long)w);
                    }
                    pre += w;
                }
            }
        }
        for (int base = 0; nsel <= kSortSel && base < nsel; base += kThreads * kOwn) {
            uint64_t key[kOwn], pre[kOwn];
#pragma unroll
            for (int q = 0; q < kOwn; q++) {
                const int i = base + q * kThreads + (int)threadIdx.x;
                key[q] = i < nsel ? s_key[s_sel[i]] : ~0ull;  // placeholder, never kept
                pre[q] = before;
            }
            for (int j = 0; j < nsel; j++) {
                const int sj = s_sel[j];
                const uint64_t kj = s_key[sj], wj = s_h[sj];
#pragma unroll
                for (int q = 0; q < kOwn; q++) pre[q] += kj > key[q] ? wj : 0ull;
            }
#pragma unroll
            for (int q = 0; q < kOwn; q++) {
                const int i = base + q * kThreads + (int)threadIdx.x;
                if (i < nsel && A + sc * (double)pre[q] < target) {
                    atomicMin(&s_tau, (unsigned long long)key[q]);
                    atomicAdd(&s_kept, (unsigned long long)s_h[s_sel[i]]);
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            fn_put_cut(fu, s_tau, A + sc * (double)(before + s_kept));
            fn_put_la(fu, la);
        }
        __syncthreads();
        return true;
    };

    // Work items: the units' cuts first (the long ones), then the rows of the
    // other classes, R per item.  A nucleus row is decided by the
    // workgroup that completes the last of its units (its FnUnit is written
    // at device scope and the completion counted with a device-scope atomic,
    // see dev_store); such rows wait in s_pend and are decided kWaves at a
    // time when the workgroup runs out of work or the list is full, so that
    // the decisions add one step to a workgroup's chain of units, not one
    // per row.
    // rows per decision item: enough that the items fit in the workgroups the
    // cuts leave free, so that no workgroup runs a cut and a group in turn
    const int n_free = (int)gridDim.x - n_work;
    // the merged launch with a workgroup free for every row: each row's
    // positions are decided side by side, kWaves at a time
    const bool walk = k >= a.d0 && !a.stats && n_free >= a.B;
    int R = n_free > 0 ? (a.B + n_free - 1) / n_free : kDecideRows;
    R = walk ? 1 : (R + kDecideRows - 1) / kDecideRows * kDecideRows;
    const int n_groups = a.stats ? 0 : (a.B + R - 1) / R;  // the statistics decide nothing
    TopkScratch* const s_ts = reinterpret_cast<TopkScratch*>(s_key);  // free between units
    static_assert(sizeof(SpecSlot) * kWaves <= sizeof(uint64_t) * kSub, "slots lie over s_sub");
    SpecSlot* const s_slot = reinterpret_cast<SpecSlot*>(s_sub);  // free between units
    // positions a decision walks: its own, or every one in a dense step
    const int k_last = k >= a.d0 ? a.K : k;
    auto decide_pending = [&]() {
        const int np = s_npend;
        for (int i = 0; i < np; i += kWaves) {
            const int j = i + wave_id();
            for (int kk = k; kk <= k_last; kk++) {
                decide_rows<DT>(a.self, &s_P, kk, j < np ? s_pend[j] : -1, false, s_it, s_dbase,
                                s_ts, nullptr);
                __syncthreads();
            }
        }
        if (threadIdx.x == 0) s_npend = 0;
        __syncthreads();
    };
    if (threadIdx.x == 0) s_npend = 0;
    __syncthreads();
    for (int wi = blockIdx.x; wi < n_work + n_groups; wi += gridDim.x) {
        if (wi >= n_work) {
            const int r0 = (wi - n_work) * R;
            if (walk) {  // row r0's positions, kWaves at a time
                for (int kk = k; kk <= a.K; kk += kWaves) {
                    decide_rows<DT>(a.self, &s_P, kk, r0, true, s_it, s_dbase, s_ts, s_slot);
                    if (s_dbase[0]) break;  // read before the next call writes it
                }
                continue;
            }
            for (int r = r0; r < r0 + R && r < a.B; r += kDecideRows) {
                const int bw = r + wave_id();
                for (int kk = k; kk <= k_last; kk++) {
                    decide_rows<DT>(a.self, &s_P, kk, bw < a.B ? bw : -1, true, s_it, s_dbase,
                                    s_ts, nullptr);
                    __syncthreads();  // LDS is reused by the next rows
                }
            }
            continue;
        }
        int li, Su;
        if (var) {  // the last unit whose first work item is at most wi
            int lo = 0, hi = n_units - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int)s_wpre[mid] <= wi)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            li = lo;
            Su = (int)s_wpre[li + 1] - (int)s_wpre[li];
        } else {
            li = wi / S;
            Su = S;
        }
        const int sl = wi - (var ? (int)s_wpre[li] : li * S);
        if (!cut_unit(li, sl, Su) || a.stats) continue;
        if (threadIdx.x == 0) {
            const int b = unit_b(a, list[li], k);
            // the row's nucleus units in this launch: the target and the
            // draft unit of the position (the target alone at its last one);
            // every drafted position's in a dense step.  The last unit to
            // finish decides the row.
            const int L = a.rows[b].L;
            const int need = k >= a.d0 ? 2 * (L - a.d0) + 1
                                     : ((a.tree ? a.rows[b].kids != 0 : k < L) ? 2 : 1);
            bool last = true;
            if (need > 1) {
                dev_stores_done();  // this unit's FnUnit stores, before the count
                last = __hip_atomic_fetch_add(&a.fn_row[b], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == need - 1;
                if (last) a.fn_row[b] = 0;  // ready for the next position's launch
            }
            if (last) s_pend[s_npend++] = b;
        }
        __syncthreads();
        if (s_npend == kPend) decide_pending();
    }
    decide_pending();
}

}  // namespace sv
