// sv_nucleus.h — the top_p cut over the whole vocabulary (top_k off).
//
// deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…", section
// "Kesme her iki tarafta eşleşmek zorunda": both distributions are cut to the
// smallest head of the ranking whose preceding mass stays below top_p.  With
// top_k disabled that head can hold tens of thousands of tokens, so the cut is
// located by mass instead of by sorting the row.  Weights and buckets are
// those of the anchor window (sv_device.h):
//
//   row pass every piece of a nucleus unit adds its tokens' fixed-point
//            weights into its own LDS histogram over the window, written out
//            whole (no atomics between workgroups);
//   hist     only units with a token above the window: the same histogram
//            again, anchored at the row max;
//   select   per unit: sum the pieces, Z = total mass; the boundary bucket is
//            the last non-empty bucket whose preceding mass is below top_p Z,
//            and its exact logit range [l_lo, l_hi];
//   collect  the keys of the boundary bucket's tokens (a bucket too large for
//            the workgroup's LDS is instead narrowed by a radix select
//            over its keys that re-reads the row, see resolve_wide);
//   resolve  per unit: a token of the boundary bucket is kept when the mass
//            before the bucket plus the mass of the bucket's tokens ranked
//            ahead of it (logit desc, id asc) is below top_p Z.  The cut key
//            tau (last kept token) and the kept mass S define the
//            distribution p(i) = [key_i >= tau] exp(t_i / 64) / S.
// Within a bucket the masses are exact fixed-point integers; across buckets
// they are combined in fp64 in one fixed order, so the cut is deterministic.
// The streaming passes split the tiles of position k's nucleus units evenly
// over the workgroups, like the row pass; the per-unit steps run one
// workgroup per unit.
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
        const uint32_t nlo = f == 0 ? lo : (uint32_t)__shfl((int)p, f - 1, kWave) + 1u;
        const uint32_t nhi = f == kWave ? hi : (uint32_t)__shfl((int)p, f, kWave);
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

// Units marked by the row pass (a token above the anchor window): the
// histogram again, anchored at the row max, so every token has t <= 0.
// Pieces of other units are skipped without reading the row.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_hist_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    __shared__ uint64_t s_h[kNW];
    __shared__ uint64_t s_red[kWaves];
    const int n = a.pos[k].n_cls[CLS_NUCLEUS];
    const PosDesc P = a.pos[k];
    const int n_units = pos_units(P);
    const int64_t T = (int64_t)n * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    const int32_t* list = nuc_list(a, k);
    while (t < t_end) {
        const int li = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)li * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        t += tu1 - tu0;
        const int u = list[li];
        if (a.fn_unit[u].rehist == 0) continue;  // uniform over the block
        const int b = u >> 1, side = u & 1;
        const RowInfo& ri = a.rows[b];
        const float m = unit_piece_max(
            a.parts,
            unit_records(unit_index(P, CLS_NUCLEUS, side ? ri.li_d : ri.li_t), n_units, a.ntiles,
                         a.g_row),
            s_red);
        const float cb = bucket_coef(ri.T);
        for (int i = threadIdx.x; i < kNW; i += kThreads) s_h[i] = 0ull;
        __syncthreads();
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t, bool)
                                       __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const float tt = nuc_t(v[i], m, cb);
                int bin;
                const uint64_t w = nuc_wfix_t(tt, &bin);
                if (nuc_in(tt)) atomicAdd((unsigned long long*)&s_h[bin], (unsigned long long)w);
            }
        });
        __syncthreads();
        uint64_t* out = a.hist2 + (int64_t)(li + blockIdx.x) * kNW;
        for (int i = threadIdx.x; i < kNW; i += kThreads) out[i] = s_h[i];
        __syncthreads();  // s_h is cleared for the next piece
    }
}

// The cut's boundary for unit u (position k, nucleus list index li): sums
// the unit's piece histograms, then Z and the boundary bucket (the last
// non-empty bucket whose preceding mass is below top_p Z).  Every thread of
// the block calls it (barriers inside); the result lands in *o, with
// o->beta = -1 when the unit has no mass (no finite logit).
struct SelOut {
    double Z, A;
    float la, l_lo, l_hi;
    int beta;
};

__device__ inline void unit_select(const StepArgs& a, int k, int li, int u,
                                   double* s_tmp /* kWaves */, uint64_t* s_red /* kWaves */,
                                   int* s_star, SelOut* o) {
    constexpr int kPer = kNW / kThreads;  // buckets per thread, taken in descending order
    const int b = u >> 1, side = u & 1;
    const RowInfo& ri = a.rows[b];
    const FnUnit* fu = a.fn_unit + u;
    const PosDesc P = a.pos[k];
    const RecRange rr = unit_records(unit_index(P, CLS_NUCLEUS, side ? ri.li_d : ri.li_t),
                                     pos_units(P), a.ntiles, a.g_row);
    const bool re = fu->rehist != 0;
    float la;
    RecRange r;
    const uint64_t* hbase;
    if (re) {
        la = unit_piece_max(a.parts, rr, s_red);  // barriers
        r = unit_records(li, a.pos[k].n_cls[CLS_NUCLEUS], a.ntiles, a.g_hist);
        hbase = a.hist2;
    } else {
        la = fu->la;
        r = rr;
        hbase = a.hist;
    }
    const int j0 = kNW - kPer * ((int)threadIdx.x + 1);  // this thread's lowest bucket
    uint64_t rel[kPer];
#pragma unroll
    for (int q = 0; q < kPer; q++) rel[q] = 0ull;
    for (int p = 0; p < r.count; p++) {
        // row-pass pieces hold the buckets [lo, hi] of their slot's range
        int lo = 0, hi = kNW - 1;
        if (!re) {
            const uint64_t rg = a.parts[r.first + p].keys[1];
            lo = (int)(uint32_t)(rg >> 32);
            hi = (int)(uint32_t)rg;
        }
        if (hi < j0 || lo > j0 + kPer - 1) continue;
        const uint64_t* h = hbase + (int64_t)(r.first + p) * kNW + j0;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            const int j = j0 + kPer - 1 - q;
            rel[q] += (j >= lo && j <= hi) ? h[kPer - 1 - q] : 0ull;
        }
    }
    double mine = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; q++)
        mine += nuc_scale(j0 + kPer - 1 - q) * ((double)rel[q] * kUnfix);
    double Z;
    const double excl0 = block_exclusive_scan(mine, s_tmp, &Z);
    const double target = (double)ri.top_p * Z;
    if (threadIdx.x == 0) *s_star = -1;
    __syncthreads();
    double run = excl0;
    int best = -1;
    double best_before = 0.0;
#pragma unroll
    for (int q = 0; q < kPer; q++) {
        const double m = nuc_scale(j0 + kPer - 1 - q) * ((double)rel[q] * kUnfix);
        if (rel[q] != 0ull && run < target) {
            best = (int)threadIdx.x * kPer + q;
            best_before = run;
        }
        run += m;
    }
    if (best >= 0) atomicMax(s_star, best);
    __syncthreads();
    const int star = *s_star;
    if (star >= 0 && best == star) {
        o->Z = Z;
        o->A = best_before;
        o->beta = kNW - 1 - star;
        o->la = la;
    }
    if (star < 0 && threadIdx.x == 0) o->beta = -1;
    if (star >= 0 && wave_id() < 2) {  // wave 0: the range's low end, wave 1: its high end
        const uint32_t im = nuc_first_image(kNW - 1 - star + wave_id(), la, bucket_coef(ri.T));
        if (lane_id() == 0) {
            if (wave_id() == 0)
                o->l_lo = ord_float(im);
            else
                o->l_hi = ord_float(im - 1u);
        }
    }
    __syncthreads();
}

// One workgroup per unit: the boundary bucket and its logit range.
__global__ __launch_bounds__(kThreads) void fn_select_kernel(StepArgs a, int k) {
    __shared__ double s_tmp[kWaves];
    __shared__ uint64_t s_red[kWaves];
    __shared__ SelOut s_sel;
    __shared__ int s_star;
    const int n = a.pos[k].n_cls[CLS_NUCLEUS];
    const int32_t* list = nuc_list(a, k);
    for (int li = blockIdx.x; li < n; li += gridDim.x) {
        const int u = list[li];
        unit_select(a, k, li, u, s_tmp, s_red, &s_star, &s_sel);  // barriers
        if (threadIdx.x == 0) {
            FnUnit* fu = a.fn_unit + u;
            const SelOut so = s_sel;
            if (so.beta >= 0) {
                fu->Z = so.Z;
                fu->A = so.A;
                fu->beta = so.beta;
                fu->la = so.la;
                fu->l_lo = so.l_lo;
                fu->l_hi = so.l_hi;
                fu->status = 0;
            } else {
                fu->status = 2;  // no finite logit: invalid row
            }
        }
        __syncthreads();  // s_sel is reused
    }
}

// Keys of the boundary bucket: the logits in [l_lo, l_hi].  Each workgroup
// gathers its piece's keys in LDS (one LDS counter update per wave and tile)
// and reserves space in the unit's list with one global atomic per piece.
// Keys beyond kCollectCap are dropped but still counted: such a bucket is
// resolved from the row itself.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_collect_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    static_assert(TS::kE <= 32, "hit mask is 32 bits");
    __shared__ uint64_t s_keys[kCollectCap];
    __shared__ int s_n, s_base;
    const int64_t T = (int64_t)a.pos[k].n_cls[CLS_NUCLEUS] * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    const int32_t* list = nuc_list(a, k);
    while (t < t_end) {
        const int li = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)li * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        t += tu1 - tu0;
        const int u = list[li];
        const int b = u >> 1, side = u & 1;
        FnUnit* fu = a.fn_unit + u;
        if (fu->status != 0) continue;  // uniform over the block
        const float l_lo = fu->l_lo, l_hi = fu->l_hi;
        if (threadIdx.x == 0) s_n = 0;
        __syncthreads();
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t t0, bool)
                                       __attribute__((always_inline)) {
            // past `end` elements read as -inf, below every boundary bucket
            uint32_t hit = 0u;
#pragma unroll
            for (int i = TS::kE - 1; i >= 0; i--)
                hit = (hit << 1) | (v[i] >= l_lo && v[i] <= l_hi ? 1u : 0u);
            if (__ballot(hit != 0u) == 0ull) return;
            int total;
            const int excl = wave_excl_count((uint32_t)__popc(hit), &total);
            int base = 0;
            if (lane_id() == 0) base = atomicAdd(&s_n, total);
            int slot = __builtin_amdgcn_readfirstlane(base) + excl;
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                if ((hit >> i) & 1u) {
                    if (slot < kCollectCap) s_keys[slot] = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
                    slot++;
                }
            }
        });
        __syncthreads();
        const int n = s_n;
        if (threadIdx.x == 0) s_base = n > 0 ? atomicAdd(&fu->ncoll, n) : 0;
        __syncthreads();
        const int nb = s_base;
        uint64_t* coll = a.coll + (int64_t)u * kCollectCap;
        for (int i = threadIdx.x; i < n && i < kCollectCap && nb + i < kCollectCap; i += kThreads)
            coll[nb + i] = s_keys[i];
        __syncthreads();  // s_keys and s_n are reused by the next piece
    }
}

// One workgroup per unit: the exact cut inside the boundary bucket.
//   1. the bucket's n tokens are split into 256 sub-buckets by the fraction
//      of their window coordinate (a finer cut of the same monotone map),
//      and the sub-bucket masses give the boundary sub-bucket the same way
//      the buckets gave the boundary bucket;
//   2. every token of the boundary sub-bucket is ranked implicitly: its
//      preceding mass is the bucket mass before the sub-bucket plus the
//      masses of the sub-bucket's tokens with a larger key.
// Inside the bucket every mass is an exact fixed-point integer scaled by the
// bucket's one factor, so these comparisons are exact up to that one product.
// The first token of the boundary sub-bucket is always kept (its preceding
// mass is below top_p Z by the choice of the sub-bucket), so the cut key tau
// lies in that sub-bucket.
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
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const uint64_t key = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
                if (key >= rlo && key <= rhi) {  // in the bucket (its keys form [lo, hi])
                    const int bin = (int)((key - rlo) >> s);
                    int bk;
                    const uint64_t w = nuc_wfix_t(nuc_t(v[i], la, cb), &bk);
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
            if (threadIdx.x == 0) fu->status = 1;
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
#pragma unroll
        for (int i = 0; i < TS::kE; i++) {
            const uint64_t key = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
            if (key >= rlo && key <= rhi) {
                const int slot = atomicAdd(&s_n, 1);
                if (slot < kThreads) {
                    int bk;
                    s_key[slot] = key;
                    s_w[slot] = nuc_wfix_t(nuc_t(v[i], la, cb), &bk);
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
        fu->tau = s_tau;
        fu->S = A + sc * (double)(pre + s_kept);
    }
    __syncthreads();
}

template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_resolve_kernel(StepArgs a, int k) {
    constexpr int kOwn = 4;  // boundary tokens a thread ranks per pass
    __shared__ uint64_t s_key[kCollectCap];
    __shared__ uint64_t s_w[kCollectCap];
    __shared__ uint16_t s_sel[kCollectCap];
    __shared__ uint8_t s_sb[kCollectCap];
    __shared__ uint64_t s_sub[kSub];
    __shared__ uint64_t s_tmp[kWaves];
    __shared__ unsigned long long s_tau, s_kept;
    __shared__ int s_star, s_nsel;
    __shared__ uint64_t s_before;
    static_assert(kBins <= kCollectCap && 2 * kBins * sizeof(uint32_t) <= sizeof(s_w) &&
                      kBins + kThreads <= kCollectCap,
                  "the wide path reuses s_key and s_w");
    const int n_units = a.pos[k].n_cls[CLS_NUCLEUS];
    const int32_t* list = nuc_list(a, k);
    for (int li = blockIdx.x; li < n_units; li += gridDim.x) {
        const int u = list[li];
        const int b = u >> 1;
        FnUnit* fu = a.fn_unit + u;
        const int status = fu->status;
        const int n = fu->ncoll;
        const float la = fu->la;
        const int beta = fu->beta;
        const double A = fu->A;
        const double target = (double)a.rows[b].top_p * fu->Z;
        __syncthreads();  // every thread has read fu before thread 0 may write it
        if (status != 0) continue;  // uniform over the block
        if (n < 1) {  // cannot happen: the boundary bucket has mass
            if (threadIdx.x == 0) fu->status = 1;
            continue;
        }
        const float cb = bucket_coef(a.rows[b].T);
        const double sc = nuc_scale(beta) * kUnfix;
        if (n > kCollectCap) {
            resolve_wide<DT, kAligned>(unit_row<DT>(a, b, u & 1, k), a.V, fu, la, cb, fu->l_lo,
                                       fu->l_hi, A, sc, target, s_key, reinterpret_cast<uint32_t*>(s_w),
                                       s_key + kBins, s_w + kBins, s_tmp);
            continue;
        }
        const uint64_t* coll = a.coll + (int64_t)u * kCollectCap;
        s_sub[threadIdx.x] = 0ull;
        if (threadIdx.x == 0) {
            s_tau = ~0ull;
            s_kept = 0ull;
            s_star = -1;
            s_nsel = 0;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kThreads) {
            const uint64_t key = coll[i];
            const float t = nuc_t(key_logit(key), la, cb);
            const float fr = t - floorf(t);
            // sub-buckets in ranking order: a larger fraction is a larger logit
            int sb = kSub - 1 - (int)(fr * (float)kSub);
            sb = sb < 0 ? 0 : (sb >= kSub ? kSub - 1 : sb);
            const uint64_t w = nuc_wrel(fr);
            s_key[i] = key;
            s_w[i] = w;
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
            if (threadIdx.x == 0) fu->status = 1;
            __syncthreads();
            continue;
        }
        for (int i = threadIdx.x; i < n; i += kThreads)
            if (s_sb[i] == star) s_sel[atomicAdd(&s_nsel, 1)] = (uint16_t)i;
        __syncthreads();
        const int nsel = s_nsel;
        const uint64_t before = s_before;
        for (int base = 0; base < nsel; base += kThreads * kOwn) {
            uint64_t key[kOwn], pre[kOwn];
#pragma unroll
            for (int q = 0; q < kOwn; q++) {
                const int i = base + q * kThreads + (int)threadIdx.x;
                key[q] = i < nsel ? s_key[s_sel[i]] : ~0ull;  // placeholder, never kept
                pre[q] = before;
            }
            for (int j = 0; j < nsel; j++) {
                const int sj = s_sel[j];
                const uint64_t kj = s_key[sj], wj = s_w[sj];
#pragma unroll
                for (int q = 0; q < kOwn; q++) pre[q] += kj > key[q] ? wj : 0ull;
            }
#pragma unroll
            for (int q = 0; q < kOwn; q++) {
                const int i = base + q * kThreads + (int)threadIdx.x;
                if (i < nsel && A + sc * (double)pre[q] < target) {
                    atomicMin(&s_tau, (unsigned long long)key[q]);
                    atomicAdd(&s_kept, (unsigned long long)s_w[s_sel[i]]);
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            fu->tau = s_tau;
            fu->S = A + sc * (double)(before + s_kept);
        }
        __syncthreads();
    }
}

}  // namespace sv
