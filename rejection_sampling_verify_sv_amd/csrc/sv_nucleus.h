// sv_nucleus.h — the top_p cut over the whole vocabulary (top_k off).
//
// deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…", section
// "Kesme her iki tarafta eşleşmek zorunda": both distributions are cut to the
// smallest head of the ranking whose preceding mass stays below top_p.  With
// top_k disabled that head can hold tens of thousands of tokens, so the cut is
// located by mass instead of by sorting the row:
//
//   hist     every token's weight w = exp((l - m) / T) (m = row max) in 40-bit
//            fixed point, added into bucket floor(64 (m - l) / T); one
//            histogram per (unit, workgroup) piece, written without atomics;
//   select   per unit: sum the pieces, Z = total mass; the boundary bucket is
//            the last non-empty bucket whose preceding mass is below top_p Z;
//   collect  the keys of the boundary bucket's tokens (a bucket too large for
//            the workgroup's LDS is instead narrowed by a radix select
//            over its keys that re-reads the row, see resolve_wide);
//   resolve  per unit: a token of the boundary bucket is kept when the mass
//            before the bucket plus the mass of the bucket's tokens ranked
//            ahead of it (logit desc, id asc) is below top_p Z.  The cut key
//            tau (last kept token) and the kept mass S define the
//            distribution p(i) = [key_i >= tau] w_i / S.
// Fixed-point sums are exact, so the cut does not depend on the order of any
// addition.  The streaming passes split the tiles of position k's nucleus
// units evenly over the workgroups, like the row pass; the per-unit steps run
// one workgroup per unit.
#pragma once

#include "sv_decide.h"

namespace sv {

// Row max of one unit from its per-(tile, wave) row-pass records; every
// thread of the block gets it.  Contains barriers.
__device__ inline float block_unit_max(const FullStat* rec, int n, float* tmp /* kWaves */) {
    float m = -INFINITY;
    for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, rec[i].m);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    __syncthreads();
    if (lane_id() == 0) tmp[wave_id()] = m;
    __syncthreads();
    float r = tmp[0];
#pragma unroll
    for (int i = 1; i < kWaves; i++) r = fmaxf(r, tmp[i]);
    return r;
}

template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_hist_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    __shared__ uint64_t s_h[kNB];
    __shared__ float s_red[kWaves];
    const int nrec = a.ntiles * kWaves;
    const int64_t T = (int64_t)a.pos[k].n_fn * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
    while (t < t_end) {
        const int li = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)li * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        const int u = list[li];
        const int b = u >> 1, side = u & 1;
        for (int i = threadIdx.x; i < kNB; i += kThreads) s_h[i] = 0ull;
        const float m = block_unit_max(a.tstat + (int64_t)u * nrec, nrec, s_red);
        const float T_ = a.rows[b].T;
        const float c = exp2_coef(T_), cb = bucket_coef(T_);
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t, bool)
                                       __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const int bk = nuc_bucket(v[i], m, cb);
                const uint64_t wf = nuc_wfix(v[i], m, c);
                // elements past `end` read as -inf and land in the dropped bucket
                if (bk < kNB && wf != 0ull)
                    atomicAdd((unsigned long long*)&s_h[bk], (unsigned long long)wf);
            }
        });
        __syncthreads();
        uint64_t* out = a.hist + (int64_t)(li + blockIdx.x) * kNB;
        for (int i = threadIdx.x; i < kNB; i += kThreads) out[i] = s_h[i];
        t += tu1 - tu0;
        __syncthreads();  // s_h is cleared for the next piece
    }
}

// One workgroup per unit: total mass, boundary bucket and row max.
__global__ __launch_bounds__(kThreads) void fn_select_kernel(StepArgs a, int k) {
    constexpr int kPer = kNB / kThreads;  // contiguous buckets per thread
    __shared__ uint64_t s_tmp[kWaves];
    __shared__ float s_red[kWaves];
    __shared__ int s_beta;
    const int n = a.pos[k].n_fn;
    const int nrec = a.ntiles * kWaves;
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
    for (int li = blockIdx.x; li < n; li += gridDim.x) {
        const int u = list[li];
        const int b = u >> 1;
        const RecRange r = unit_records(li, n, a.ntiles, a.g_hist);
        const int b0 = threadIdx.x * kPer;
        uint64_t mass[kPer];
#pragma unroll
        for (int j = 0; j < kPer; j++) mass[j] = 0ull;
        for (int p = 0; p < r.count; p++) {
            const uint64_t* h = a.hist + (int64_t)(r.first + p) * kNB + b0;
#pragma unroll
            for (int j = 0; j < kPer; j++) mass[j] += h[j];
        }
        uint64_t mine = 0ull;
#pragma unroll
        for (int j = 0; j < kPer; j++) mine += mass[j];
        uint64_t Z;
        const uint64_t excl0 = block_exclusive_scan(mine, s_tmp, &Z);
        const double target = (double)a.rows[b].top_p * (double)Z;
        if (threadIdx.x == 0) s_beta = -1;
        __syncthreads();
        uint64_t run = excl0;
        int best = -1;
        uint64_t best_before = 0ull;
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            if (mass[j] != 0ull && (double)run < target) {
                best = b0 + j;
                best_before = run;
            }
            run += mass[j];
        }
        if (best >= 0) atomicMax(&s_beta, best);
        const float m = block_unit_max(a.tstat + (int64_t)u * nrec, nrec, s_red);  // barriers
        const int beta = s_beta;
        FnUnit* fu = a.fn_unit + u;
        if (beta >= 0 && best == beta) {
            fu->Zfix = Z;
            fu->Afix = best_before;
            fu->beta = beta;
            fu->m = m;
            fu->ncoll = 0;
            fu->status = 0;
        }
        if (beta < 0 && threadIdx.x == 0) {  // no finite logit: invalid row
            fu->status = 2;
            fu->ncoll = 0;
        }
        __syncthreads();
    }
}

// Keys of the boundary bucket.  Each workgroup gathers its piece's keys in
// LDS (one LDS counter update per wave and tile) and reserves space in the
// unit's list with one global atomic per piece.  Keys beyond kCollectCap are
// dropped but still counted: such a bucket is resolved from the row itself.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_collect_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    static_assert(TS::kE <= 32, "hit mask is 32 bits");
    __shared__ uint64_t s_keys[kCollectCap];
    __shared__ int s_n, s_base;
    const int64_t T = (int64_t)a.pos[k].n_fn * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
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
        if (threadIdx.x == 0) s_n = 0;
        __syncthreads();
        const int beta = fu->beta;
        const float m = fu->m;
        const float cb = bucket_coef(a.rows[b].T);
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t t0, bool)
                                       __attribute__((always_inline)) {
            // past `end` elements read as -inf and land in the dropped bucket
            uint32_t hit = 0u;
#pragma unroll
            for (int i = TS::kE - 1; i >= 0; i--)
                hit = (hit << 1) | (nuc_bucket(v[i], m, cb) == beta ? 1u : 0u);
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
//      of their bucket coordinate (a finer cut of the same monotone map), and
//      the sub-bucket masses give the boundary sub-bucket the same way the
//      buckets gave the boundary bucket;
//   2. every token of the boundary sub-bucket is ranked implicitly: its
//      preceding mass is the bucket mass before the sub-bucket plus the
//      masses of the sub-bucket's tokens with a larger key.
// The first token of the boundary sub-bucket is always kept (its preceding
// mass is below top_p Z by the choice of the sub-bucket), so the cut key tau
// lies in that sub-bucket.
constexpr int kSub = 256;
static_assert(kSub == kThreads, "one sub-bucket per thread");

// Boundary buckets of more than kCollectCap tokens (nearly flat rows, high
// temperatures) are resolved by the unit's workgroup alone, re-reading the
// row once per step of a radix select over the bucket's keys:
//   range  the bucket's keys form one interval [lo, hi] of the key order
//          (the bucket index never decreases as the logit falls, and equal
//          logits share a bucket); one pass finds it;
//   level  the interval is cut into at most kNB bins of 2^s consecutive
//          keys; one pass adds every token's fixed-point weight and a count
//          into its bin; the boundary bin is chosen as the boundary bucket
//          was (last bin with mass whose preceding mass is below top_p Z),
//          the mass of the bins ahead of it joins the mass before the
//          interval, and the interval shrinks to that bin;
//   rank   once the interval holds at most kThreads tokens (with 2^s = 1 it
//          holds one, as keys are distinct), they are ranked one per thread
//          like the boundary sub-bucket of the narrow path.
// The first token of every chosen bin is kept, so tau stays in the interval.
// Returns the cut key and the kept mass through fu.  Contains barriers; every
// thread of the block calls it.
template <int DT, bool kAligned>
__device__ void resolve_wide(const void* row, int64_t V, FnUnit* fu, float m, float c, float cb,
                             int beta, double target, uint64_t* s_mass /* kNB */,
                             uint32_t* s_cnt /* kNB */, uint64_t* s_key /* kThreads */,
                             uint64_t* s_w /* kThreads */, uint64_t* s_tmp /* kWaves */) {
    using TS = TileShape<DT>;
    constexpr int kPer = kNB / kThreads;  // bins per thread, in descending key order
    __shared__ unsigned long long s_lo, s_hi, s_tau, s_kept;
    __shared__ uint64_t s_A;
    __shared__ int s_star, s_n;
    __shared__ uint32_t s_bincnt;
    static_assert(kNB == 2048, "11-bit bins");
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
                if (nuc_bucket(v[i], m, cb) == beta) {
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
    uint64_t A = fu->Afix;
    for (;;) {
        // bin width 2^s with (rhi - rlo) >> s < kNB
        const uint64_t span = rhi - rlo;
        const int bits = span == 0ull ? 0 : 64 - __clzll((long long)span);
        const int s = bits > 11 ? bits - 11 : 0;
        for (int i = threadIdx.x; i < kNB; i += kThreads) {
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
                if (key >= rlo && key <= rhi) {
                    const int bin = (int)((key - rlo) >> s);
                    const uint64_t w = nuc_wfix(v[i], m, c);
                    if (w != 0ull) atomicAdd((unsigned long long*)&s_mass[bin], (unsigned long long)w);
                    atomicAdd(&s_cnt[bin], 1u);
                }
            }
        });
        __syncthreads();
        uint64_t mass[kPer];
        uint64_t mine = 0ull;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            mass[q] = s_mass[kNB - 1 - (threadIdx.x * kPer + q)];
            mine += mass[q];
        }
        uint64_t tot;
        uint64_t run = A + block_exclusive_scan(mine, s_tmp, &tot);
        int cand = -1;
        uint64_t cand_before = 0ull;
#pragma unroll
        for (int q = 0; q < kPer; q++) {
            if (mass[q] != 0ull && (double)run < target) {
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
            s_A = cand_before;
            s_bincnt = s_cnt[kNB - 1 - star];
        }
        __syncthreads();
        A = s_A;
        const uint32_t nbin = s_bincnt;
        const uint64_t j = (uint64_t)(kNB - 1 - star);
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
                    s_key[slot] = key;
                    s_w[slot] = nuc_wfix(v[i], m, c);
                }
            }
        }
    });
    __syncthreads();
    const int n = s_n < kThreads ? s_n : kThreads;
    if ((int)threadIdx.x < n) {
        const uint64_t key = s_key[threadIdx.x];
        uint64_t pre = 0ull;
        for (int j = 0; j < n; j++) pre += s_key[j] > key ? s_w[j] : 0ull;
        if ((double)(A + pre) < target) {
            atomicMin(&s_tau, (unsigned long long)key);
            atomicAdd(&s_kept, (unsigned long long)s_w[threadIdx.x]);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        fu->tau = s_tau;
        fu->Sfix = A + s_kept;
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
    const int n_units = a.pos[k].n_fn;
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
    for (int li = blockIdx.x; li < n_units; li += gridDim.x) {
        const int u = list[li];
        const int b = u >> 1;
        FnUnit* fu = a.fn_unit + u;
        const int status = fu->status;
        const int n = fu->ncoll;
        __syncthreads();  // every thread has read fu before thread 0 may write it
        if (status != 0) continue;  // uniform over the block
        if (n < 1) {  // cannot happen: the boundary bucket has mass
            if (threadIdx.x == 0) fu->status = 1;
            continue;
        }
        const float m = fu->m;
        const float T = a.rows[b].T;
        const float c = exp2_coef(T), cb = bucket_coef(T);
        if (n > kCollectCap) {
            resolve_wide<DT, kAligned>(unit_row<DT>(a, b, u & 1, k), a.V, fu, m, c, cb, fu->beta,
                                       (double)a.rows[b].top_p * (double)fu->Zfix, s_key,
                                       reinterpret_cast<uint32_t*>(s_w), s_key + kNB,
                                       s_w + kNB, s_tmp);
            continue;
        }
        const float beta = (float)fu->beta;
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
            const float l = key_logit(key);
            const uint64_t w = nuc_wfix(l, m, c);
            // same coordinate as nuc_bucket; its fraction in the bucket, in [0, 1)
            const float d = m - l;
            const float f = (d > 0.f ? d * cb : 0.f) - beta;
            int sb = (int)(f * (float)kSub);
            sb = sb < 0 ? 0 : (sb >= kSub ? kSub - 1 : sb);
            s_key[i] = key;
            s_w[i] = w;
            s_sb[i] = (uint8_t)sb;
            atomicAdd((unsigned long long*)&s_sub[sb], (unsigned long long)w);
        }
        __syncthreads();
        const double target = (double)a.rows[b].top_p * (double)fu->Zfix;
        const uint64_t A = fu->Afix;
        {
            const uint64_t mine = s_sub[threadIdx.x];
            uint64_t tot;
            const uint64_t before = block_exclusive_scan(mine, s_tmp, &tot);
            const bool cand = mine != 0ull && (double)(A + before) < target;
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
        const uint64_t A2 = A + s_before;
        for (int base = 0; base < nsel; base += kThreads * kOwn) {
            uint64_t key[kOwn], pre[kOwn];
#pragma unroll
            for (int q = 0; q < kOwn; q++) {
                const int i = base + q * kThreads + (int)threadIdx.x;
                key[q] = i < nsel ? s_key[s_sel[i]] : ~0ull;  // placeholder, never kept
                pre[q] = 0ull;
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
                if (i < nsel && (double)(A2 + pre[q]) < target) {
                    atomicMin(&s_tau, (unsigned long long)key[q]);
                    atomicAdd(&s_kept, (unsigned long long)s_w[s_sel[i]]);
                }
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            fu->tau = s_tau;
            fu->Sfix = A2 + s_kept;
        }
        __syncthreads();
    }
}

}  // namespace sv
