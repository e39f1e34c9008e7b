// sv_nucleus.h — the exact top_p cut over the whole vocabulary (top_k off).
//
// deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…", section
// "Kesme her iki tarafta eşleşmek zorunda": both distributions are cut to the
// smallest head of the ranking whose preceding mass stays below top_p.  With
// top_k disabled that head can hold tens of thousands of tokens, so the cut is
// located by mass instead of by sorting:
//
//   masses  w = exp((l - m) / T), m = the row max, z = (m - l) / T >= 0.
//           Bucket b = floor(32 z) (z < 64; larger z is a tail whose total
//           mass, below V * e^-64, is dropped).  Inside a bucket
//           w = e^(-b/32) * e^(-d) with d = z - b/32 in [0, 1/32), so every
//           bucket's mass is e^(-b/32) times a sum of e^(-d) terms, each in
//           (0.969, 1], evaluated by a degree-8 Taylor polynomial (truncation
//           below 1e-19).  The sums are kept in 80-bit fixed point (two 64-bit
//           integer words at 2^-40 and 2^-80 per unit), so the histogram is
//           exact up to the term rounding and independent of the order in
//           which workgroups add into it.
//   select  Z = total mass; the boundary bucket is the last non-empty bucket
//           whose preceding mass is still below top_p * Z.
//   collect the keys of the boundary bucket's tokens.
//   resolve sort them by (logit desc, id asc), walk the running mass and keep
//           tokens while the preceding mass is below top_p * Z.  The cut key
//           tau (last kept token) and the kept mass Z_S define the
//           distribution: p(i) = [key_i >= tau] w_i / Z_S.
// The streaming passes split the tiles of position k's nucleus units evenly
// over the workgroups, like the row pass; the per-unit steps run one
// workgroup per unit.
#pragma once

#include "sv_decide.h"

namespace sv {

struct FnWork {
    uint64_t* hi;    // [2B][kNB]
    uint64_t* lo;    // [2B][kNB]
    uint32_t* cnt;   // [2B][kNB]
    uint64_t* coll;  // [2B][kCollectCap]
};

// Row max of unit (b, side) at position k from its row-pass records.
__device__ inline float unit_max(const StepArgs& a, int b, int side, int k) {
    const int li = side == 0 ? a.rows[b].li_t : a.rows[b].li_d;
    const RecRange r = unit_records(li, a.pos[k].n_units, a.ntiles);
    float m = -INFINITY;
    for (int s = 0; s < r.count; s++)
        m = fmaxf(m, reinterpret_cast<const FullStat*>(a.parts + r.first + s)->m);
    return m;
}

// Zero the histograms of the nucleus units of position 0 (every nucleus row).
__global__ __launch_bounds__(kThreads) void fn_zero_kernel(StepArgs a, FnWork w) {
    const int n = a.pos[0].n_fn;
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
        const int u = a.flist[i];
        for (int j = threadIdx.x; j < kNB; j += kThreads) {
            w.hi[(int64_t)u * kNB + j] = 0ull;
            w.lo[(int64_t)u * kNB + j] = 0ull;
            w.cnt[(int64_t)u * kNB + j] = 0u;
        }
    }
}

template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_hist_kernel(StepArgs a, FnWork w, int k) {
    using TS = TileShape<DT>;
    __shared__ uint64_t s_hi[kNB];
    __shared__ uint64_t s_lo[kNB];
    __shared__ uint32_t s_cnt[kNB];
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
        for (int i = threadIdx.x; i < kNB; i += kThreads) {
            s_hi[i] = 0ull;
            s_lo[i] = 0ull;
            s_cnt[i] = 0u;
        }
        __syncthreads();
        const float m = unit_max(a, b, side, k);
        const double invT = 1.0 / (double)a.rows[b].T;
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t t0, bool full) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                if (!full && elem_id<DT>(t0, i) >= end) continue;
                double d;
                const int bk = fn_bucket(v[i], m, invT, &d);
                if (bk >= kNB) continue;
                uint64_t h, l;
                fixed80(exp_neg_small(d), &h, &l);
                atomicAdd((unsigned long long*)&s_hi[bk], (unsigned long long)h);
                atomicAdd((unsigned long long*)&s_lo[bk], (unsigned long long)l);
                atomicAdd(&s_cnt[bk], 1u);
            }
        });
        __syncthreads();
        for (int i = threadIdx.x; i < kNB; i += kThreads) {
            if (s_cnt[i] == 0u) continue;
            atomicAdd((unsigned long long*)&w.hi[(int64_t)u * kNB + i],
                      (unsigned long long)s_hi[i]);
            atomicAdd((unsigned long long*)&w.lo[(int64_t)u * kNB + i],
                      (unsigned long long)s_lo[i]);
            atomicAdd(&w.cnt[(int64_t)u * kNB + i], s_cnt[i]);
        }
        t += tu1 - tu0;
        __syncthreads();
    }
}

// One workgroup per unit: total mass and the boundary bucket.
__global__ __launch_bounds__(kThreads) void fn_select_kernel(StepArgs a, FnWork w, int k) {
    constexpr int kPer = kNB / kThreads;  // contiguous buckets per thread
    __shared__ double s_tmp[kWaves];
    __shared__ int s_beta;
    const int n = a.pos[k].n_fn;
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
    for (int li = blockIdx.x; li < n; li += gridDim.x) {
        const int u = list[li];
        const int b = u >> 1, side = u & 1;
        double mass[kPer];
        double mine = 0.0;
        const int b0 = threadIdx.x * kPer;
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const int bk = b0 + j;
            mass[j] = unfixed80(w.hi[(int64_t)u * kNB + bk], w.lo[(int64_t)u * kNB + bk]) * a.ebk[bk];
            mine += mass[j];
        }
        double Z;
        const double excl0 = block_exclusive_scan(mine, s_tmp, &Z);
        const double target = (double)a.rows[b].top_p * Z;
        if (threadIdx.x == 0) s_beta = -1;
        __syncthreads();
        double run = excl0;
        int best = -1;
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const int bk = b0 + j;
            if (w.cnt[(int64_t)u * kNB + bk] > 0u && run < target) best = bk;
            run += mass[j];
        }
        if (best >= 0) atomicMax(&s_beta, best);
        __syncthreads();
        const int beta = s_beta;
        FnUnit& fu = a.fn_unit[u];
        if (beta >= b0 && beta < b0 + kPer) {
            double before = excl0;
#pragma unroll
            for (int j = 0; j < kPer; j++)
                if (j < beta - b0) before += mass[j];
            fu.Z = Z;
            fu.Mabove = before;
            fu.beta = beta;
            fu.count = (int)w.cnt[(int64_t)u * kNB + beta];
            fu.ncoll = 0;
            fu.status = 0;
            fu.m = unit_max(a, b, side, k);
        }
        if (beta < 0 && threadIdx.x == 0) {  // no finite logit: invalid row
            fu.status = 2;
            fu.ncoll = 0;
        }
        __syncthreads();
    }
}

template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void fn_collect_kernel(StepArgs a, FnWork w, int k) {
    using TS = TileShape<DT>;
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
        if (fu->status != 0) continue;
        const int beta = fu->beta;
        const float m = fu->m;
        const double invT = 1.0 / (double)a.rows[b].T;
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        uint64_t* coll = w.coll + (int64_t)u * kCollectCap;
        stream_range<DT, kAligned>(unit_row<DT>(a, b, side, k), start, end,
                                   [&](float (&v)[TS::kE], int64_t t0, bool full) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const int64_t id = elem_id<DT>(t0, i);
                if (!full && id >= end) continue;
                double d;
                if (fn_bucket(v[i], m, invT, &d) != beta) continue;
                const int slot = atomicAdd(&fu->ncoll, 1);
                if (slot < kCollectCap) coll[slot] = make_key(v[i], (uint32_t)id);
            }
        });
    }
}

// One workgroup per unit: exact cut inside the boundary bucket.  Always
// clears the unit's histogram for the next position.
__global__ __launch_bounds__(kThreads) void fn_resolve_kernel(StepArgs a, FnWork w, int k) {
    __shared__ uint64_t s_key[kCollectCap];
    __shared__ double s_tmp[kWaves];
    __shared__ int s_keep;
    const int n_units = a.pos[k].n_fn;
    const int32_t* list = a.flist + (int64_t)k * 2 * a.B;
    for (int li = blockIdx.x; li < n_units; li += gridDim.x) {
        const int u = list[li];
        const int b = u >> 1;
        FnUnit* fu = a.fn_unit + u;
        const int status = fu->status;
        const int n = fu->ncoll;
        const bool ok = status == 0 && n <= kCollectCap && n >= 1;
        if (ok) {
            const int P = pow2_ceil(n < 2 ? 2 : n);
            const uint64_t* coll = w.coll + (int64_t)u * kCollectCap;
            for (int i = threadIdx.x; i < P; i += kThreads) s_key[i] = (i < n) ? coll[i] : 0ull;
            __syncthreads();
            block_sort_desc(s_key, P);
            const double invT = 1.0 / (double)a.rows[b].T;
            const float m = fu->m;
            const double target = (double)a.rows[b].top_p * fu->Z;
            const double Mabove = fu->Mabove;
            // every collected token sits in the boundary bucket: w = e^(-beta/32) e^(-d)
            const double eb = a.ebk[fu->beta];
            // thread t owns sorted positions [t*kPer, (t+1)*kPer)
            constexpr int kPer = kCollectCap / kThreads;
            const int j0 = threadIdx.x * kPer;
            double wv[kPer];
            double mine = 0.0;
#pragma unroll
            for (int q = 0; q < kPer; q++) {
                double d;
                const int j = j0 + q;
                wv[q] = 0.0;
                if (j < n) {
                    (void)fn_bucket(key_logit(s_key[j]), m, invT, &d);
                    wv[q] = eb * exp_neg_small(d);
                }
                mine += wv[q];
            }
            double tot;
            const double excl = block_exclusive_scan(mine, s_tmp, &tot);
            if (threadIdx.x == 0) s_keep = 0;
            __syncthreads();
            double cum = Mabove + excl;
            int keep_here = 0;
#pragma unroll
            for (int q = 0; q < kPer; q++) {
                if (j0 + q < n && cum < target) keep_here = j0 + q + 1;
                cum += wv[q];
            }
            if (keep_here > 0) atomicMax(&s_keep, keep_here);
            __syncthreads();
            const int nk = s_keep;  // >= 1: the first token's preceding mass is below target
            double kept = 0.0;
#pragma unroll
            for (int q = 0; q < kPer; q++)
                if (j0 + q < nk) kept += wv[q];
            double ktot;
            (void)block_exclusive_scan(kept, s_tmp, &ktot);
            if (threadIdx.x == 0) {
                if (nk < 1) {
                    fu->status = 1;
                } else {
                    fu->tau = s_key[nk - 1];
                    fu->Zs = Mabove + ktot;
                }
            }
        } else if (threadIdx.x == 0 && status == 0) {
            fu->status = 1;  // boundary bucket larger than kCollectCap
        }
        for (int i = threadIdx.x; i < kNB; i += kThreads) {
            w.hi[(int64_t)u * kNB + i] = 0ull;
            w.lo[(int64_t)u * kNB + i] = 0ull;
            w.cnt[(int64_t)u * kNB + i] = 0u;
        }
        __syncthreads();
    }
}

}  // namespace sv
