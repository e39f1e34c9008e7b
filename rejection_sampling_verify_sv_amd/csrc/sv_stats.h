// sv_stats.h — acceptance statistics of one draft position.
//
// deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…": section
// "Örnekleme altında doğrulama yanlıştı" compares a check that draws one
// token from each model and accepts when they agree with the rejection test
// min(1, p / q); section "Kesme her iki tarafta eşleşmek zorunda" explains
// the remaining gap by the draft truncating (top_k, top_p) while the
// verification did not, and says the acceptance of the rejection test is
// the overlap of the two distributions.  For one row these are, with p, q
// the target and draft distributions after temperature and truncation and
// p~, q~ after temperature only:
//   [0]  sum_i min(p_i, q_i)     acceptance of the rejection test (a draft
//                                token x ~ q is kept with min(1, p(x)/q(x)),
//                                whose mean over x is this sum)
//   [1]  sum_i p_i q_i           probability that independent draws from p
//                                and q agree (the two-sample check)
//   [2]  sum_i min(p~_i, q_i)    the rejection test when only the draft
//                                truncates
//   [3]  sum_i min(p~_i, q~_i)   neither side truncates
// Greedy rows (T = 0) are 1 in every slot when the two argmaxes agree, else 0.
//
// After the row pass, the nucleus cut and an untruncated row pass over the
// same units (launched by sv_accept_stats):
//   stats_prep    one wave per row: the untruncated normalisers of both
//                 sides, the truncated distribution of each side as a key
//                 threshold and a scale (top-k list, nucleus cut, or none),
//                 greedy rows finished here;
//   stats_stream  the listed rows' tiles split evenly over the grid: per
//                 (row, tile, wave) the four partial sums, fp64;
//   stats_reduce  one wave per listed row: the partial sums in one fixed
//                 order.
#pragma once

#include "sv_decide.h"

namespace sv {

template <int DT>
__global__ __launch_bounds__(kThreads) void stats_prep_kernel(StepArgs a) {
    const int lane = lane_id();
    const int b = (int)blockIdx.x * kWaves + wave_id();
    if (b >= a.B) return;  // one wave per row, no barriers
    const RowInfo ri = a.rows[b];
    double* o = a.sout + (int64_t)b * 4;
    auto put = [&](double v) {
        if (lane == 0)
            for (int j = 0; j < 4; j++) o[j] = v;
    };
    const double nan = __longlong_as_double(0x7FF8000000000000ll);
    if (ri.cls < 0) {  // invalid parameters or an unsupported top_k
        put(nan);
        return;
    }
    const PosDesc P = a.pos[0];
    if (ri.cls == CLS_GREEDY) {
        uint64_t best[2];
        for (int s = 0; s < 2; s++) {
            const RecRange r = unit_records(
                P, unit_index(P, CLS_GREEDY, s == 0 ? ri.li_t : ri.li_d), a.ntiles, a.g_row);
            uint64_t m = 0ull;
            for (int i = lane; i < r.count; i += kWave) {
                const uint64_t k = a.parts[r.first + i].keys[0];
                m = k > m ? k : m;
            }
            best[s] = wave_max_u64(m);
        }
        put(key_id(best[0]) == key_id(best[1]) ? 1.0 : 0.0);
        return;
    }
    const double T = (double)ri.T, invT = 1.0 / T;
    const int nrec = a.ntiles * kWaves;
    double mt, zt, md, zd;  // untruncated (the forced untruncated row pass)
    full_stats(a.tstat + (int64_t)(2 * b) * nrec, nrec, invT, &mt, &zt);
    full_stats(a.tstat + (int64_t)(2 * b + 1) * nrec, nrec, invT, &md, &zd);
    if (!(mt > -INFINITY) || !(md > -INFINITY)) {
        put(nan);
        return;
    }
    StatDesc d;
    d.m_t = (float)mt;
    d.m_d = (float)md;
    d.c = exp2_coef(ri.T);
    d.iz_t = 1.0 / zt;
    d.iz_d = 1.0 / zd;
    d.pad = 0;
    if (ri.cls == CLS_FULL) {
        d.tau_t = d.tau_d = 0ull;
        d.kap_t = d.iz_t;
        d.kap_d = d.iz_d;
    } else if (ri.cls == CLS_TOPK) {
        // the kept tokens are a prefix of each ranked list: tau is the key of
        // its last one, the scale exp((m - l0) / T) over the kept mass
        for (int s = 0; s < 2; s++) {
            const uint64_t key = unit_top(
                a.parts, unit_records(P, unit_index(P, CLS_TOPK, s == 0 ? ri.li_t : ri.li_d),
                                      a.ntiles, a.g_row));
            double pr;
            bool keep;
            if (!topk_dist_wave(key, ri.k_eff, T, (double)ri.top_p, &pr, &keep)) {
                put(nan);
                return;
            }
            const int nk = __popcll(__ballot(keep));
            const uint64_t tau = lane_value(key, nk - 1);  // nk >= 1: the best token is kept
            const double l = (double)key_logit(key);
            const double l0 = lane_value(l, 0);
            const double zs = wave_sum(keep ? exp((l - l0) * invT) : 0.0);
            const double kap = exp(((s == 0 ? mt : md) - l0) * invT) / zs;
            if (s == 0) {
                d.tau_t = tau;
                d.kap_t = kap;
            } else {
                d.tau_d = tau;
                d.kap_d = kap;
            }
        }
    } else {  // nucleus: the cut of each unit
        const FnUnit ut = a.fn_unit[2 * b], ud = a.fn_unit[2 * b + 1];
        if (ut.status != 0 || ud.status != 0) {
            put(nan);
            return;
        }
        d.tau_t = ut.tau;
        d.tau_d = ud.tau;
        d.kap_t = exp((mt - (double)ut.la) * invT) / ut.S;
        d.kap_d = exp((md - (double)ud.la) * invT) / ud.S;
    }
    if (lane == 0) {
        a.sdesc[b] = d;
        a.slist[atomicAdd(&a.pos[a.K + 1].n_sample, 1)] = b;
    }
}

// The listed rows' tiles split evenly over the workgroups; every wave leaves
// its four partial sums of each tile at srec[((b*ntiles + tile)*kWaves + wave)*4].
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void stats_stream_kernel(StepArgs a) {
    using TS = TileShape<DT>;
    const int n = a.pos[a.K + 1].n_sample;
    const int64_t T = (int64_t)n * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    while (t < t_end) {
        const int si = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)si * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        t += tu1 - tu0;
        const int b = a.slist[si];
        const StatDesc d = a.sdesc[b];
        const void* trow = unit_row<DT>(a, b, 0, 0);
        const void* drow = unit_row<DT>(a, b, 1, 0);
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        double* out = a.srec + (int64_t)b * a.ntiles * kWaves * 4;
        stream_range2<DT, kAligned>(trow, drow, start, end,
                                    [&](float (&vt)[TS::kE], float (&vd)[TS::kE], int64_t t0,
                                        bool) __attribute__((always_inline)) {
            // elements past `end` read as -inf on both rows and weigh 0
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            uint32_t id0 = (uint32_t)elem_id<DT>(t0, 0);
            asm volatile("" : "+v"(id0));  // keeps 16-32 ids from being hoisted
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                constexpr int kVec = Elt<DT>::kVec;
                const uint32_t id = id0 + (uint32_t)((i / kVec) * kThreads * kVec + i % kVec);
                const double et = (double)fast_exp2((vt[i] - d.m_t) * d.c);
                const double ed = (double)fast_exp2((vd[i] - d.m_d) * d.c);
                const double pu = et * d.iz_t, qu = ed * d.iz_d;
                const double p = make_key(vt[i], id) >= d.tau_t ? et * d.kap_t : 0.0;
                const double q = make_key(vd[i], id) >= d.tau_d ? ed * d.kap_d : 0.0;
                s0 += p < q ? p : q;
                s1 += p * q;
                s2 += pu < q ? pu : q;
                s3 += pu < qu ? pu : qu;
                if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
            s0 = wave_sum(s0);
            s1 = wave_sum(s1);
            s2 = wave_sum(s2);
            s3 = wave_sum(s3);
            if (lane_id() == 0) {
                double* r = out + ((t0 / TS::kTile) * kWaves + wave_id()) * 4;
                r[0] = s0;
                r[1] = s1;
                r[2] = s2;
                r[3] = s3;
            }
        });
    }
}

// One wave per listed row: lane j adds the records j, j + 64, ... in order,
// then the fixed DPP tree.
__global__ __launch_bounds__(kThreads) void stats_reduce_kernel(StepArgs a) {
    const int si = (int)blockIdx.x * kWaves + wave_id();
    if (si >= a.pos[a.K + 1].n_sample) return;  // no barriers
    const int b = a.slist[si];
    const int nrec = a.ntiles * kWaves;
    const double* r = a.srec + (int64_t)b * nrec * 4;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    for (int i = lane_id(); i < nrec; i += kWave)
        for (int j = 0; j < 4; j++) s[j] += r[(int64_t)i * 4 + j];
    for (int j = 0; j < 4; j++) s[j] = wave_sum(s[j]);
    if (lane_id() == 0)
        for (int j = 0; j < 4; j++) a.sout[(int64_t)b * 4 + j] = s[j];
}

}  // namespace sv
