// sv_decide.h — per-row decision at one draft position.
//
// After the row pass of position k, one workgroup per live row:
//   * merges the segment records of the target (and draft) row;
//   * top-k rows: sorts the <= 64 survivors, applies temperature, the top_p
//     walk over the renormalised top-k and renormalisation, all in fp64 and
//     in the same summation order as the definition; then runs the accept
//     test and, if the row ends here, the residual or bonus draw over the
//     <= 64 kept tokens in ascending id order;
//   * greedy rows: compares the draft token with the target argmax;
//   * full-vocab rows: forms p(x), q(x) from {max, sum-exp} and the two
//     gathered logits, runs the accept test and, if the row ends here, hands
//     the draw to the full-vocab sampler (sv_sample.h).
//
// Rule sources: deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…",
// sections "Örnekleme altında doğrulama yanlıştı" (greedy check; accept with
// min(1, p/q); residual draw) and "Kesme her iki tarafta eşleşmek zorunda"
// (same truncation on both sides); tinycto.tv "Spekülatif Kod Çözme…",
// section "1. Temel Çalışma Mekanizması" (first rejection ends the row).
#pragma once

#include "sv_device.h"
#include "sv_rowpass.h"

namespace sv {

struct StepArgs {
    const void* target;
    const void* draft;
    int64_t t_stride, d_stride;
    int K, V, nseg, nch;
    const int32_t* tokens;
    const float* uniforms;
    RowInfo* rows;
    const PartSlot* parts;
    double2* chunks;
    int32_t* out_tokens;
    int32_t* out_acc;
    double* diag;
    FnUnit* fn_unit;    // [B*2] nucleus cut of the current position
    const double* ebk;  // [kNB] e^(-b/32)
};

__device__ inline void diag_nan_row(double* diag, int b, int K) {
    if (!diag) return;
    double* d = diag + (int64_t)b * 4 * (K + 1);
    for (int i = threadIdx.x; i < 4 * (K + 1); i += kThreads) d[i] = __longlong_as_double(0x7FF8000000000000ll);
}

// Single thread: write accepted drafts + final token, close the row.
__device__ inline void emit_row(const StepArgs& a, int b, int acc, int y) {
    int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
    const int32_t* t = a.tokens + (int64_t)b * a.K;
    for (int j = 0; j < acc; j++) o[j] = t[j];
    o[acc] = y;
    a.out_acc[b] = acc;
    a.rows[b].acc = acc;
    a.rows[b].status = ST_DONE;
}

__device__ inline void fail_row(const StepArgs& a, int b) {
    // every thread of the block calls this (uniform)
    diag_nan_row(a.diag, b, a.K);
    if (threadIdx.x == 0) {
        int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
        for (int j = 0; j <= a.K; j++) o[j] = -1;
        a.out_acc[b] = -1;
        a.rows[b].status = ST_ERROR;
    }
}

// Row the build does not serve (boundary bucket over capacity): -2.
__device__ inline void unsup_row(const StepArgs& a, int b) {
    diag_nan_row(a.diag, b, a.K);
    if (threadIdx.x == 0) {
        int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
        for (int j = 0; j <= a.K; j++) o[j] = -1;
        a.out_acc[b] = -2;
        a.rows[b].status = ST_ERROR;
    }
}

// Inverse CDF over n weights listed in ascending id order (single thread).
// Returns the index of the first positive weight whose running sum exceeds
// u * W; writes the bin edges as fractions of W and the margin of u.
__device__ inline int invcdf_small(const double* w, int n, double u, double* lo, double* hi,
                                   double* margin, double* Wout) {
    double W = 0.0;
    for (int j = 0; j < n; j++) W += w[j];
    *Wout = W;
    const double target = u * W;
    double S = 0.0, last_before = 0.0;
    int last = -1;
    for (int j = 0; j < n; j++) {
        if (!(w[j] > 0.0)) continue;
        const double before = S;
        S += w[j];
        last = j;
        last_before = before;
        if (target < S) {
            *lo = before / W;
            *hi = S / W;
            const double d1 = u - *lo, d2 = *hi - u;
            *margin = d1 < d2 ? d1 : d2;
            return j;
        }
    }
    *lo = last_before / W;
    *hi = 1.0;
    *margin = 0.0;
    return last;
}

struct TopkDecideSmem {
    uint64_t buf[64 * kMaxTopK];
    uint64_t top[2][kMaxTopK];
    double w[2][kMaxTopK];
    double prob[2][kMaxTopK];
    int id[2][kMaxTopK];
    int keep[2];
    // residual / bonus, ascending id
    double sw[kMaxTopK];
    double sp[kMaxTopK];
    int sid[kMaxTopK];
    int err;
};

// Merge nseg descending lists of one side into the block-wide top k_eff.
__device__ inline void merge_side(TopkDecideSmem& sm, const PartSlot* slots, int nseg, int k_eff,
                                  int side) {
    if (nseg == 1) {
        for (int i = threadIdx.x; i < k_eff; i += kThreads) sm.top[side][i] = slots[0].keys[i];
        __syncthreads();
        return;
    }
    const int n = nseg * k_eff;
    const int P = pow2_ceil(n);
    for (int i = threadIdx.x; i < P; i += kThreads) {
        uint64_t key = 0ull;
        if (i < n) key = slots[i / k_eff].keys[i % k_eff];
        sm.buf[i] = key;
    }
    __syncthreads();
    block_sort_desc(sm.buf, P);
    for (int i = threadIdx.x; i < k_eff; i += kThreads) sm.top[side][i] = sm.buf[i];
    __syncthreads();
}

// Wave 0 builds the truncated distribution of one side from its sorted keys.
__device__ inline void topk_dist(TopkDecideSmem& sm, int side, int k_eff, double T, double top_p) {
    const int lane = threadIdx.x;
    if (lane < kWave) {
        const double l0 = (double)key_logit(sm.top[side][0]);
        if (lane < k_eff) {
            const uint64_t key = sm.top[side][lane];
            const double l = (double)key_logit(key);
            sm.w[side][lane] = exp((l - l0) / T);
            sm.id[side][lane] = (int)key_id(key);
        }
        if (lane == 0 && !(l0 > -INFINITY)) sm.err = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0 && !sm.err) {
        const double* w = sm.w[side];
        double zk = 0.0;
        for (int j = 0; j < k_eff; j++) zk += w[j];
        int keep = k_eff;
        if (top_p < 1.0) {
            double cum = 0.0;
            keep = 0;
            while (keep < k_eff && cum < top_p) {
                cum += w[keep] / zk;
                keep++;
            }
        }
        double zs = 0.0;
        for (int j = 0; j < keep; j++) zs += w[j];
        for (int j = 0; j < k_eff; j++) sm.prob[side][j] = (j < keep) ? w[j] / zs : 0.0;
        sm.keep[side] = keep;
    }
    __syncthreads();
}

__device__ inline double lookup_prob(const TopkDecideSmem& sm, int side, int token) {
    double p = 0.0;
    for (int j = 0; j < sm.keep[side]; j++)
        if (sm.id[side][j] == token) p = sm.prob[side][j];
    return p;
}

__device__ void decide_topk(const StepArgs& a, int b, int k, const RowInfo& ri) {
    __shared__ TopkDecideSmem sm;
    const int k_eff = ri.k_eff;
    const double T = (double)ri.T, top_p = (double)ri.top_p;
    const bool has_draft = k < ri.L;
    if (threadIdx.x == 0) sm.err = 0;
    const PartSlot* base = a.parts + (int64_t)b * 2 * a.nseg;
    merge_side(sm, base, a.nseg, k_eff, 0);
    if (has_draft) merge_side(sm, base + a.nseg, a.nseg, k_eff, 1);
    topk_dist(sm, 0, k_eff, T, top_p);
    if (has_draft) topk_dist(sm, 1, k_eff, T, top_p);
    if (sm.err) {
        fail_row(a, b);
        return;
    }
    const float* u = a.uniforms + (int64_t)b * (a.K + 1);
    double* dg = a.diag ? a.diag + (int64_t)b * 4 * (a.K + 1) : nullptr;
    bool final_draw = true;
    bool use_resid = false;
    if (has_draft) {
        __shared__ int s_accept;
        if (threadIdx.x == 0) {
            const int x = a.tokens[(int64_t)b * a.K + k];
            const double px = lookup_prob(sm, 0, x), qx = lookup_prob(sm, 1, x);
            double acc;
            if (qx > 0.0) {
                acc = px / qx;
                if (acc > 1.0) acc = 1.0;
            } else {
                acc = (px > 0.0) ? 1.0 : 0.0;
            }
            const double uk = (double)u[k];
            if (dg) {
                dg[4 * k + 0] = px;
                dg[4 * k + 1] = qx;
                dg[4 * k + 2] = acc;
                dg[4 * k + 3] = fabs(uk - acc);
            }
            s_accept = uk < acc;
            if (s_accept) a.rows[b].acc = k + 1;
        }
        __syncthreads();
        if (s_accept) return;
        use_resid = true;
    }
    if (!final_draw) return;
    // weights over p's kept set in ascending id order (rank by id)
    const int kp = sm.keep[0];
    if (threadIdx.x < kp) {
        const int j = threadIdx.x;
        const int id = sm.id[0][j];
        int rank = 0;
        for (int i = 0; i < kp; i++) rank += sm.id[0][i] < id;
        const double pj = sm.prob[0][j];
        double wj = pj;
        if (use_resid) {
            const double qj = lookup_prob(sm, 1, id);
            const double d = pj - qj;
            wj = d > 0.0 ? d : 0.0;
        }
        sm.sid[rank] = id;
        sm.sw[rank] = wj;
        sm.sp[rank] = pj;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const double uf = (double)u[a.K];
        double lo, hi, mg, W;
        const double* w = sm.sw;
        if (use_resid) {
            double Wr = 0.0;
            for (int j = 0; j < kp; j++) Wr += sm.sw[j];
            if (!(Wr > 0.0)) w = sm.sp;
        }
        const int j = invcdf_small(w, kp, uf, &lo, &hi, &mg, &W);
        const int y = sm.sid[j];
        if (dg) {
            dg[4 * a.K + 0] = use_resid ? w[j] / W : sm.sp[j];
            dg[4 * a.K + 1] = lo;
            dg[4 * a.K + 2] = hi;
            dg[4 * a.K + 3] = mg;
        }
        emit_row(a, b, k, y);
    }
}

__device__ void decide_greedy(const StepArgs& a, int b, int k, const RowInfo& ri) {
    if (threadIdx.x != 0) return;
    const PartSlot* base = a.parts + (int64_t)b * 2 * a.nseg;
    uint64_t best = 0ull;
    for (int s = 0; s < a.nseg; s++) best = base[s].keys[0] > best ? base[s].keys[0] : best;
    const int g = (int)key_id(best);
    if (k < ri.L && a.tokens[(int64_t)b * a.K + k] == g) {
        a.rows[b].acc = k + 1;
        return;
    }
    emit_row(a, b, k, g);
}

// {max, sum-exp} of one full-vocab row from its segment records.
__device__ inline void full_stats(const PartSlot* slots, int nseg, double invT, double* m,
                                  double* z) {
    float mm = -INFINITY;
    double ss = 0.0;
    for (int s = 0; s < nseg; s++) {
        const FullStat* fs = reinterpret_cast<const FullStat*>(slots + s);
        ms_combine(mm, ss, fs->m, fs->s, invT);
    }
    *m = (double)mm;
    *z = ss;
}

template <int DT>
__device__ void decide_full(const StepArgs& a, int b, int k, const RowInfo& ri) {
    __shared__ int s_fail;
    if (threadIdx.x == 0) {
        s_fail = 0;
        const double T = (double)ri.T, invT = 1.0 / T;
        const PartSlot* base = a.parts + (int64_t)b * 2 * a.nseg;
        double mt, zt, md = 0.0, zd = 0.0;
        full_stats(base, a.nseg, invT, &mt, &zt);
        RowInfo& w = a.rows[b];
        if (!(mt > -INFINITY)) {
            s_fail = 1;
        } else if (k == ri.L) {
            w.need = NEED_BONUS;
            w.kpos = k;
            w.mt = mt;
            w.zt = zt;
            w.status = ST_SAMPLE;
        } else {
            full_stats(base + a.nseg, a.nseg, invT, &md, &zd);
            if (!(md > -INFINITY)) {
                s_fail = 1;
            } else {
                const int x = a.tokens[(int64_t)b * a.K + k];
                const char* trow = static_cast<const char*>(a.target) +
                                   ((int64_t)b * (a.K + 1) + k) * a.t_stride * Elt<DT>::kSize;
                const char* drow = static_cast<const char*>(a.draft) +
                                   ((int64_t)b * a.K + k) * a.d_stride * Elt<DT>::kSize;
                const double lx = (double)load_one<DT>(trow, x);
                const double ld = (double)load_one<DT>(drow, x);
                const double px = exp((lx - mt) / T) / zt;
                const double qx = exp((ld - md) / T) / zd;
                double acc;
                if (qx > 0.0) {
                    acc = px / qx;
                    if (acc > 1.0) acc = 1.0;
                } else {
                    acc = (px > 0.0) ? 1.0 : 0.0;
                }
                const double uk = (double)a.uniforms[(int64_t)b * (a.K + 1) + k];
                if (a.diag) {
                    double* dg = a.diag + (int64_t)b * 4 * (a.K + 1);
                    dg[4 * k + 0] = px;
                    dg[4 * k + 1] = qx;
                    dg[4 * k + 2] = acc;
                    dg[4 * k + 3] = fabs(uk - acc);
                }
                if (uk < acc) {
                    w.acc = k + 1;
                } else {
                    w.need = NEED_RESID;
                    w.kpos = k;
                    w.mt = mt;
                    w.zt = zt;
                    w.md = md;
                    w.zd = zd;
                    w.status = ST_SAMPLE;
                }
            }
        }
    }
    __syncthreads();
    if (s_fail) fail_row(a, b);
}

// Nucleus rows: p(x) = [key(x) >= tau] w(x) / Z_S with the exact masses of
// the cut computed by the nucleus kernels for this position.
template <int DT>
__device__ void decide_nucleus(const StepArgs& a, int b, int k, const RowInfo& ri) {
    __shared__ int s_fail;  // 0 ok, 1 invalid data, 2 not served
    if (threadIdx.x == 0) {
        s_fail = 0;
        const double invT = 1.0 / (double)ri.T;
        const FnUnit ut = a.fn_unit[b * 2];
        RowInfo& w = a.rows[b];
        if (ut.status != 0) {
            s_fail = ut.status == 1 ? 2 : 1;
        } else if (k == ri.L) {
            w.need = NEED_BONUS;
            w.kpos = k;
            w.mt = (double)ut.m;
            w.zt = ut.Zs;
            w.tau_t = ut.tau;
            w.status = ST_SAMPLE;
        } else {
            const FnUnit ud = a.fn_unit[b * 2 + 1];
            if (ud.status != 0) {
                s_fail = ud.status == 1 ? 2 : 1;
            } else {
                const int x = a.tokens[(int64_t)b * a.K + k];
                const char* trow = static_cast<const char*>(a.target) +
                                   ((int64_t)b * (a.K + 1) + k) * a.t_stride * Elt<DT>::kSize;
                const char* drow = static_cast<const char*>(a.draft) +
                                   ((int64_t)b * a.K + k) * a.d_stride * Elt<DT>::kSize;
                const float lx = load_one<DT>(trow, x);
                const float ld = load_one<DT>(drow, x);
                const double px = (make_key(lx, (uint32_t)x) >= ut.tau)
                                      ? fn_weight(lx, ut.m, invT, a.ebk) / ut.Zs : 0.0;
                const double qx = (make_key(ld, (uint32_t)x) >= ud.tau)
                                      ? fn_weight(ld, ud.m, invT, a.ebk) / ud.Zs : 0.0;
                double acc;
                if (qx > 0.0) {
                    acc = px / qx;
                    if (acc > 1.0) acc = 1.0;
                } else {
                    acc = (px > 0.0) ? 1.0 : 0.0;
                }
                const double uk = (double)a.uniforms[(int64_t)b * (a.K + 1) + k];
                if (a.diag) {
                    double* dg = a.diag + (int64_t)b * 4 * (a.K + 1);
                    dg[4 * k + 0] = px;
                    dg[4 * k + 1] = qx;
                    dg[4 * k + 2] = acc;
                    dg[4 * k + 3] = fabs(uk - acc);
                }
                if (uk < acc) {
                    w.acc = k + 1;
                } else {
                    w.need = NEED_RESID;
                    w.kpos = k;
                    w.mt = (double)ut.m;
                    w.zt = ut.Zs;
                    w.tau_t = ut.tau;
                    w.md = (double)ud.m;
                    w.zd = ud.Zs;
                    w.tau_d = ud.tau;
                    w.status = ST_SAMPLE;
                }
            }
        }
    }
    __syncthreads();
    if (s_fail == 1)
        fail_row(a, b);
    else if (s_fail == 2)
        unsup_row(a, b);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void decide_kernel(StepArgs a, int k) {
    const int b = blockIdx.x;
    const RowInfo ri = a.rows[b];
    if (ri.status != ST_LIVE || k > ri.L) return;
    if (ri.cls == CLS_GREEDY)
        decide_greedy(a, b, k, ri);
    else if (ri.cls == CLS_TOPK)
        decide_topk(a, b, k, ri);
    else if (ri.cls == CLS_NUCLEUS)
        decide_nucleus<DT>(a, b, k, ri);
    else
        decide_full<DT>(a, b, k, ri);
}

// Row classification and output initialisation (one thread per row).
// A row is invalid when T is negative, NaN or infinite, top_p is not > 0,
// draft_len is outside [0, K] or a read draft token is outside [0, V).
__global__ __launch_bounds__(kThreads) void plan_kernel(StepArgs a, int B, const int32_t* draft_len,
                                                        const sv_sampler_params* params) {
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= B) return;
    const sv_sampler_params prm = params[b];
    const int L = draft_len ? draft_len[b] : a.K;
    const float T = prm.temperature, tp = prm.top_p;
    const int tk = prm.top_k;
    bool bad = !(T >= 0.f) || !(T < INFINITY) || !(tp > 0.f) || L < 0 || L > a.K;
    if (!bad) {
        for (int j = 0; j < L; j++) {
            const int t = a.tokens[(int64_t)b * a.K + j];
            if (t < 0 || t >= a.V) bad = true;
        }
    }
    int cls;
    if (bad)
        cls = CLS_ERROR;
    else if (T == 0.f)
        cls = CLS_GREEDY;
    else if (tk > 0 && tk < a.V)
        cls = (tk <= kMaxTopK) ? CLS_TOPK : CLS_UNSUP;
    else
        cls = (tp < 1.f) ? CLS_NUCLEUS : CLS_FULL;
    RowInfo ri;
    ri.cls = cls;
    ri.L = L;
    ri.status = (cls >= 0) ? ST_LIVE : ST_ERROR;
    ri.acc = 0;
    ri.kpos = 0;
    ri.need = NEED_NONE;
    ri.k_eff = (cls == CLS_TOPK) ? tk : 0;
    ri.flags = 0;
    ri.T = T;
    ri.top_p = tp;
    ri.pad0 = ri.pad1 = 0;
    ri.mt = ri.zt = ri.md = ri.zd = 0.0;
    ri.tau_t = ri.tau_d = 0ull;
    a.rows[b] = ri;
    int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
    for (int j = 0; j <= a.K; j++) o[j] = -1;
    a.out_acc[b] = (cls == CLS_ERROR) ? -1 : (cls == CLS_UNSUP ? -2 : 0);
    if (a.diag) {
        double* d = a.diag + (int64_t)b * 4 * (a.K + 1);
        for (int j = 0; j < 4 * (a.K + 1); j++) d[j] = __longlong_as_double(0x7FF8000000000000ll);
    }
}

}  // namespace sv
