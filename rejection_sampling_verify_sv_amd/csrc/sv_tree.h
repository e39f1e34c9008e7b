// sv_tree.h — child rounds of a tree verify on full-vocab rows.
//
// tinycto.tv "Spekülatif Kod Çözme (Speculative Decoding)…", question
// "Medusa / Eagle spekülatif taslak mekanizması nedir?": draft heads propose
// several candidate tokens; the pages give no rule for checking them.  The
// reading taken here keeps the output law equal to the target's when a
// node's candidates are drawn independently from the draft distribution q
// there: recursive rejection.  The node's children are tested in turn, child
// i against the residual r_{i-1} left by the previous rejections
// (r_0 = p, r_i = (r_{i-1} - q)+ / W_i with W_i its mass), and when all are
// rejected the final token is drawn from what is left.
//
// Top-k and greedy rows run the whole loop inside the decision wave (their
// distributions sit in registers).  A full-vocab row needs W_i, a sum over
// the whole vocabulary, before it can test child i + 1: after the decision of
// a level tested the first child, round j = 1, 2, ... of the level runs
//   sample_sums_kernel   over the rows of round j's list: per (tile, wave)
//                        the mass of (r_{j-1} - q)+ on the node's two rows
//   tree_round_kernel    one wave per row: W_j from those chunks (fixed
//                        order), then the test of the next child against
//                        r_j; accept: the child's units go to the next
//                        level's lists; reject: the row joins round j + 1's
//                        list, or, with no child left, the final draw list.
#pragma once

#include "sv_decide.h"

namespace sv {

// Normalised p and q of one token of a full-vocab row, from the statistics
// the decision stored (untruncated: max and normaliser; nucleus: anchor,
// kept mass and cut key).
template <int DT>
__device__ inline void full_pq(const StepArgs& a, const RowInfo& ri, int b, int v, int x,
                               double* px, double* qx) {
    const float lx = load_one<DT>(unit_row<DT>(a, b, 0, v), x);
    const float ld = load_one<DT>(unit_row<DT>(a, b, 1, v), x);
    if (ri.cls == CLS_NUCLEUS) {
        const float cb = bucket_coef(ri.T);
        *px = (make_key(lx, (uint32_t)x) >= ri.tau_t)
                  ? exp((double)nuc_t(lx, (float)ri.mt, cb) * (1.0 / 64.0)) / ri.zt
                  : 0.0;
        *qx = (make_key(ld, (uint32_t)x) >= ri.tau_d)
                  ? exp((double)nuc_t(ld, (float)ri.md, cb) * (1.0 / 64.0)) / ri.zd
                  : 0.0;
    } else {
        const double T = (double)ri.T;
        *px = exp(((double)lx - ri.mt) / T) / ri.zt;
        *qx = exp(((double)ld - ri.md) / T) / ri.zd;
    }
}

// Round j of level k: one wave per row of round j's list.
template <int DT>
__global__ __launch_bounds__(kThreads) void tree_round_kernel(StepArgs a, int k, int j) {
    const int n = a.tcount[k * kMaxKids + j];
    const int32_t* list = a.tlist + (int64_t)j * a.B;
    const int lane = lane_id();
    for (int i = blockIdx.x * kWaves + wave_id(); i < n; i += gridDim.x * kWaves) {
        const int b = list[i];
        const RowInfo ri = a.rows[b];
        const int v = ri.node;
        // W_j: the chunk masses of (r_{j-1} - q)+, tiles in order per lane,
        // then the lanes in the fixed DPP tree
        const double2* cs = a.chunks + (int64_t)b * a.ntiles * kWaves;
        double part = 0.0;
        for (int t = lane; t < a.ntiles; t += kWave)
            for (int q = 0; q < kWaves; q++) part += cs[t * kWaves + q].x;
        const double W = wave_sum(part);
        double* wc = a.wchain + (int64_t)b * kMaxKids;
        const int c = ri.nxt;
        const int x = a.tokens[(int64_t)b * a.K + c - 1];
        const bool kids = next_child(a, b, c, c, ri.L) >= 0;
        const int nxt = next_child(a, b, v, c, ri.L);
        if (lane != 0) continue;
        wc[j - 1] = W;
        double px, qx;
        full_pq<DT>(a, ri, b, v, x, &px, &qx);
        const double rx = resid_chain(px, qx, j, wc);
        const double acc = accept_prob(rx, qx);
        const double uc = (double)a.uniforms[(int64_t)b * (a.K + 1) + c - 1];
        write_accept_diag(a, b, c - 1, rx, qx, acc, uc);
        RowInfo& w = a.rows[b];
        w.rounds = j;
        if (uc < acc) {
            DecideIntent it;
            it.nu = 0;
            it.cls = 0;
            it.draw = 0;
            it.rnd = 0;
            it.pick = 0;
            tree_continue(a, b, k, c, x, kids, ri, it);
            // the child's units join level k + 1's lists
            const int li = atomicAdd(&a.pos[k + 1].n_cls[it.cls], it.nu);
            int32_t* ul = a.ulist + ((int64_t)(k + 1) * kNumCls + it.cls) * a.ustride;
            ul[li] = b * 2;
            w.li_t = li;
            if (it.nu == 2) {
                ul[li + 1] = b * 2 + 1;
                w.li_d = li + 1;
            }
            if (it.cls == CLS_NUCLEUS) {
                a.fn_unit[b * 2].rehist = 0;
                if (it.nu == 2) a.fn_unit[b * 2 + 1].rehist = 0;
            }
        } else if (nxt >= 0) {
            w.nxt = nxt;
            const int s = atomicAdd(&a.tcount[k * kMaxKids + j + 1], 1);
            a.tlist[(int64_t)(j + 1) * a.B + s] = b;
        } else {
            w.need = NEED_RESID;
            w.nxt = -1;
            a.slist[atomicAdd(&a.pos[a.K + 1].n_sample, 1)] = b;
            w.status = ST_SAMPLE;
        }
    }
}

}  // namespace sv
