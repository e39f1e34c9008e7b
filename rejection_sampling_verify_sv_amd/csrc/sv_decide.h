// sv_decide.h — per-row decision at one draft position, and row set-up.
//
// After the row pass (and, for nucleus rows, the nucleus cut) of position k,
// one wave per live row:
//   * merges the segment records of the target (and draft) row;
//   * top-k rows: applies temperature, the top_p walk over the renormalised
//     top-k and renormalisation in fp64 across the lanes (lane j holds the
//     j-th ranked token); then runs the accept test and, if the row ends here,
//     the residual or bonus draw over the <= 64 kept tokens in ascending id
//     order;
//   * greedy rows: compares the draft token with the target argmax;
//   * full-vocab rows: forms p(x), q(x) from {max, sum-exp} (untruncated) or
//     from the exact nucleus cut, runs the accept test and, if the row ends
//     here, queues the draw for the full-vocab sampler (sv_sample.h).
// A row that accepts and continues lists its units for position k+1.
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

// One wave per row, kDecideRows rows per workgroup.  A row's wave only
// records what it adds to the next position's unit lists or to the draw list
// (DecideIntent, in LDS); the workgroup then reserves space for all its rows
// with one global atomic per list, instead of one per row.
constexpr int kDecideRows = kWaves;

struct DecideIntent {
    int32_t nu;    // units to list at position k+1 (0: none)
    int32_t cls;   // their class region
    int32_t draw;  // 1: the row draws over the full vocabulary at the end
    int32_t rnd;   // 1: tree verify, the row tests its node's next child after a pass
    int32_t pick;  // 1: that draw is an untruncated bonus draw (no second pass)
};

// Per-wave LDS of the top-k draw, passed in by the kernel (which lays it over
// memory that its other steps use).
struct TopkScratch {
    double w[kWave];
    double p[kWave];
    int32_t id[kWave];
};

// A nucleus unit's cut, as another workgroup of the same launch may have
// left it (device-scope loads, see dev_store).
__device__ inline FnUnit fn_unit_load(const FnUnit* f) {
    FnUnit* m = const_cast<FnUnit*>(f);
    FnUnit r;
    r.S = __longlong_as_double((long long)dev_load(reinterpret_cast<uint64_t*>(&m->S)));
    r.tau = dev_load(&m->tau);
    r.la = __int_as_float(dev_load(reinterpret_cast<int32_t*>(&m->la)));
    r.status = dev_load(&m->status);
    r.rehist = 0;
    return r;
}

__device__ inline void diag_nan_row(double* diag, int b, int K) {
    if (!diag) return;
    double* d = diag + (int64_t)b * 4 * (K + 1);
    for (int i = lane_id(); i < 4 * (K + 1); i += kWave)
        d[i] = __longlong_as_double(0x7FF8000000000000ll);
}

// One lane: write accepted drafts + final token, close the row.  A tree
// verify writes each accepted token as its walk takes it (tree_continue).
__device__ inline void emit_row(const StepArgs& a, int b, int acc, int y) {
    int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
    if (!a.tree) {
        const int32_t* t = a.tokens + (int64_t)b * a.K;
        for (int j = 0; j < acc; j++) o[j] = t[j];
    }
    o[acc] = y;
    a.out_acc[b] = acc;
    a.rows[b].acc = acc;
    a.rows[b].status = ST_DONE;
}

// Every lane of the wave calls these (the diagnostics are cleared in parallel).
__device__ inline void close_row_invalid(const StepArgs& a, int b, int code) {
    diag_nan_row(a.diag, b, a.K);
    if (lane_id() == 0) {
        int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
        for (int j = 0; j <= a.K; j++) o[j] = -1;
        if (a.out_path)  // a tree verify writes its path as it walks
            for (int j = 0; j <= a.K; j++) a.out_path[(int64_t)b * (a.K + 1) + j] = -1;
        a.out_acc[b] = code;  // -1 invalid data, -2 not served
        a.rows[b].status = ST_ERROR;
    }
}

// Index of the first lane where pred holds, or -1.
__device__ __forceinline__ int first_lane(bool pred) {
    const uint64_t m = __ballot(pred);
    return m ? __ffsll((unsigned long long)m) - 1 : -1;
}

// Top-64 keys (descending, lane j = j-th) of one or two units from their
// records, merged in record order.  The first kPreRec records of both units
// are loaded before the first merge: the decision then waits about one memory
// round trip for them, not one per record.
constexpr int kPreRec = 8;
__device__ __forceinline__ void unit_tops(const PartSlot* parts, RecRange ra, RecRange rb,
                                          bool two, uint64_t* ta, uint64_t* tb) {
    const int lane = lane_id();
    uint64_t xa[kPreRec], xb[kPreRec];
#pragma unroll
    for (int j = 0; j < kPreRec; j++) {
        xa[j] = j < ra.count ? parts[ra.first + j].keys[lane] : 0ull;
        xb[j] = (two && j < rb.count) ? parts[rb.first + j].keys[lane] : 0ull;
    }
    uint64_t x = xa[0], y = xb[0];
#pragma unroll
    for (int j = 1; j < kPreRec; j++) {
        if (j < ra.count) x = wave_merge_top(x, xa[j]);
        if (two && j < rb.count) y = wave_merge_top(y, xb[j]);
    }
    for (int i = kPreRec; i < ra.count; i++) x = wave_merge_top(x, parts[ra.first + i].keys[lane]);
    if (two)
        for (int i = kPreRec; i < rb.count; i++) y = wave_merge_top(y, parts[rb.first + i].keys[lane]);
    *ta = x;
    *tb = y;
}
__device__ __forceinline__ uint64_t unit_top(const PartSlot* parts, RecRange r) {
    uint64_t x, y;
    unit_tops(parts, r, r, false, &x, &y);
    return x;
}

// Record slots of unit (b, position k, side) of row class cls: in the list of
// position k's launch, or of the one launch of a dense step.
// P: the descriptor of the launch that streamed the unit (position k's, or
// the dense step's one launch), held in LDS by the caller.
__device__ __forceinline__ RecRange unit_rec(const StepArgs& a, const PosDesc& P, int cls, int li) {
    return unit_records(P, unit_index(P, cls, li), a.ntiles, a.g_row);
}
// Index of unit (b, position k, side) in its class region: kept in the row's
// info, or, in the merged launch, in dli (loaded with the row's info).
struct UnitIdx {
    int t, d;
};
__device__ __forceinline__ UnitIdx unit_idx_prefetch(const StepArgs& a, int b, int k) {
    UnitIdx u;
    u.t = k >= a.d0 ? a.dli[unit_code(a, b, k, 0)] : -1;
    u.d = k >= a.d0 ? a.dli[unit_code(a, b, k, 1)] : -1;
    return u;
}
__device__ __forceinline__ UnitIdx unit_idx(const StepArgs& a, const RowInfo& ri, UnitIdx pre,
                                            int k) {
    if (k >= a.d0) return pre;
    UnitIdx u;
    u.t = ri.li_t;
    u.d = ri.li_d;
    return u;
}

// Truncated distribution over a ranked list (lane j = j-th ranked token):
// temperature, top_k (first k_eff lanes), renormalise, keep while the mass
// before the token is < top_p, renormalise.  Returns false when the best
// logit is -inf (no finite logit).
__device__ bool topk_dist_wave(uint64_t key, int k_eff, double T, double top_p, double* p,
                               bool* keep) {
    const int lane = lane_id();
    const bool valid = lane < k_eff;
    const double l = (double)key_logit(key);
    const double l0 = lane_value(l, 0);
    if (!(l0 > -INFINITY)) return false;
    const double w = valid ? exp((l - l0) / T) : 0.0;
    int nkeep = k_eff;
    if (top_p < 1.0) {
        const double zk = wave_sum(w);
        const double P = w / zk;
        const double mass_before = wave_shift_up1(wave_incl_scan(P));  // 0 in lane 0
        const int f = first_lane(valid && !(mass_before < top_p));
        nkeep = f < 0 ? k_eff : f;
    }
    *keep = lane < nkeep;
    const double zs = wave_sum(*keep ? w : 0.0);
    *p = *keep ? w / zs : 0.0;
    return true;
}

__device__ __forceinline__ double lookup_lane(bool keep, int id, double p, int token) {
    const int j = first_lane(keep && id == token);
    return j < 0 ? 0.0 : lane_value(p, j);
}

__device__ __forceinline__ double accept_prob(double px, double qx) {
    if (qx > 0.0) {
        const double a = px / qx;
        return a > 1.0 ? 1.0 : a;
    }
    return (px > 0.0) ? 1.0 : 0.0;
}

// Diagnostics of one accept test, slot `slot` (draft position k, or node c's
// test at c - 1 in a tree verify).
__device__ __forceinline__ void write_accept_diag(const StepArgs& a, int b, int slot, double px,
                                                  double qx, double acc, double uk) {
    if (a.diag && lane_id() == 0) {
        double* dg = a.diag + (int64_t)b * 4 * (a.K + 1);
        dg[4 * slot + 0] = px;
        dg[4 * slot + 1] = qx;
        dg[4 * slot + 2] = acc;
        dg[4 * slot + 3] = fabs(uk - acc);
    }
}

// ---- tree verify helpers -----------------------------------------------------
// Node c >= 1 of row b has parent parents[b][c-1] < c, so the children of v
// are nodes in (v, L].  Wave-wide scans (every lane gets the result).
// The first child of v after node `after`, or -1.
__device__ inline int next_child(const StepArgs& a, int b, int v, int after, int L) {
    const int32_t* par = a.parents + (int64_t)b * a.K;
    for (int c0 = (after > v ? after : v) + 1; c0 <= L; c0 += kWave) {
        const int c = c0 + lane_id();
        const uint64_t m = __ballot(c <= L && par[c - 1] == v);
        if (m) return c0 + __ffsll((unsigned long long)m) - 1;
    }
    return -1;
}
// The first child of v whose token is `tok`, or -1.
__device__ inline int child_with_token(const StepArgs& a, int b, int v, int L, int tok) {
    const int32_t* par = a.parents + (int64_t)b * a.K;
    const int32_t* tk = a.tokens + (int64_t)b * a.K;
    for (int c0 = v + 1; c0 <= L; c0 += kWave) {
        const int c = c0 + lane_id();
        const uint64_t m = __ballot(c <= L && par[c - 1] == v && tk[c - 1] == tok);
        if (m) return c0 + __ffsll((unsigned long long)m) - 1;
    }
    return -1;
}
// The first child of the row's current node, or -1 (a verify step: the next
// drafted position, node k + 1, while k < L).
__device__ inline int first_child(const StepArgs& a, int b, int k, const RowInfo& ri) {
    if (!a.tree) return k < ri.L ? k + 1 : -1;
    return next_child(a, b, ri.node, ri.node, ri.L);
}
// Row b accepts child c (token x) of its node at level k: the token and the
// node are written out, c becomes the row's node, and its units are listed
// for level k + 1 (c's draft row only when c has children).  One lane.
__device__ inline void tree_continue(const StepArgs& a, int b, int k, int c, int x, bool kids,
                                     const RowInfo& ri, DecideIntent& it) {
    a.out_tokens[(int64_t)b * (a.K + 1) + k] = x;
    if (a.out_path) a.out_path[(int64_t)b * (a.K + 1) + k] = c;
    RowInfo& w = a.rows[b];
    w.acc = k + 1;
    w.node = c;
    w.kids = kids ? 1 : 0;
    w.rounds = 0;
    w.nxt = -1;
    it.nu = (ri.cls != CLS_GREEDY && kids) ? 2 : 1;
    it.cls = ri.cls;
}

// Row b accepted the draft at position k: its units go to position k+1's
// lists (one lane calls this).
// Units of row ri at positions k0..L, target then draft at each (the draft
// unit up to L - 1, none for greedy rows).
__device__ __forceinline__ int units_from(const RowInfo& ri, int k0) {
    return ri.cls == CLS_GREEDY ? ri.L - k0 + 1 : 2 * (ri.L - k0) + 1;
}
__device__ inline void note_continue(const StepArgs& a, int b, int k, const RowInfo& ri,
                                     DecideIntent& it) {
    a.rows[b].acc = k + 1;
    // the merged launch streams every remaining position of the row
    it.nu = (k + 1 == a.d0) ? units_from(ri, k + 1)
                            : ((ri.cls != CLS_GREEDY && k + 1 < ri.L) ? 2 : 1);
    it.cls = ri.cls;
}
__device__ inline void continue_row(const StepArgs& a, int b, int k, const RowInfo& ri,
                                    DecideIntent& it) {
    if (lane_id() == 0) note_continue(a, b, k, ri, it);
}

// Row b ends at position k with a draw over the full vocabulary (one lane).
__device__ inline void queue_draw(DecideIntent& it) { it.draw = 1; }
// An untruncated bonus draw: its chunk masses are the row pass's (tile, wave)
// records rescaled, so only the chosen chunk is read again (the draw list's
// far end).  The records outlive the later launches: a row that stopped is
// not streamed again, and the merged launch's unit codes lie past the others.
// In a tree verify the bonus node was reached by an accepted child (no
// residual chain), and the row pass of its level left its records.
__device__ inline void queue_bonus(DecideIntent& it) { it.pick = 1; }

// q of each lane's kept p token (0 when q drops it): the kept q tokens are a
// prefix of the lanes, broadcast one at a time by scalar lane reads.
__device__ __forceinline__ double q_of_lane(int id_p, int id_q, double q, bool keep_q) {
    const int nq = __popcll(__ballot(keep_q));
    double qj = 0.0;
    const int q_lo = __double2loint(q), q_hi = __double2hiint(q);
    for (int s = 0; s < nq; s++) {
        const int ids = __builtin_amdgcn_readlane(id_q, s);
        const double qs = __hiloint2double(__builtin_amdgcn_readlane(q_hi, s),
                                           __builtin_amdgcn_readlane(q_lo, s));
        if (ids == id_p) qj = qs;
    }
    return qj;
}

// Final draw of a top-k row over p's kept tokens in ascending id order, with
// weight fw in the lane of each kept token: the residual after a rejection
// (resid; p itself when the residual has no mass), p for the bonus token.
// Every lane gets the token and its diagnostics (the drawn token's
// final-distribution probability, its CDF bin [lo, hi) and the uniform's
// margin to it).
__device__ int topk_draw_calc(double p, bool keep_p, int id_p, double fw, bool resid, double uf,
                              TopkScratch& ts, double (&dg)[4]) {
    double* s_w = ts.w;
    double* s_p = ts.p;
    int* s_id = ts.id;
    const int lane = lane_id();
    const int np = __popcll(__ballot(keep_p));
    int rank = 0;
    for (int s = 0; s < np; s++) rank += __builtin_amdgcn_readlane(id_p, s) < id_p ? 1 : 0;
    if (keep_p) {
        s_w[rank] = fw;
        s_p[rank] = p;
        s_id[rank] = id_p;
    }
    wave_lds_sync();
    const int kp = np;
    double wr = lane < kp ? s_w[lane] : 0.0;
    const double pr = lane < kp ? s_p[lane] : 0.0;
    const int idr = lane < kp ? s_id[lane] : -1;
    double W = wave_sum(wr);
    const bool fallback = resid && !(W > 0.0);
    if (fallback) {  // p == q up to rounding: draw from p
        wr = pr;
        W = wave_sum(wr);
    }
    const double target = uf * W;
    const double incl = wave_incl_scan(wr);
    const double excl = wave_shift_up1(incl);  // 0 in lane 0
    int j = first_lane(wr > 0.0 && target < incl);
    double margin_scale = 1.0;
    if (j < 0) {  // not reachable for u < 1; keeps the function total
        const uint64_t pos = __ballot(wr > 0.0);
        j = 63 - __clzll((unsigned long long)pos);
        margin_scale = 0.0;
    }
    // j is the same in every lane: scalar reads of lane j
    const int y = __builtin_amdgcn_readlane(idr, j);
    const double lo = lane_value(excl, j) / W;
    const double hi = (margin_scale == 0.0) ? 1.0 : lane_value(incl, j) / W;
    const double wy = lane_value(wr, j);
    const double py = lane_value(pr, j);
    const double d1 = uf - lo, d2 = hi - uf;
    dg[0] = resid ? wy / W : py;
    dg[1] = lo;
    dg[2] = hi;
    dg[3] = margin_scale * (d1 < d2 ? d1 : d2);
    return y;
}
// The final draw's diagnostics (slot K) of row b.
__device__ __forceinline__ void write_final_diag(const StepArgs& a, int b, const double (&dg)[4]) {
    if (a.diag) {
        double* d = a.diag + (int64_t)b * 4 * (a.K + 1) + 4 * a.K;
        for (int i = 0; i < 4; i++) d[i] = dg[i];
    }
}
// The draw, written out: the row ends at accept length k with the drawn token.
__device__ void topk_draw(const StepArgs& a, int b, int k, double p, bool keep_p, int id_p,
                          double fw, bool resid, double uf, TopkScratch& ts) {
    double dg[4];
    const int y = topk_draw_calc(p, keep_p, id_p, fw, resid, uf, ts, dg);
    if (lane_id() == 0) {
        write_final_diag(a, b, dg);
        emit_row(a, b, k, y);
    }
}

// Returns true (in every lane) when the row accepted and goes on to the next
// position; the same for the other classes below.
__device__ bool decide_topk(const StepArgs& a, const PosDesc& P, int b, int k, const RowInfo& ri,
                            UnitIdx ui, TopkScratch& ts, DecideIntent& it) {
    const int k_eff = ri.k_eff;
    const double T = (double)ri.T, top_p = (double)ri.top_p;
    const int child = first_child(a, b, k, ri);
    const bool has_draft = child >= 0;
    const float* u = a.uniforms + (int64_t)b * (a.K + 1);
    // every load first, so that their latencies overlap
    int x = 0;
    double uk = 0.0;
    if (has_draft) {
        x = a.tokens[(int64_t)b * a.K + child - 1];
        uk = (double)u[child - 1];
    }
    uint64_t kt, kd;
    unit_tops(a.parts, unit_rec(a, P, CLS_TOPK, ui.t), unit_rec(a, P, CLS_TOPK, ui.d), has_draft,
              &kt, &kd);
    const double uf = (double)u[a.K];
    double p;
    bool keep_p;
    if (!topk_dist_wave(kt, k_eff, T, top_p, &p, &keep_p)) {
        close_row_invalid(a, b, -1);
        return false;
    }
    const int id_p = (int)key_id(kt);
    if (!has_draft) {  // bonus token from p
        topk_draw(a, b, k, p, keep_p, id_p, p, false, uf, ts);
        return false;
    }
    double q;
    bool keep_q;
    if (!topk_dist_wave(kd, k_eff, T, top_p, &q, &keep_q)) {
        close_row_invalid(a, b, -1);
        return false;
    }
    const int id_q = (int)key_id(kd);
    if (!a.tree) {
        const double px = lookup_lane(keep_p, id_p, p, x);
        const double qx = lookup_lane(keep_q, id_q, q, x);
        const double acc = accept_prob(px, qx);
        write_accept_diag(a, b, k, px, qx, acc, uk);
        if (uk < acc) {
            continue_row(a, b, k, ri, it);
            return true;
        }
        // the residual (p - q)+ over p's kept tokens
        const double d = p - q_of_lane(id_p, id_q, q, keep_q);
        topk_draw(a, b, k, p, keep_p, id_p, d > 0.0 ? d : 0.0, true, uf, ts);
        return false;
    }
    // Tree verify: the node's children in turn against r, which starts as p
    // and becomes the normalised residual (r - q)+ after each rejection
    // (unchanged when that has no mass); all rejected: draw from what is
    // left of r.
    const double qj = q_of_lane(id_p, id_q, q, keep_q);
    double r = keep_p ? p : 0.0;
    int c = child;
    double fw;
    for (;;) {
        const double rx = lookup_lane(keep_p, id_p, r, x);
        const double qx = lookup_lane(keep_q, id_q, q, x);
        const double acc = accept_prob(rx, qx);
        write_accept_diag(a, b, c - 1, rx, qx, acc, uk);
        if (uk < acc) {
            const bool kids = next_child(a, b, c, c, ri.L) >= 0;
            if (lane_id() == 0) tree_continue(a, b, k, c, x, kids, ri, it);
            return true;
        }
        const double d = keep_p ? r - qj : 0.0;
        const double w = d > 0.0 ? d : 0.0;
        const double W = wave_sum(w);
        c = next_child(a, b, ri.node, c, ri.L);
        if (c < 0) {
            fw = W > 0.0 ? w : r;
            break;
        }
        if (W > 0.0) r = w / W;
        x = a.tokens[(int64_t)b * a.K + c - 1];
        uk = (double)u[c - 1];
    }
    topk_draw(a, b, k, p, keep_p, id_p, fw, true, uf, ts);
    return false;
}

__device__ bool decide_greedy(const StepArgs& a, const PosDesc& P, int b, int k,
                              const RowInfo& ri, UnitIdx ui, DecideIntent& it) {
    const int lane = lane_id();
    // the drafted token, loaded with the records
    const int tok = (!a.tree && k < ri.L) ? a.tokens[(int64_t)b * a.K + k] : -1;
    const RecRange r = unit_rec(a, P, CLS_GREEDY, ui.t);
    const PartSlot* s = a.parts + r.first;
    uint64_t best = 0ull;
    for (int i = lane; i < r.count; i += kWave) best = s[i].keys[0] > best ? s[i].keys[0] : best;
    best = wave_max_u64(best);
    const int g = (int)key_id(best);
    if (a.tree) {  // the first child whose token is the argmax, if any
        const int c = child_with_token(a, b, ri.node, ri.L, g);
        if (c >= 0) {
            const bool kids = next_child(a, b, c, c, ri.L) >= 0;
            if (lane == 0) tree_continue(a, b, k, c, g, kids, ri, it);
            return true;
        }
    } else if (k < ri.L && tok == g) {
        continue_row(a, b, k, ri, it);
        return true;
    }
    if (lane == 0) emit_row(a, b, k, g);
    return false;
}

// {max, sum-exp} of one full-vocab unit from its n per-(tile, wave) records
// {m_i, s_i}: M = max m_i, Z = sum s_i exp((m_i - M) / T), each lane summing
// its records in index order and the lanes in the fixed DPP tree, so every
// lane gets the same bits.  One exp per record, none along the tree.
// Two units at once (rb may be null): the first kPreStat records of each lane
// of both are loaded before any is used.
constexpr int kPreStat = 4;
__device__ inline void full_stats2(const FullStat* ra, const FullStat* rb, int n, double invT,
                                   double* ma, double* za, double* mb, double* zb) {
    const int lane = lane_id();
    FullStat xa[kPreStat], xb[kPreStat];
#pragma unroll
    for (int j = 0; j < kPreStat; j++) {
        const int i = lane + j * kWave;
        xa[j].m = -INFINITY;
        xa[j].s = 0.0;
        xb[j] = xa[j];
        if (i < n) {
            xa[j] = ra[i];
            if (rb) xb[j] = rb[i];
        }
    }
    float mx = -INFINITY, my = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPreStat; j++) {
        mx = fmaxf(mx, xa[j].m);
        my = fmaxf(my, xb[j].m);
    }
    for (int i = lane + kPreStat * kWave; i < n; i += kWave) {
        mx = fmaxf(mx, ra[i].m);
        if (rb) my = fmaxf(my, rb[i].m);
    }
    const float MX = wave_max_f32(mx), MY = wave_max_f32(my);
    double sx = 0.0, sy = 0.0;
#pragma unroll
    for (int j = 0; j < kPreStat; j++) {
        if (MX > -INFINITY && xa[j].m > -INFINITY)
            sx += xa[j].s * exp(((double)xa[j].m - (double)MX) * invT);
        if (MY > -INFINITY && xb[j].m > -INFINITY)
            sy += xb[j].s * exp(((double)xb[j].m - (double)MY) * invT);
    }
    for (int i = lane + kPreStat * kWave; i < n; i += kWave) {
        const FullStat r = ra[i];
        if (MX > -INFINITY && r.m > -INFINITY) sx += r.s * exp(((double)r.m - (double)MX) * invT);
        if (rb) {
            const FullStat q = rb[i];
            if (MY > -INFINITY && q.m > -INFINITY)
                sy += q.s * exp(((double)q.m - (double)MY) * invT);
        }
    }
    *ma = (double)MX;
    *za = wave_sum(sx);
    *mb = (double)MY;
    *zb = wave_sum(sy);
}
__device__ inline void full_stats(const FullStat* rec, int n, double invT, double* m, double* z) {
    double m2, z2;
    full_stats2(rec, nullptr, n, invT, m, z, &m2, &z2);
}

// Tree verify, full-vocab rows: the row rejected child `c` of its node and the
// node has another child, nxt: the next test needs the mass of the residual,
// one more pass over the node's two rows (tree_sums / tree_round).  One lane.
__device__ inline void tree_to_round(const StepArgs& a, int b, int v, int nxt, DecideIntent& it) {
    RowInfo& w = a.rows[b];
    w.kpos = v;
    w.rounds = 0;
    w.nxt = nxt;
    it.rnd = 1;
}

template <int DT>
__device__ bool decide_full(const StepArgs& a, int b, int k, const RowInfo& ri, DecideIntent& it) {
    const double T = (double)ri.T, invT = 1.0 / T;
    double mt, zt, md = 0.0, zd = 0.0;
    const int nrec = a.ntiles * kWaves;
    const int v = row_at(a, b, k);
    const int child = first_child(a, b, k, ri);
    // the drafted token's logits and the uniform, loaded while the records are
    float lx = 0.f, ld = 0.f, ukf = 0.f;
    int x = 0;
    if (child >= 0) {
        x = a.tokens[(int64_t)b * a.K + child - 1];
        if (x >= 0 && x < a.V) {  // validated by the plan; kept in range here regardless
            lx = load_one<DT>(unit_row<DT>(a, b, 0, v), x);
            ld = load_one<DT>(unit_row<DT>(a, b, 1, v), x);
        }
        ukf = a.uniforms[(int64_t)b * (a.K + 1) + child - 1];
    }
    full_stats2(a.tstat + (int64_t)unit_code(a, b, k, 0) * nrec,
                child >= 0 ? a.tstat + (int64_t)unit_code(a, b, k, 1) * nrec : nullptr, nrec, invT,
                &mt, &zt, &md, &zd);
    if (!(mt > -INFINITY)) {
        close_row_invalid(a, b, -1);
        return false;
    }
    if (child < 0) {
        if (lane_id() == 0) {
            RowInfo& w = a.rows[b];
            w.need = NEED_BONUS;
            w.kpos = v;
            w.mt = mt;
            w.zt = zt;
            queue_bonus(it);
        }
        return false;
    }
    if (!(md > -INFINITY)) {
        close_row_invalid(a, b, -1);
        return false;
    }
    // tree verify: whether the child has children, the node's next child
    const bool kids = a.tree && next_child(a, b, child, child, ri.L) >= 0;
    const int nxt = a.tree ? next_child(a, b, v, child, ri.L) : -1;
    // every lane holds the same statistics and logits: the decision is the
    // same in all of them, lane 0 writes it
    const double px = exp(((double)lx - mt) / T) / zt;
    const double qx = exp(((double)ld - md) / T) / zd;
    const double acc = accept_prob(px, qx);
    const double uk = (double)ukf;
    const bool cont = uk < acc;
    write_accept_diag(a, b, child - 1, px, qx, acc, uk);
    if (lane_id() != 0) return cont;
    RowInfo& w = a.rows[b];
    if (cont) {
        if (a.tree)
            tree_continue(a, b, k, child, x, kids, ri, it);
        else
            note_continue(a, b, k, ri, it);
    } else {
        w.mt = mt;
        w.zt = zt;
        w.md = md;
        w.zd = zd;
        if (nxt >= 0) {
            tree_to_round(a, b, v, nxt, it);
            return cont;
        }
        w.need = NEED_RESID;
        w.kpos = v;
        queue_draw(it);
    }
    return cont;
}

// Nucleus rows: p(x) = [key(x) >= tau] exp(t(x) / 64) / S with the anchor
// coordinate t and the kept mass S of the cut computed by the nucleus kernels
// for this position.
template <int DT>
__device__ bool decide_nucleus(const StepArgs& a, int b, int k, const RowInfo& ri,
                               DecideIntent& it) {
    const FnUnit ut = fn_unit_load(a.fn_unit + unit_code(a, b, k, 0));
    const int v = row_at(a, b, k);
    const int child = first_child(a, b, k, ri);
    const bool has_draft = child >= 0;
    FnUnit ud;
    ud.status = 0;
    float lx = 0.f, ld = 0.f, ukf = 0.f;
    int x = 0;
    if (has_draft) {  // loaded together with the cut states
        ud = fn_unit_load(a.fn_unit + unit_code(a, b, k, 1));
        x = a.tokens[(int64_t)b * a.K + child - 1];
        if (x >= 0 && x < a.V) {  // validated by the plan; kept in range here regardless
            lx = load_one<DT>(unit_row<DT>(a, b, 0, v), x);
            ld = load_one<DT>(unit_row<DT>(a, b, 1, v), x);
        }
        ukf = a.uniforms[(int64_t)b * (a.K + 1) + child - 1];
    }
    const int st = ut.status != 0 ? ut.status : (has_draft ? ud.status : 0);
    if (st != 0) {
        close_row_invalid(a, b, st == 1 ? -2 : -1);
        return false;
    }
    const bool kids = a.tree && has_draft && next_child(a, b, child, child, ri.L) >= 0;
    const int nxt = (a.tree && has_draft) ? next_child(a, b, v, child, ri.L) : -1;
    if (!has_draft) {
        if (lane_id() == 0) {
            RowInfo& w = a.rows[b];
            w.need = NEED_BONUS;
            w.kpos = v;
            w.mt = (double)ut.la;
            w.zt = ut.S;
            w.tau_t = ut.tau;
            queue_draw(it);
        }
        return false;
    }
    // the same cut states and logits in every lane: one decision, lane 0
    // writes it
    const float cb = bucket_coef(ri.T);
    const double px = (make_key(lx, (uint32_t)x) >= ut.tau)
                          ? exp((double)nuc_t(lx, ut.la, cb) * (1.0 / 64.0)) / ut.S
                          : 0.0;
    const double qx = (make_key(ld, (uint32_t)x) >= ud.tau)
                          ? exp((double)nuc_t(ld, ud.la, cb) * (1.0 / 64.0)) / ud.S
                          : 0.0;
    const double acc = accept_prob(px, qx);
    const double uk = (double)ukf;
    const bool cont = uk < acc;
    write_accept_diag(a, b, child - 1, px, qx, acc, uk);
    if (lane_id() != 0) return cont;
    RowInfo& w = a.rows[b];
    if (cont) {
        if (a.tree)
            tree_continue(a, b, k, child, x, kids, ri, it);
        else
            note_continue(a, b, k, ri, it);
    } else {
        w.mt = (double)ut.la;
        w.zt = ut.S;
        w.tau_t = ut.tau;
        w.md = (double)ud.la;
        w.zd = ud.S;
        w.tau_d = ud.tau;
        if (nxt >= 0) {
            tree_to_round(a, b, v, nxt, it);
            return cont;
        }
        w.need = NEED_RESID;
        w.kpos = v;
        queue_draw(it);
    }
    return cont;
}

// ---- the merged launch with few rows: a row's positions side by side --------
// When every row of a merged (or dense) launch can have a workgroup of its
// own, the workgroup's waves decide positions base .. base + kWaves - 1 of
// its row at once, each into a slot, and wave 0 then walks the slots in
// order: it writes what the walk reaches (accept diagnostics, then the
// first rejection's token or full-vocab draw, or the invalid row) and stops
// there.  Each position's decision depends only on that position's records,
// token and uniform, so the outcome is the one the position-by-position walk
// gives; the positions past the row's end are computed and dropped.
enum SpecKind : int32_t { SP_ACCEPT = 0, SP_EMIT = 1, SP_DRAW = 2, SP_INVALID = 3 };
struct SpecSlot {
    double px, qx, acc, u;   // the accept test, when one ran (tested)
    double dy[4];            // an emitted top-k draw's final diagnostics (has_dy)
    double mt, zt, md, zd;   // a full-vocab draw's statistics (SP_DRAW)
    uint64_t tau_t, tau_d;
    int32_t kind, y, code, need, tested, has_dy, pick, pad;
};

// The decision at position kk of row b, side effects left out, into slot
// `out` (LDS, written by lane 0 as the values are known); every lane of the
// wave calls it.
template <int DT>
__device__ void spec_position(const StepArgs& a, const PosDesc& P, int b, int kk, const RowInfo& ri,
                              UnitIdx ui, TopkScratch& ts, SpecSlot* out) {
    const bool l0 = lane_id() == 0;
    if (l0) {
        out->kind = SP_ACCEPT;
        out->tested = 0;
        out->has_dy = 0;
        out->pick = 0;
    }
    const int L = ri.L;
    const bool has_draft = kk < L;
    const float* u = a.uniforms + (int64_t)b * (a.K + 1);
    const int x = has_draft ? a.tokens[(int64_t)b * a.K + kk] : 0;
    const double uk = has_draft ? (double)u[kk] : 0.0;
    auto tested = [&](double px, double qx, double acc) __attribute__((always_inline)) {
        if (l0) {
            out->px = px;
            out->qx = qx;
            out->acc = acc;
            out->u = uk;
            out->tested = 1;
        }
    };
    auto invalid = [&](int code) __attribute__((always_inline)) {
        if (l0) {
            out->kind = SP_INVALID;
            out->code = code;
        }
    };
    if (ri.cls == CLS_GREEDY) {
        const RecRange rr = unit_rec(a, P, CLS_GREEDY, ui.t);
        const PartSlot* s = a.parts + rr.first;
        uint64_t best = 0ull;
        for (int i = lane_id(); i < rr.count; i += kWave)
            best = s[i].keys[0] > best ? s[i].keys[0] : best;
        best = wave_max_u64(best);
        const int g = (int)key_id(best);
        if (l0 && !(has_draft && x == g)) {
            out->kind = SP_EMIT;
            out->y = g;
        }
    } else if (ri.cls == CLS_TOPK) {
        const double T = (double)ri.T, top_p = (double)ri.top_p;
        const double uf = (double)u[a.K];
        uint64_t kt, kd;
        unit_tops(a.parts, unit_rec(a, P, CLS_TOPK, ui.t), unit_rec(a, P, CLS_TOPK, ui.d), has_draft,
                  &kt, &kd);
        double p, q;
        bool keep_p, keep_q;
        if (!topk_dist_wave(kt, ri.k_eff, T, top_p, &p, &keep_p)) {
            invalid(-1);
            return;
        }
        const int id_p = (int)key_id(kt);
        double dg[4];
        int y;
        if (!has_draft) {  // the bonus token from p
            y = topk_draw_calc(p, keep_p, id_p, p, false, uf, ts, dg);
        } else {
            if (!topk_dist_wave(kd, ri.k_eff, T, top_p, &q, &keep_q)) {
                invalid(-1);
                return;
            }
            const int id_q = (int)key_id(kd);
            const double px = lookup_lane(keep_p, id_p, p, x);
            const double qx = lookup_lane(keep_q, id_q, q, x);
            const double acc = accept_prob(px, qx);
            tested(px, qx, acc);
            if (uk < acc) return;
            // the residual (p - q)+ over p's kept tokens
            const double d = p - q_of_lane(id_p, id_q, q, keep_q);
            y = topk_draw_calc(p, keep_p, id_p, d > 0.0 ? d : 0.0, true, uf, ts, dg);
        }
        if (l0) {
            out->kind = SP_EMIT;
            out->y = y;
            out->has_dy = 1;
            for (int i = 0; i < 4; i++) out->dy[i] = dg[i];
        }
    } else if (ri.cls == CLS_NUCLEUS) {
        const FnUnit ut = fn_unit_load(a.fn_unit + unit_code(a, b, kk, 0));
        FnUnit ud;
        ud.status = 0;
        float lx = 0.f, ld = 0.f;
        if (has_draft) {
            ud = fn_unit_load(a.fn_unit + unit_code(a, b, kk, 1));
            if (x >= 0 && x < a.V) {
                lx = load_one<DT>(unit_row<DT>(a, b, 0, kk), x);
                ld = load_one<DT>(unit_row<DT>(a, b, 1, kk), x);
            }
        }
        const int st = ut.status != 0 ? ut.status : (has_draft ? ud.status : 0);
        if (st != 0) {
            invalid(st == 1 ? -2 : -1);
            return;
        }
        bool draw = !has_draft;
        if (has_draft) {
            const float cb = bucket_coef(ri.T);
            const double px = (make_key(lx, (uint32_t)x) >= ut.tau)
                                  ? exp((double)nuc_t(lx, ut.la, cb) * (1.0 / 64.0)) / ut.S
                                  : 0.0;
            const double qx = (make_key(ld, (uint32_t)x) >= ud.tau)
                                  ? exp((double)nuc_t(ld, ud.la, cb) * (1.0 / 64.0)) / ud.S
                                  : 0.0;
            const double acc = accept_prob(px, qx);
            tested(px, qx, acc);
            draw = !(uk < acc);
        }
        if (l0 && draw) {
            out->kind = SP_DRAW;
            out->need = has_draft ? NEED_RESID : NEED_BONUS;
            out->mt = (double)ut.la;
            out->zt = ut.S;
            out->tau_t = ut.tau;
            out->md = (double)ud.la;
            out->zd = ud.S;
            out->tau_d = ud.tau;
        }
    } else {  // untruncated
        const double T = (double)ri.T, invT = 1.0 / T;
        const int nrec = a.ntiles * kWaves;
        float lx = 0.f, ld = 0.f;
        if (has_draft && x >= 0 && x < a.V) {
            lx = load_one<DT>(unit_row<DT>(a, b, 0, kk), x);
            ld = load_one<DT>(unit_row<DT>(a, b, 1, kk), x);
        }
        double mt, zt, md = 0.0, zd = 0.0;
        full_stats2(a.tstat + (int64_t)unit_code(a, b, kk, 0) * nrec,
                    has_draft ? a.tstat + (int64_t)unit_code(a, b, kk, 1) * nrec : nullptr, nrec,
                    invT, &mt, &zt, &md, &zd);
        if (!(mt > -INFINITY) || (has_draft && !(md > -INFINITY))) {
            invalid(-1);
            return;
        }
        bool draw = !has_draft;
        if (has_draft) {
            const double px = exp(((double)lx - mt) / T) / zt;
            const double qx = exp(((double)ld - md) / T) / zd;
            const double acc = accept_prob(px, qx);
            tested(px, qx, acc);
            draw = !(uk < acc);
        }
        if (l0 && draw) {
            out->kind = SP_DRAW;
            out->need = has_draft ? NEED_RESID : NEED_BONUS;
            out->pick = has_draft ? 0 : 1;
            out->mt = mt;
            out->zt = zt;
            out->md = md;
            out->zd = zd;
        }
    }
}

// Wave 0: the walk over slots base .. last of row b; true when the row ended.
__device__ bool spec_commit(const StepArgs& a, int b, int base, int last, const SpecSlot* slots) {
    for (int kk = base; kk <= last; kk++) {
        const SpecSlot& r = slots[kk - base];
        if (r.kind == SP_INVALID) {
            close_row_invalid(a, b, r.code);
            return true;
        }
        if (r.tested) write_accept_diag(a, b, kk, r.px, r.qx, r.acc, r.u);
        if (lane_id() != 0) {
            if (r.kind != SP_ACCEPT) return true;
            continue;
        }
        RowInfo& w = a.rows[b];
        if (r.kind == SP_ACCEPT) {
            w.acc = kk + 1;
            continue;
        }
        if (r.kind == SP_EMIT) {
            if (r.has_dy) write_final_diag(a, b, r.dy);
            emit_row(a, b, kk, r.y);
            return true;
        }
        w.need = r.need;  // SP_DRAW: the full-vocabulary draw at kk
        w.kpos = kk;
        w.mt = r.mt;
        w.zt = r.zt;
        w.md = r.md;
        w.zd = r.zd;
        w.tau_t = r.tau_t;
        w.tau_d = r.tau_d;
        if (r.pick)
            a.slist[a.B - 1 - atomicAdd(&a.pos[a.K + 1].n_pick, 1)] = b;
        else
            a.slist[atomicAdd(&a.pos[a.K + 1].n_sample, 1)] = b;
        w.status = ST_SAMPLE;
        return true;
    }
    return false;
}

// One row per wave (b_w < 0: none; rows not live at position k, and
// nucleus rows when skip_nucleus is set, do nothing), then the workgroup's
// list updates: per class region, for the draw list and for a tree verify's
// first child round, one global atomic
// reserves the space of all its rows, and each row writes its entries in
// wave order.  Every thread of the workgroup calls it (barriers inside).
// Not inlined, so that its registers are not added to those of the cut
// around it; the arguments come from their copy in device memory (a kernel
// argument passed by reference would be copied to private memory first).
// With s_slot set it decides positions k .. k + kWaves - 1 of the one row
// b_w side by side instead (wave w: position k + w; see spec_position), and
// s_base[0] tells every thread afterwards whether the row ended there (or
// was not live); a row that goes on has accepted all of them.
template <int DT>
__device__ __attribute__((noinline)) void decide_rows(const StepArgs* ga, const PosDesc* sP, int k,
                                                      int b_w,
                                                      bool skip_nucleus, DecideIntent* s_it,
                                                      int* s_base, TopkScratch* s_ts,
                                                      SpecSlot* s_slot) {
    const StepArgs& a = *ga;
    const int w = wave_id(), lane = lane_id();
    if (s_slot) {
        const int b = b_w;
        const RowInfo ri = a.rows[b];
        const bool go = ri.status == ST_LIVE && k <= ri.L && !(skip_nucleus && ri.cls == CLS_NUCLEUS);
        const int kk = k + w;
        if (go && kk <= ri.L) {
            const UnitIdx ui = unit_idx(a, ri, unit_idx_prefetch(a, b, kk), kk);
            spec_position<DT>(a, *sP, b, kk, ri, ui, s_ts[w], &s_slot[w]);
        }
        __syncthreads();
        if (w == 0) {
            const int last = k + kWaves - 1 < ri.L ? k + kWaves - 1 : ri.L;
            const bool ended = !go || spec_commit(a, b, k, last, s_slot);
            if (lane == 0) s_base[0] = ended ? 1 : 0;
        }
        __syncthreads();
        return;
    }
    if (lane == 0) {
        s_it[w].nu = 0;
        s_it[w].cls = 0;
        s_it[w].draw = 0;
        s_it[w].rnd = 0;
        s_it[w].pick = 0;
    }
    if (b_w >= 0) {
        const int b = b_w;
        const UnitIdx pre = unit_idx_prefetch(a, b, k);  // loaded with the row's info
        const RowInfo ri = a.rows[b];
        const UnitIdx ui = unit_idx(a, ri, pre, k);
        // a dense step decides position k of the rows that accepted every
        // position before it (the caller walks the positions)
        if (ri.status == ST_LIVE && k <= ri.L && !(skip_nucleus && ri.cls == CLS_NUCLEUS) &&
            (k < a.d0 || ri.acc == k)) {
            DecideIntent& it = s_it[w];
            if (ri.cls == CLS_GREEDY)
                decide_greedy(a, *sP, b, k, ri, ui, it);
            else if (ri.cls == CLS_TOPK)
                decide_topk(a, *sP, b, k, ri, ui, s_ts[w], it);
            else if (ri.cls == CLS_NUCLEUS)
                decide_nucleus<DT>(a, b, k, ri, it);
            else
                decide_full<DT>(a, b, k, ri, it);
            // no unit lists to extend: every position was in this launch
            if (k >= a.d0 && lane == 0) it.nu = 0;
        }
    }
    __syncthreads();
    // thread c < kNumCls: class region c; kNumCls: draws; kNumCls + 1: the
    // first child round of a tree verify; kNumCls + 2: draws without a pass
    if (threadIdx.x <= kNumCls + 2) {
        const int c = threadIdx.x;
        int cnt = 0;
        for (int j = 0; j < kWaves; j++)
            cnt += (c < kNumCls)       ? (s_it[j].cls == c ? s_it[j].nu : 0)
                   : c == kNumCls     ? s_it[j].draw
                   : c == kNumCls + 1 ? s_it[j].rnd
                                      : s_it[j].pick;
        int base = 0;
        if (cnt > 0)
            base = atomicAdd(c < kNumCls        ? &a.pos[k + 1].n_cls[c]
                             : c == kNumCls     ? &a.pos[a.K + 1].n_sample
                             : c == kNumCls + 1 ? &a.tcount[k * kMaxKids + 1]
                                                : &a.pos[a.K + 1].n_pick,
                             cnt);
        s_base[c] = base;
    }
    __syncthreads();
    const DecideIntent it = s_it[w];
    const int b = b_w;
    if (lane == 0 && it.nu > 0) {
        int li = s_base[it.cls];
        for (int j = 0; j < w; j++) li += s_it[j].cls == it.cls ? s_it[j].nu : 0;
        int32_t* ul = a.ulist + ((int64_t)(k + 1) * kNumCls + it.cls) * a.ustride;
        if (k + 1 == a.d0) {
            // the merged launch: every remaining position's units, target
            // then draft, their list indices in dli
            const int L = a.rows[b].L;
            for (int kk = k + 1; kk <= L; kk++) {
                const int sides = (it.cls != CLS_GREEDY && kk < L) ? 2 : 1;
                for (int side = 0; side < sides; side++) {
                    const int code = unit_code(a, b, kk, side);
                    ul[li] = code;
                    a.dli[code] = li++;
                    if (it.cls == CLS_NUCLEUS) a.fn_unit[code].rehist = 0;
                }
            }
        } else {
            ul[li] = b * 2;
            RowInfo& r = a.rows[b];
            r.li_t = li;
            if (it.nu == 2) {
                ul[li + 1] = b * 2 + 1;
                r.li_d = li + 1;
            }
            if (it.cls == CLS_NUCLEUS) {
                a.fn_unit[b * 2].rehist = 0;
                if (it.nu == 2) a.fn_unit[b * 2 + 1].rehist = 0;
            }
        }
    }
    if (lane == 0 && it.draw) {
        int i = s_base[kNumCls];
        for (int j = 0; j < w; j++) i += s_it[j].draw;
        a.slist[i] = b;
        a.rows[b].status = ST_SAMPLE;
    }
    if (lane == 0 && it.pick) {
        int i = s_base[kNumCls + 2];
        for (int j = 0; j < w; j++) i += s_it[j].pick;
        a.slist[a.B - 1 - i] = b;
        a.rows[b].status = ST_SAMPLE;
    }
    if (lane == 0 && it.rnd) {
        int i = s_base[kNumCls + 1];
        for (int j = 0; j < w; j++) i += s_it[j].rnd;
        a.tlist[a.B + i] = b;  // round 1's list
    }
}

// The classifying workgroups (plan_groups) each take a contiguous share of
// the rows: classify them, set their accept lengths and list their
// position-0 units after those of the rows before (counted again by each);
// workgroup 0 also zeroes the work counters.  The other workgroups fill the
// token, path and diagnostic outputs.  A row is invalid when T is negative,
// NaN or infinite, top_p is not > 0, draft_len is outside [0, K] or a read
// draft token is outside [0, V).
constexpr int kPlanThreads = 1024;
// Workgroups of the plan that classify: one per kPlanThreads rows (at most
// kPlanGroups) on a step whose position-0 list holds at most two units per
// row; one for a dense step or a tree verify (their rows list more units,
// or check a tree), which then works through every row.
constexpr int kPlanGroups = 16;
constexpr int kPlanRows = 4;  // rows per thread whose loads go out together
__host__ __device__ __forceinline__ int plan_groups(int64_t B, int tree, int d0) {
    if (tree || d0 == 0 || B <= kPlanThreads) return 1;
    const int64_t g = (B + kPlanThreads - 1) / kPlanThreads;
    return (int)(g < kPlanGroups ? g : kPlanGroups);
}
// The whole plan launch: those, and enough workgroups to fill the outputs of
// B rows of K + 1 positions (about 32 tokens per thread, at most 64).
__host__ __device__ __forceinline__ unsigned plan_grid(int64_t B, int64_t K, int tree, int d0) {
    const int64_t per = (int64_t)kPlanThreads * 32;
    const int64_t n = (B * (K + 1) + per - 1) / per;
    return (unsigned)plan_groups(B, tree, d0) + (unsigned)(n < 64 ? n : 64);
}

// Class of row b (CLS_ERROR when invalid; see the plan), with its draft
// length.  check_tree: also the tree checks of a tree verify (which use the
// row's scratch in nscr).
__device__ __forceinline__ int plan_class(const StepArgs& a, const int32_t* draft_len,
                                          const sv_sampler_params& prm, int b, int* L_out) {
    const int L = draft_len ? draft_len[b] : a.K;
    *L_out = L;
    const float T = prm.temperature, tp = prm.top_p;
    const int tk = prm.top_k;
    bool bad = !(T >= 0.f) || !(T < INFINITY) || !(tp > 0.f) || L < 0 || L > a.K;
    if (!bad && !a.stats) {  // the statistics read no draft tokens
        for (int j = 0; j < L; j++) {
            const int t = a.tokens[(int64_t)b * a.K + j];
            if (t < 0 || t >= a.V) bad = true;
        }
    }
    if (!bad && a.tree) {
        // nodes 1..L: parent in [0, c), depth at most max_depth, at most
        // max_kids children per node (the host loops over that many levels
        // and child rounds)
        const int32_t* par = a.parents + (int64_t)b * a.K;
        int32_t* ns = a.nscr + (int64_t)b * (a.K + 1);
        ns[0] = 0;
        for (int c = 1; c <= L && !bad; c++) {
            const int pc = par[c - 1];
            if (pc < 0 || pc >= c) {
                bad = true;
            } else {
                ns[c] = ns[pc] + 1;
                bad = ns[c] > a.max_depth;
            }
        }
        if (!bad) {
            for (int c = 0; c <= L; c++) ns[c] = 0;
            for (int c = 1; c <= L; c++) bad |= ++ns[par[c - 1]] > a.max_kids;
        }
    }
    if (bad) return CLS_ERROR;
    if (T == 0.f) return CLS_GREEDY;
    if (tk > 0 && tk < a.V) return (tk <= kMaxTopK) ? CLS_TOPK : CLS_UNSUP;
    return (tp < 1.f) ? CLS_NUCLEUS : CLS_FULL;
}
// Position-0 units of a row of class cls (>= 0) and draft length L: the
// target, and the draft unless the row is greedy (the statistics read both).
__device__ __forceinline__ int plan_units0(const StepArgs& a, int cls, int L) {
    return ((cls != CLS_GREEDY || a.stats) && 0 < L) ? 2 : 1;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(StepArgs a, const int32_t* draft_len,
                                                            const sv_sampler_params* params) {
    const int n_cls_groups = plan_groups(a.B, a.tree, a.d0);
    if ((int)blockIdx.x >= n_cls_groups) {
        // the other workgroups fill the outputs every row starts from (-1
        // tokens and path nodes, NaN diagnostics) as flat arrays, so that
        // their stores are coalesced and run beside the classification
        if (a.stats) return;  // no verify outputs
        const int nf = (int)gridDim.x - n_cls_groups, f = (int)blockIdx.x - n_cls_groups;
        const int64_t stride = (int64_t)nf * kPlanThreads;
        const int64_t i0 = (int64_t)f * kPlanThreads + threadIdx.x;
        const int64_t nt = (int64_t)a.B * (a.K + 1);
        for (int64_t i = i0; i < nt; i += stride) a.out_tokens[i] = -1;
        if (a.out_path)
            for (int64_t i = i0; i < nt; i += stride) a.out_path[i] = -1;
        if (a.diag)
            for (int64_t i = i0; i < 4 * nt; i += stride)
                a.diag[i] = __longlong_as_double(0x7FF8000000000000ll);
        return;
    }
    __shared__ int s_nc[kNumCls];    // this workgroup's region lengths (LDS counters)
    __shared__ int s_base[kNumCls];  // units the rows before this workgroup's list
    const int G = plan_groups(a.B, a.tree, a.d0), w = blockIdx.x;
    const int chunk = (a.B + G - 1) / G;
    const int r0 = w * chunk, r1 = r0 + chunk < a.B ? r0 + chunk : a.B;
    if (w == 0) {
        for (int i = threadIdx.x; i < a.K + 2; i += kPlanThreads) {
            // pos[0].n_cls is written at the end, by the last workgroup
            if (i > 0)
                for (int c = 0; c < kNumCls; c++) a.pos[i].n_cls[c] = 0;
            a.pos[i].n_sample = 0;
            a.pos[i].n_pick = 0;
        }
        if (threadIdx.x == 0) *const_cast<StepArgs*>(a.self) = a;
        // counters of split nucleus units (each launch leaves them at zero);
        // a split unit's index is below both the list length of a launch
        // (ustride) and kGrid / 2
        const int rows = a.ustride < kGrid / 2 ? a.ustride : kGrid / 2;
        for (int i = threadIdx.x; i < 2 * rows; i += kPlanThreads) a.fn_sync[i] = 0;
        if (a.tree)  // rows per (level, child round) of a tree verify
            for (int i = threadIdx.x; i < (a.K + 1) * kMaxKids; i += kPlanThreads) a.tcount[i] = 0;
    }
    for (int i = r0 + threadIdx.x; i < r1; i += kPlanThreads) a.fn_row[i] = 0;
    if (threadIdx.x < kNumCls) s_nc[threadIdx.x] = s_base[threadIdx.x] = 0;
    // The units of the rows before r0, per class, counted here again (no
    // workgroup waits for another): kPlanRows rows per thread at a time, so
    // that their loads go out together.
    if (r0 > 0) {  // (the same threads clear and then set s_base)
        int cnt[kNumCls] = {0, 0, 0, 0};
        for (int b0 = threadIdx.x; b0 < r0; b0 += kPlanThreads * kPlanRows) {
#pragma unroll
            for (int r = 0; r < kPlanRows; r++) {
                const int b = b0 + r * kPlanThreads;
                if (b < r0) {
                    int L;
                    const int cls = plan_class(a, draft_len, params[b], b, &L);
#pragma unroll
                    for (int c = 0; c < kNumCls; c++)
                        cnt[c] += (cls == c) ? plan_units0(a, cls, L) : 0;
                }
            }
        }
        __shared__ int s_red[kNumCls][kPlanThreads / kWave];
#pragma unroll
        for (int c = 0; c < kNumCls; c++) {
            const int t = (int)wave_sum((double)cnt[c]);  // exact: integers below 2^53
            if (lane_id() == 0) s_red[c][wave_id()] = t;
        }
        __syncthreads();
        if (threadIdx.x < kNumCls) {
            int t = 0;
            for (int j = 0; j < kPlanThreads / kWave; j++) t += s_red[threadIdx.x][j];
            s_base[threadIdx.x] = t;
        }
    }
    __syncthreads();
    for (int b = r0 + threadIdx.x; b < r1; b += kPlanThreads) {
        const sv_sampler_params prm = params[b];
        int L;
        const int cls = plan_class(a, draft_len, prm, b, &L);
        const float T = prm.temperature, tp = prm.top_p;
        const int tk = prm.top_k;
        RowInfo ri;
        ri.cls = cls;
        ri.L = L;
        ri.status = (cls >= 0) ? ST_LIVE : ST_ERROR;
        ri.acc = 0;
        ri.kpos = 0;
        ri.need = NEED_NONE;
        ri.k_eff = (cls == CLS_TOPK) ? tk : 0;
        ri.node = 0;
        ri.rounds = 0;
        ri.nxt = -1;
        ri.kids = (L > 0) ? 1 : 0;  // in a tree node 1's parent is node 0
        ri.pad = 0;
        ri.T = T;
        ri.top_p = tp;
        ri.li_t = ri.li_d = -1;
        ri.mt = ri.zt = ri.md = ri.zd = 0.0;
        ri.tau_t = ri.tau_d = 0ull;
        if (cls >= 0 && a.d0 == 0) {
            // a dense step (one workgroup): the units of every position,
            // target then draft
            const bool drafts = cls != CLS_GREEDY && 0 < L;
            const int nu = (L + 1) + (drafts ? L : 0);
            int li = atomicAdd(&s_nc[cls], nu);
            int32_t* ul = a.ulist + (int64_t)cls * a.ustride;
            for (int k = 0; k <= L; k++) {
                for (int side = 0; side < ((drafts && k < L) ? 2 : 1); side++) {
                    const int code = unit_code(a, b, k, side);
                    ul[li] = code;
                    a.dli[code] = li++;
                    if (cls == CLS_NUCLEUS) a.fn_unit[code].rehist = 0;
                }
            }
        } else if (cls >= 0) {
            // position-0 units (the layout the decisions use, LDS counters
            // after the rows of the workgroups before)
            const int nu = plan_units0(a, cls, L);
            const int li = s_base[cls] + atomicAdd(&s_nc[cls], nu);
            int32_t* ul = a.ulist + (int64_t)cls * a.ustride;
            ul[li] = b * 2;
            ri.li_t = li;
            if (nu == 2) {
                ul[li + 1] = b * 2 + 1;
                ri.li_d = li + 1;
            }
            if (cls == CLS_NUCLEUS) {
                a.fn_unit[b * 2].rehist = 0;
                if (nu == 2) a.fn_unit[b * 2 + 1].rehist = 0;
            }
        }
        a.rows[b] = ri;
        if (a.stats) continue;  // no verify outputs
        a.out_acc[b] = (cls == CLS_ERROR) ? -1 : (cls == CLS_UNSUP ? -2 : 0);
    }
    __syncthreads();
    if (w == G - 1 && threadIdx.x < kNumCls)
        a.pos[0].n_cls[threadIdx.x] = s_base[threadIdx.x] + s_nc[threadIdx.x];
}

}  // namespace sv
