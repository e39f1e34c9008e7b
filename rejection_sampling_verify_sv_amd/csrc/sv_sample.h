// sv_sample.h — the final draw for full-vocab rows (inverse CDF over V).
//
// Rows that ended at position kpos with a rejection draw from the normalised
// residual (p - q)+ (deniz.in "Üç düzeltmeden sonra…", section "Örnekleme
// altında doğrulama yanlıştı"; "MTPLX…" section 3.3); rows whose drafts were
// all accepted draw the bonus token from p at position L.  The walk is in
// ascending token id (the reading used throughout this library).
//
// Two steps over the list of rows that need such a draw:
//   sample_sums_kernel  the tiles of those rows split evenly over the grid:
//                       each tile's residual mass and p mass, fp64, fixed
//                       reduction trees (one partial per wave);
//   sample_pick_kernel  one workgroup per row: running sum over the chunk
//                       masses, then a block-wide fp64 prefix scan inside the
//                       chosen chunk (one 16-byte vector per thread) to find
//                       the token.
// Untruncated rows use the same exp2 terms as the row pass that produced
// their normalisers; nucleus rows the anchor-relative weights of their cut.
#pragma once

#include "sv_decide.h"

namespace sv {

struct DrawCtx {
    bool nucleus, resid;
    float mt, md, c, cb;
    double izt, izd;  // reciprocals of the normalisers (no division per token)
    uint64_t tau_t, tau_d;
    int rounds;             // tree verify: residual masses known before this draw
    const double* wchain;   // their values
};

// A tree verify's row whose node had `rounds` children rejected before the
// current one: r_0 = p and r_i = (r_{i-1} - q)+ / W_i (r_{i-1} when W_i <= 0)
// at one token, from its normalised probabilities.
__device__ __forceinline__ double resid_chain(double pe, double qe, int rounds,
                                              const double* wchain) {
    double r = pe;
    for (int i = 0; i < rounds; i++) {
        const double W = wchain[i];
        const double d = r - qe;
        r = W > 0.0 ? (d > 0.0 ? d : 0.0) / W : r;
    }
    return r;
}

__device__ __forceinline__ DrawCtx draw_ctx(const StepArgs& a, int b, const RowInfo& ri,
                                            bool resid) {
    DrawCtx x;
    x.nucleus = ri.cls == CLS_NUCLEUS;
    x.resid = resid;
    x.rounds = ri.rounds;
    x.wchain = a.wchain + (int64_t)b * kMaxKids;
    x.mt = (float)ri.mt;
    x.md = (float)ri.md;
    x.c = exp2_coef(ri.T);
    x.cb = bucket_coef(ri.T);
    x.izt = 1.0 / ri.zt;
    x.izd = ri.zd != 0.0 ? 1.0 / ri.zd : 0.0;
    x.tau_t = ri.tau_t;
    x.tau_d = ri.tau_d;
    return x;
}

// Draw weights of token `id`: the residual (p - q)+ and the target weight
// (unnormalised exp2 terms on untruncated rows; on nucleus rows the kept
// token's weight exp(t / 64) over the kept mass, with mt / md holding the
// anchors).
__device__ __forceinline__ void draw_weights(const DrawCtx& x, float lt, float ld, uint32_t id,
                                             double* wr, double* wp) {
    if (x.rounds > 0) {
        // tree verify after earlier rejections at this node: the residual of
        // the residual chain (r_R - q)+ and, for its fallback, r_R itself
        double pe, qe;
        if (x.nucleus) {
            pe = (make_key(lt, id) >= x.tau_t)
                     ? (double)fast_exp2(nuc_t(lt, x.mt, x.cb) * kLog2e64) * x.izt
                     : 0.0;
            qe = (make_key(ld, id) >= x.tau_d)
                     ? (double)fast_exp2(nuc_t(ld, x.md, x.cb) * kLog2e64) * x.izd
                     : 0.0;
        } else {
            pe = (double)fast_exp2((lt - x.mt) * x.c) * x.izt;
            qe = (double)fast_exp2((ld - x.md) * x.c) * x.izd;
        }
        const double r = resid_chain(pe, qe, x.rounds, x.wchain);
        const double d = r - qe;
        *wr = d > 0.0 ? d : 0.0;
        *wp = r;
        return;
    }
    if (x.nucleus) {
        // only tokens kept on the target side carry mass in either sum
        *wp = 0.0;
        *wr = 0.0;
        if (make_key(lt, id) >= x.tau_t) {
            const double p = (double)fast_exp2(nuc_t(lt, x.mt, x.cb) * kLog2e64) * x.izt;
            *wp = p;
            if (x.resid) {
                const double q = (make_key(ld, id) >= x.tau_d)
                                     ? (double)fast_exp2(nuc_t(ld, x.md, x.cb) * kLog2e64) * x.izd
                                     : 0.0;
                const double d = p - q;
                *wr = d > 0.0 ? d : 0.0;
            }
        }
    } else {
        const float ep = fast_exp2((lt - x.mt) * x.c);
        *wp = (double)ep;
        if (x.resid) {
            const float eq = fast_exp2((ld - x.md) * x.c);
            const double d = fma((double)ep, x.izt, -((double)eq * x.izd));
            *wr = d > 0.0 ? d : 0.0;
        } else {
            *wr = 0.0;
        }
    }
}

// Element i of a raw tile (i = j kVec + e: element e of the thread's vector j).
template <int DT>
__device__ __forceinline__ float raw_elem(const RawTile& r, int i) {
    constexpr int kVec = Elt<DT>::kVec;
    const u32x4& q = r.q[i / kVec];
    if constexpr (DT == SV_F32) {
        const int e = i % kVec;
        return __uint_as_float(e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w);
    } else {
        const int e = (i % kVec) >> 1;
        const uint32_t w = e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
        return (i & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

// The tiles [start, end) of a row, or of two rows in lockstep (kTwo), for the
// draw masses: full tiles are double-buffered as in stream_range and reach
// the body as their raw loads, each element converted where the body uses it,
// so no unpacked copy of a tile sits beside the loads in flight (that copy
// held the kernel to two or three workgroups per compute unit); the ragged
// tail comes as floats, -inf past end.  body(gt, gd, t0): gt(i), gd(i) are
// element i of the tile at t0 in the two rows (gd gives -inf without kTwo).
template <int DT, bool kAligned, bool kTwo, class Body>
__device__ __forceinline__ void stream_draw(const void* ra, const void* rb, int64_t start,
                                            int64_t end, Body&& body) {
    using TS = TileShape<DT>;
    int64_t t0 = start;
    if constexpr (kAligned) {
        const int64_t full_end = start + ((end - start) / TS::kTile) * TS::kTile;
        if (t0 < full_end) {
            const int64_t nt = (full_end - t0) / TS::kTile;
            const int64_t last = full_end - TS::kTile;
            RawTile A, A2, B, B2;
            auto run = [&](const RawTile& X, const RawTile& X2, int64_t at)
                           __attribute__((always_inline)) {
                body([&](int i) __attribute__((always_inline)) { return raw_elem<DT>(X, i); },
                     [&](int i) __attribute__((always_inline)) {
                         if constexpr (kTwo)
                             return raw_elem<DT>(X2, i);
                         else
                             return -INFINITY;
                     },
                     at);
            };
            issue_tile<DT>(ra, t0, A);
            if constexpr (kTwo) issue_tile<DT>(rb, t0, A2);
            for (int64_t p = nt >> 1; p > 0; --p) {
                issue_tile<DT>(ra, t0 + TS::kTile, B);
                if constexpr (kTwo) issue_tile<DT>(rb, t0 + TS::kTile, B2);
                __builtin_amdgcn_sched_barrier(0);
                run(A, A2, t0);
                const int64_t tn = t0 + 2 * TS::kTile;
                issue_tile<DT>(ra, tn <= last ? tn : last, A);
                if constexpr (kTwo) issue_tile<DT>(rb, tn <= last ? tn : last, A2);
                __builtin_amdgcn_sched_barrier(0);
                run(B, B2, t0 + TS::kTile);
                t0 += 2 * TS::kTile;
            }
            if (nt & 1) {
                run(A, A2, t0);
                t0 += TS::kTile;
            }
        }
    }
    float va[TS::kE], vb[TS::kE];
    while (t0 < end) {
        if constexpr (kAligned) {
            load_tile_tail<DT>(ra, t0, end, va);
            if constexpr (kTwo) load_tile_tail<DT>(rb, t0, end, vb);
        } else {
            load_tile_partial<DT>(ra, t0, end, va);
            if constexpr (kTwo) load_tile_partial<DT>(rb, t0, end, vb);
        }
        body([&](int i) __attribute__((always_inline)) { return va[i]; },
             [&](int i) __attribute__((always_inline)) {
                 if constexpr (kTwo)
                     return vb[i];
                 else
                     return -INFINITY;
             },
             t0);
        t0 += TS::kTile;
    }
}

// One piece of a row's draw masses: per (tile, wave) the sums of the
// residual weights and of the target weights that w(lt, ld, id, &wr, &wp)
// gives, fp64, in element order then the fixed DPP tree.  kTwo false: the
// target row alone (a bonus draw; w gets -inf for ld).
template <int DT, bool kAligned, bool kTwo, class W>
__device__ __forceinline__ void draw_sums(const void* trow, const void* drow, int64_t start,
                                          int64_t end, double2* out, W&& w) {
    using TS = TileShape<DT>;
    stream_draw<DT, kAligned, kTwo>(trow, drow, start, end,
                                    [&](auto&& gt, auto&& gd, int64_t t0)
                                        __attribute__((always_inline)) {
        // elements past `end` read as -inf and weigh 0
        double sr = 0.0, sp = 0.0;
        uint32_t id0 = (uint32_t)elem_id<DT>(t0, 0);
        asm volatile("" : "+v"(id0));  // keeps 16-32 ids from being hoisted
#pragma unroll
        for (int i = 0; i < TS::kE; i++) {
            constexpr int kVec = Elt<DT>::kVec;
            const uint32_t id = id0 + (uint32_t)((i / kVec) * kThreads * kVec + i % kVec);
            double wr, wp;
            w(gt(i), gd(i), id, &wr, &wp);
            sr += wr;
            sp += wp;
            // four elements at a time: the fp64 terms of all of them would
            // otherwise be live at once
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        sr = wave_sum(sr);
        sp = wave_sum(sp);
        if (lane_id() == 0) {
            double2 r;
            r.x = sr;
            r.y = sp;
            out[(t0 / TS::kTile) * kWaves + wave_id()] = r;
        }
    });
}

// The workgroups split the tiles of the listed rows evenly; every wave leaves
// its partial masses of each tile at chunks[(b*ntiles + tile)*kWaves + wave].
// The rows: those that draw over the full vocabulary at the end (list slist,
// count pos[K+1].n_sample), or, in a tree verify, those that need the mass of
// a residual before testing their node's next child (round lists).  Each
// kind of draw streams through a loop of its own (the weights of
// draw_weights, specialised): a bonus draw reads the target row alone, and no
// element branches on the kind.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void sample_sums_kernel(StepArgs a, const int32_t* list,
                                                               const int32_t* count) {
    using TS = TileShape<DT>;
    const int n = *count;
    const int64_t T = (int64_t)n * a.ntiles;
    int64_t t = flat_begin(T, gridDim.x, blockIdx.x);
    const int64_t t_end = flat_begin(T, gridDim.x, blockIdx.x + 1);
    while (t < t_end) {
        const int si = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)si * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        t += tu1 - tu0;
        const int b = list[si];
        const RowInfo& ri = a.rows[b];
        const int kpos = ri.kpos;
        const DrawCtx x = draw_ctx(a, b, ri, ri.need != NEED_BONUS);
        const void* trow = unit_row<DT>(a, b, 0, kpos);
        const void* drow = x.resid ? unit_row<DT>(a, b, 1, kpos) : nullptr;
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        double2* out = a.chunks + (int64_t)b * a.ntiles * kWaves;
        if (x.rounds > 0) {  // a tree verify's residual chain
            draw_sums<DT, kAligned, true>(trow, x.resid ? drow : trow, start, end, out,
                                          [&](float lt, float ld, uint32_t id, double* wr,
                                              double* wp) __attribute__((always_inline)) {
                draw_weights(x, lt, ld, id, wr, wp);
            });
        } else if (x.nucleus) {
            const float mt = x.mt, md = x.md, cb = x.cb;
            const double izt = x.izt, izd = x.izd;
            const uint64_t tau_t = x.tau_t, tau_d = x.tau_d;
            auto pw = [&](float lt, uint32_t id) __attribute__((always_inline)) {
                return make_key(lt, id) >= tau_t
                           ? (double)fast_exp2(nuc_t(lt, mt, cb) * kLog2e64) * izt
                           : 0.0;
            };
            if (x.resid)
                draw_sums<DT, kAligned, true>(trow, drow, start, end, out,
                                              [&](float lt, float ld, uint32_t id, double* wr,
                                                  double* wp) __attribute__((always_inline)) {
                    // only tokens kept on the target side carry mass
                    const double p = pw(lt, id);
                    const double q = (p > 0.0 && make_key(ld, id) >= tau_d)
                                         ? (double)fast_exp2(nuc_t(ld, md, cb) * kLog2e64) * izd
                                         : 0.0;
                    const double d = p - q;
                    *wp = p;
                    *wr = d > 0.0 ? d : 0.0;
                });
            else
                draw_sums<DT, kAligned, false>(trow, nullptr, start, end, out,
                                               [&](float lt, float, uint32_t id, double* wr,
                                                   double* wp) __attribute__((always_inline)) {
                    *wp = pw(lt, id);
                    *wr = 0.0;
                });
        } else {
            const float mt = x.mt, md = x.md, c = x.c;
            const double izt = x.izt, izd = x.izd;
            if (x.resid)
                draw_sums<DT, kAligned, true>(trow, drow, start, end, out,
                                              [&](float lt, float ld, uint32_t, double* wr,
                                                  double* wp) __attribute__((always_inline)) {
                    const float ep = fast_exp2((lt - mt) * c);
                    const float eq = fast_exp2((ld - md) * c);
                    const double d = fma((double)ep, izt, -((double)eq * izd));
                    *wp = (double)ep;
                    *wr = d > 0.0 ? d : 0.0;
                });
            else
                draw_sums<DT, kAligned, false>(trow, nullptr, start, end, out,
                                               [&](float lt, float, uint32_t, double* wr,
                                                   double* wp) __attribute__((always_inline)) {
                    *wp = (double)fast_exp2((lt - mt) * c);
                    *wr = 0.0;
                });
        }
    }
}

// The pick runs one thread per 16-byte vector of the chosen chunk (a tile),
// so that each thread weighs and walks kVec tokens only.
constexpr int kPickThreads = kThreads * kLoads;
constexpr int kPickWaves = kPickThreads / kWave;

// The kVec elements from i0 of a row; elements at or past end read as -inf.
template <int DT, bool kAligned>
__device__ __forceinline__ void load_vec(const void* row, int64_t i0, int64_t end,
                                         float (&v)[Elt<DT>::kVec]) {
    constexpr int kVec = Elt<DT>::kVec;
    if (kAligned && i0 + kVec <= end) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const char*>(row) +
                                                        i0 * Elt<DT>::kSize);
        if constexpr (DT == SV_F32) {
            v[0] = __uint_as_float(q.x);
            v[1] = __uint_as_float(q.y);
            v[2] = __uint_as_float(q.z);
            v[3] = __uint_as_float(q.w);
        } else {
            v[0] = bf16_lo(q.x);
            v[1] = bf16_hi(q.x);
            v[2] = bf16_lo(q.y);
            v[3] = bf16_hi(q.y);
            v[4] = bf16_lo(q.z);
            v[5] = bf16_hi(q.z);
            v[6] = bf16_lo(q.w);
            v[7] = bf16_hi(q.w);
        }
    } else {  // the vector that straddles end, or a row that is not aligned
#pragma unroll
        for (int e = 0; e < kVec; e++) {
            const int64_t i = i0 + e;
            const float x = load_one<DT>(row, i < end ? i : end - 1);
            v[e] = i < end ? x : -INFINITY;
        }
    }
}

// One workgroup (kPickThreads): the drawn token of row b from its chunk masses,
// or, for an untruncated bonus draw (stats), from the row pass's records of
// the row: the target mass of a (tile, wave) is its sum of exp2((t - m_w) c)
// rescaled by exp2((m_w - mt) c), the same terms the sums kernel would add up
// one by one (each term rounded apart, so the chunk's own running sums below
// may end a little off its record; the fallback to the chunk's last token
// covers that).
template <int DT, bool kAligned, bool stats>
__device__ __forceinline__ void pick_row(const StepArgs& a, int b) {
    using TS = TileShape<DT>;
    constexpr int kVec = Elt<DT>::kVec;
    static_assert(kPickThreads * kVec == TS::kTile, "one vector per thread covers a chunk");
    __shared__ int s_chunk, s_lastc, s_best, s_last;
    __shared__ double s_base, s_lbase;
    __shared__ double s_tmp[2 * kPickWaves];
    __shared__ double s_lo, s_hi, s_wy;
    const RowInfo ri = a.rows[b];
    const bool resid = ri.need == NEED_RESID;
    const double u = (double)a.uniforms[(int64_t)b * (a.K + 1) + a.K];
    // chunk masses: thread t sums the tiles [c0, c1), one chunk = one tile
    // (its kWaves partials in wave order); block scans give the running sums
    const double2* cs = a.chunks + (int64_t)b * a.ntiles * kWaves;
    auto chunk_pair = [&](int c, int q) __attribute__((always_inline)) {
        if constexpr (!stats) return cs[c * kWaves + q];
        const FullStat r =
            a.tstat[((int64_t)unit_code(a, b, ri.kpos, 0) * a.ntiles + c) * kWaves + q];
        double2 m;
        m.x = 0.0;
        m.y = r.m > -INFINITY ? r.s * (double)fast_exp2((r.m - (float)ri.mt) * exp2_coef(ri.T))
                              : 0.0;
        return m;
    };
    const int per = (a.ntiles + kPickThreads - 1) / kPickThreads;
    const int c0 = min(a.ntiles, (int)threadIdx.x * per), c1 = min(a.ntiles, c0 + per);
    double mine2[2] = {0.0, 0.0};  // residual, target
    double r0 = 0.0, p0 = 0.0;      // the first tile's masses, kept (later ones are read again)
    for (int c = c0; c < c1; c++) {
        double wr = 0.0, wp = 0.0;
        for (int q = 0; q < kWaves; q++) {
            const double2 m = chunk_pair(c, q);
            wr += m.x;
            wp += m.y;
        }
        if (c == c0) {
            r0 = wr;
            p0 = wp;
        }
        mine2[0] += wr;
        mine2[1] += wp;
    }
    double ex2[2], tot2[2];
    block_exclusive_scan_n<2, kPickWaves>(mine2, s_tmp, ex2, tot2);
    const bool use_r = resid && tot2[0] > 0.0;
    const double W = use_r ? tot2[0] : tot2[1];
    const double target = u * W;
    if (threadIdx.x == 0) {
        s_chunk = 0x7FFFFFFF;
        s_lastc = -1;
        s_best = 0x7FFFFFFF;
        s_last = -1;
        s_lo = s_hi = s_wy = 0.0;
    }
    __syncthreads();
    double S = use_r ? ex2[0] : ex2[1], my_base = 0.0, my_lbase = 0.0;
    int my_chunk = -1, my_last = -1;
    for (int c = c0; c < c1; c++) {
        double wc = use_r ? r0 : p0;
        if (c != c0) {
            wc = 0.0;
            for (int q = 0; q < kWaves; q++) {
                const double2 m = chunk_pair(c, q);
                wc += use_r ? m.x : m.y;
            }
        }
        if (!(wc > 0.0)) continue;
        const double before = S;
        S += wc;
        my_last = c;
        my_lbase = before;
        if (my_chunk < 0 && target < S) {
            my_chunk = c;
            my_base = before;
        }
    }
    {  // one LDS atomic per wave
        const int wc = wave_min_i32(my_chunk >= 0 ? my_chunk : 0x7FFFFFFF);
        const int wl = wave_max_i32(my_last);
        if (lane_id() == 0) {
            if (wc != 0x7FFFFFFF) atomicMin(&s_chunk, wc);
            if (wl >= 0) atomicMax(&s_lastc, wl);
        }
    }
    __syncthreads();
    // rounding can leave the target past every running sum: then the last
    // chunk with positive mass is used
    if (s_chunk != 0x7FFFFFFF && my_chunk == s_chunk) s_base = my_base;
    if (s_chunk == 0x7FFFFFFF && my_last >= 0 && my_last == s_lastc) s_lbase = my_lbase;
    __syncthreads();
    if (s_chunk == 0x7FFFFFFF) {
        if (threadIdx.x == 0) {
            s_chunk = s_lastc;
            s_base = s_lbase;
        }
        __syncthreads();
    }
    if (s_chunk < 0) {  // no positive mass anywhere: only reachable on corrupt stats
        if (threadIdx.x == 0) {
            a.out_acc[b] = -1;
            a.rows[b].status = ST_ERROR;
        }
        __syncthreads();
        return;
    }
    const int kpos = ri.kpos;
    const DrawCtx x = draw_ctx(a, b, ri, resid);
    const void* trow = unit_row<DT>(a, b, 0, kpos);
    const void* drow = x.resid ? unit_row<DT>(a, b, 1, kpos) : nullptr;
    // the chosen chunk, thread t's vector at t kVec: thread order is id order
    const int64_t cstart = (int64_t)s_chunk * TS::kTile;
    const int64_t cend = cstart + TS::kTile < a.V ? cstart + TS::kTile : a.V;
    const int64_t i0 = cstart + (int64_t)threadIdx.x * kVec;
    float lt[kVec], ld[kVec];
    load_vec<DT, kAligned>(trow, i0, cend, lt);
    if (x.resid) {
        load_vec<DT, kAligned>(drow, i0, cend, ld);
    } else {
#pragma unroll
        for (int e = 0; e < kVec; e++) ld[e] = 0.f;
    }
    double w[kVec];
    // the weights, one loop per kind of draw (the kind is the row's)
    auto fill = [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < kVec; e++) {
            const int64_t id = i0 + e;
            double wr, wp;
            f(lt[e], ld[e], (uint32_t)id, &wr, &wp);
            w[e] = id < cend ? (use_r ? wr : wp) : 0.0;
        }
    };
    if (stats) {  // an untruncated bonus draw
        const float mt = x.mt, c = x.c;
        fill([&](float lt, float, uint32_t, double* wr, double* wp)
                 __attribute__((always_inline)) {
            *wp = (double)fast_exp2((lt - mt) * c);
            *wr = 0.0;
        });
    } else if (x.rounds > 0) {
        fill([&](float lt, float ld, uint32_t id, double* wr, double* wp)
                 __attribute__((always_inline)) { draw_weights(x, lt, ld, id, wr, wp); });
    } else if (x.nucleus) {
        const float mt = x.mt, md = x.md, cb = x.cb;
        const double izt = x.izt, izd = x.izd;
        const uint64_t tau_t = x.tau_t, tau_d = x.tau_d;
        if (x.resid)
            fill([&](float lt, float ld, uint32_t id, double* wr, double* wp)
                     __attribute__((always_inline)) {
                const double p = make_key(lt, id) >= tau_t
                                     ? (double)fast_exp2(nuc_t(lt, mt, cb) * kLog2e64) * izt
                                     : 0.0;
                const double q = (p > 0.0 && make_key(ld, id) >= tau_d)
                                     ? (double)fast_exp2(nuc_t(ld, md, cb) * kLog2e64) * izd
                                     : 0.0;
                const double d = p - q;
                *wp = p;
                *wr = d > 0.0 ? d : 0.0;
            });
        else
            fill([&](float lt, float, uint32_t id, double* wr, double* wp)
                     __attribute__((always_inline)) {
                *wp = make_key(lt, id) >= tau_t
                          ? (double)fast_exp2(nuc_t(lt, mt, cb) * kLog2e64) * izt
                          : 0.0;
                *wr = 0.0;
            });
    } else {
        const float mt = x.mt, md = x.md, c = x.c;
        const double izt = x.izt, izd = x.izd;
        if (x.resid)
            fill([&](float lt, float ld, uint32_t, double* wr, double* wp)
                     __attribute__((always_inline)) {
                const float ep = fast_exp2((lt - mt) * c);
                const float eq = fast_exp2((ld - md) * c);
                const double d = fma((double)ep, izt, -((double)eq * izd));
                *wp = (double)ep;
                *wr = d > 0.0 ? d : 0.0;
            });
        else
            fill([&](float lt, float, uint32_t, double* wr, double* wp)
                     __attribute__((always_inline)) {
                *wp = (double)fast_exp2((lt - mt) * c);
                *wr = 0.0;
            });
    }
    // running sums: a block scan over the threads' vector sums
    double m[1] = {0.0}, ex[1], tot[1];
#pragma unroll
    for (int e = 0; e < kVec; e++) m[0] += w[e];
    block_exclusive_scan_n<1, kPickWaves>(m, s_tmp, ex, tot);
    int found = -1;
    double f_before = 0.0, f_after = 0.0, f_w = 0.0;
    int lastpos = -1;
    double l_before = 0.0, l_after = 0.0, l_w = 0.0;
    S = s_base + ex[0];
#pragma unroll
    for (int e = 0; e < kVec; e++) {
        if (!(w[e] > 0.0)) continue;
        const double before = S;
        S += w[e];
        lastpos = e;
        l_before = before;
        l_after = S;
        l_w = w[e];
        if (found < 0 && target < S) {
            found = e;
            f_before = before;
            f_after = S;
            f_w = w[e];
        }
    }
    const int f_id = found >= 0 ? (int)(i0 + found) : -1;
    const int l_id = lastpos >= 0 ? (int)(i0 + lastpos) : -1;
    // rounding can push the target past this chunk's own running sums;
    // then the chunk's last positive-weight token is taken (margin 0)
    {  // one LDS atomic per wave
        const int wf = wave_min_i32(found >= 0 ? f_id : 0x7FFFFFFF);
        const int wl = wave_max_i32(l_id);
        if (lane_id() == 0) {
            if (wf != 0x7FFFFFFF) atomicMin(&s_best, wf);
            if (wl >= 0) atomicMax(&s_last, wl);
        }
    }
    __syncthreads();
    const bool fallback = s_best == 0x7FFFFFFF;
    const int y = fallback ? s_last : s_best;
    if (!fallback && found >= 0 && f_id == y) {
        s_lo = f_before;
        s_hi = f_after;
        s_wy = f_w;
    } else if (fallback && lastpos >= 0 && l_id == y) {
        s_lo = l_before;
        s_hi = l_after;
        s_wy = l_w;
    }
    int32_t* o = a.out_tokens + (int64_t)b * (a.K + 1);
    if (y >= 0 && !a.tree)  // the accepted drafts, one per thread
        for (int j = threadIdx.x; j < kpos; j += kPickThreads) o[j] = a.tokens[(int64_t)b * a.K + j];
    __syncthreads();
    if (threadIdx.x == 0) {
        if (a.diag) {
            double* dg = a.diag + (int64_t)b * 4 * (a.K + 1) + 4 * a.K;
            const double lo = s_lo / W, hi = s_hi / W;
            const double d1 = u - lo, d2 = hi - u;
            dg[0] = s_wy / W;
            dg[1] = lo;
            dg[2] = hi;
            dg[3] = fallback ? 0.0 : (d1 < d2 ? d1 : d2);
        }
        if (y < 0) {
            a.out_acc[b] = -1;
            a.rows[b].status = ST_ERROR;
            if (a.tree) {  // the walk wrote its accepted tokens and nodes already
                for (int j = 0; j <= a.K; j++) o[j] = -1;
                if (a.out_path)
                    for (int j = 0; j <= a.K; j++) a.out_path[(int64_t)b * (a.K + 1) + j] = -1;
            }
        } else if (a.tree) {
            // tree verify: kpos is the node, the accepted path's length is acc
            o[ri.acc] = y;
            a.out_acc[b] = ri.acc;
            a.rows[b].status = ST_DONE;
        } else {
            o[kpos] = y;
            a.out_acc[b] = kpos;
            a.rows[b].acc = kpos;
            a.rows[b].status = ST_DONE;
        }
    }
    __syncthreads();
}
// One workgroup per row that draws over the full vocabulary.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kPickThreads) void sample_pick_kernel(StepArgs a) {
    // the rows whose masses the sums kernel wrote, then (from the list's far
    // end) the untruncated bonus draws, whose masses come from the row pass
    const int ns = a.pos[a.K + 1].n_sample, n = ns + a.pos[a.K + 1].n_pick;
    int si = blockIdx.x;
    for (; si < ns; si += gridDim.x) {
        pick_row<DT, kAligned, false>(a, a.slist[si]);
        __syncthreads();
    }
    for (; si < n; si += gridDim.x) {
        pick_row<DT, kAligned, true>(a, a.slist[a.B - 1 - (si - ns)]);
        __syncthreads();
    }
}

}  // namespace sv
