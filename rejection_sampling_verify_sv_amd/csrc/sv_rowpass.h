// sv_rowpass.h — the streaming pass over logits rows (the HBM-bound step).
//
// The workgroups split the tiles of the units live at position k evenly.
// A workgroup reads its tiles exactly once, in 16-byte coalesced,
// double-buffered vectors, and leaves one small record per unit it touches:
//   * greedy rows:   the best (logit, lowest id) key of the segment;
//   * top-k rows:    the segment's best 64 keys, descending (k <= 64);
//   * full-vocab:    per (tile, wave): {max m, sum of exp((l - m) / T)};
//   * nucleus rows:  the segment's fixed-point mass histogram over the
//                    unit's anchor window (see sv_device.h) and its max.
// Selection uses raw logits (the ranking does not depend on T > 0), so the
// candidate sets are exact; probabilities are formed later in fp64.
//
// Top-k selection is per wave and free of workgroup barriers while streaming:
// each wave keeps its running top-64 list in registers (one key per lane),
// skips a tile with one max and one ballot when no lane holds a value above
// the list's k-th key, and otherwise compacts candidates into a small
// wave-private LDS buffer with ballot prefix counts, merging 64 at a time with
// a wave bitonic sort and a bitonic merge.
//
// Coalesced single reads follow the read-coalescing technique described on
// "Apple Silikon İçin Cihaz Üstü Çıkarımı Optimize Etme", section "Dikkat
// önbelleği okumalarını birleştirin" (neighbouring lanes ask for neighbouring
// bytes); the selection rule itself is deniz.in "Üç düzeltmeden sonra…",
// section "Kesme her iki tarafta eşleşmek zorunda" (same top_k on both sides).
#pragma once

#include "sv_device.h"

namespace sv {

struct RowpassSmem {
    uint64_t cbuf[kWaves][kCandBuf];
    uint64_t lists[kWaves][kWave];
    uint64_t red[kWaves];
    uint64_t wthr[kWaves];  // each wave's current k-th key in this piece
    uint64_t wq[kWaves];    // a key that at least ceil(k/4) of the wave's elements reach
};

// Running top-64 of one wave.
struct WaveTopk {
    uint64_t lst;  // this lane's entry of the list (descending over lanes)
    uint64_t thr;  // keys <= thr cannot be in the piece's top-k (same in every lane)
    int cnt;       // keys waiting in the wave's buffer (same in every lane)
};

// A threshold every wave of the workgroup may use for this piece, from what
// the waves published:
//   * a wave's k-th key: the wave holds k elements at or above it, so the
//     piece's k-th key is at least that large;
//   * the smallest of the four wq keys: each wave holds ceil(k/4) elements at
//     or above its wq key and the waves' elements are distinct, so together
//     they hold k elements at or above the smallest one.
// Published values only grow, so a stale read is merely a weaker bound.
__device__ __forceinline__ uint64_t shared_thr(const RowpassSmem& sm) {
    uint64_t t = lds_load_relaxed(&sm.wthr[0]);
    uint64_t q = lds_load_relaxed(&sm.wq[0]);
#pragma unroll
    for (int i = 1; i < kWaves; i++) {
        const uint64_t x = lds_load_relaxed(&sm.wthr[i]);
        const uint64_t y = lds_load_relaxed(&sm.wq[i]);
        t = x > t ? x : t;
        q = y < q ? y : q;
    }
    // keys equal to the smallest wq key may still belong to the top k
    return (q > 0ull && q - 1ull > t) ? q - 1ull : t;
}

// v[i] for a per-lane index i: a tree of selects on the bits of i.
template <int N>
__device__ __forceinline__ float pick_elem(const float (&v)[N], int i) {
    static_assert((N & (N - 1)) == 0, "power of two");
    float t[N];
#pragma unroll
    for (int j = 0; j < N; j++) t[j] = v[j];
#pragma unroll
    for (int w = N / 2, b = 0; w >= 1; w /= 2, b++) {
#pragma unroll
        for (int j = 0; j < w; j++) t[j] = ((i >> b) & 1) ? t[2 * j + 1] : t[2 * j];
    }
    return t[0];
}

// Buffered candidates hold the raw float bits and the id; the ranking key is
// formed when they are merged, so nothing per element has to stay in
// registers while candidates are appended.
__device__ __forceinline__ uint64_t make_raw(float f, uint32_t id) {
    return ((uint64_t)__float_as_uint(f) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint64_t raw_to_key(uint64_t r) {
    return ((uint64_t)ord32(__uint_as_float((uint32_t)(r >> 32))) << 32) | (r & 0xFFFFFFFFull);
}

// Merge up to 64 buffered candidates into the list; publish the new k-th key.
__device__ __forceinline__ void wt_flush(WaveTopk& st, uint64_t* cbuf, int k_eff, RowpassSmem& sm) {
    const int lane = lane_id();
    wave_lds_sync();
    const int take = st.cnt < kWave ? st.cnt : kWave;
    const int left = st.cnt - take;
    uint64_t c = lane < take ? raw_to_key(cbuf[lane]) : 0ull;
    const uint64_t rest = lane < left ? cbuf[kWave + lane] : 0ull;
    wave_lds_sync();
    if (lane < left) cbuf[lane] = rest;
    st.cnt = left;
    st.lst = wave_merge_top_asc(st.lst, wave_sort_asc(c));
    const uint64_t kth = lane_value(st.lst, k_eff - 1);
    const uint64_t qth = lane_value(st.lst, (k_eff + kWaves - 1) / kWaves - 1);
    if (lane == 0 && qth != 0ull) lds_store_relaxed(&sm.wq[wave_id()], qth);
    if (kth > st.thr) {
        st.thr = kth;
        if (lane == 0) lds_store_relaxed(&sm.wthr[wave_id()], kth);
    }
}

// Top-k of one piece.  A tile is skipped after one max and one ballot when
// no lane holds a value at or above the floor of the threshold; otherwise
// every lane marks its candidates in a bit mask and the wave appends them to
// its LDS buffer in rounds (one prefix count per round, no per-element
// ballots), merging 64 at a time.
template <int DT, bool kAligned>
__device__ __forceinline__ void seg_topk(const void* row, int64_t start, int64_t end, int k_eff,
                                         RowpassSmem& sm, PartSlot* out) {
    using TS = TileShape<DT>;
    static_assert(TS::kE <= 32, "candidate mask is 32 bits");
    const int w = wave_id(), lane = lane_id();
    uint64_t* cbuf = sm.cbuf[w];
    if (lane == 0) {
        sm.wthr[w] = 0ull;
        sm.wq[w] = 0ull;
    }
    __syncthreads();  // no wave reads a threshold left by the previous piece
    WaveTopk st;
    st.lst = 0ull;
    st.thr = 0ull;
    st.cnt = 0;
    bool first = true;
    stream_range<DT, kAligned>(row, start, end, [&](float (&v)[TS::kE], int64_t t0, bool full)
                                                    __attribute__((always_inline)) {
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        if (first) {
            // The k-th largest of the lanes' best keys is reached by k
            // distinct elements of this wave, so every key of the wave's
            // top-k is at least that large.
            first = false;
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const bool valid = full || elem_id<DT>(t0, i) < end;
                if (best == 0ull && valid && v[i] == vmax)
                    best = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
            }
            const uint64_t sl = wave_sort_desc(best);
            const uint64_t th = lane_value(sl, k_eff - 1);
            const uint64_t thq = lane_value(sl, (k_eff + kWaves - 1) / kWaves - 1);
            if (th > 0ull && th - 1ull > st.thr) st.thr = th - 1ull;
            if (lane == 0 && thq != 0ull) lds_store_relaxed(&sm.wq[w], thq);
        }
        if (__ballot(vmax >= thr_floor(st.thr)) == 0ull) return;
        const uint64_t tsh = shared_thr(sm);
        if (tsh > st.thr) st.thr = tsh;
        float fl = thr_floor(st.thr);
        // masks are built by shifting in one bit per element (highest index
        // first) so that no per-element constant has to live in a register
        uint32_t bits = 0u;
#pragma unroll
        for (int i = TS::kE - 1; i >= 0; i--) {
            const bool valid = full || elem_id<DT>(t0, i) < end;
            bits = (bits << 1) | (valid && v[i] >= fl ? 1u : 0u);
        }
        while (__ballot(bits != 0u) != 0ull) {
            int total;
            const uint32_t c = (uint32_t)__popc(bits);
            const int excl = wave_excl_count(c, &total);
            // this lane's candidates that still fit in the buffer
            int room = kCandBuf - (st.cnt + excl);
            room = room < 0 ? 0 : room;
            const int nw = (int)c < room ? (int)c : room;
            // the ids are formed inside the loop: hoisting 16-32 keys out of
            // it would cost registers for the whole streaming loop
            uint32_t id0 = (uint32_t)elem_id<DT>(t0, 0);
            asm volatile("" : "+v"(id0));
            const int pos = st.cnt + excl;
            // one iteration per candidate this lane writes (lanes hold few of
            // them once the threshold has risen), element picked by its index
            for (int j = 0; j < nw; j++) {
                constexpr int kVec = Elt<DT>::kVec;
                const int i = __builtin_ctz(bits);
                bits &= bits - 1u;
                const uint32_t id = id0 + (uint32_t)((i / kVec) * kThreads * kVec + i % kVec);
                cbuf[pos + j] = make_raw(pick_elem(v, i), id);
            }
            st.cnt = st.cnt + total < kCandBuf ? st.cnt + total : kCandBuf;
            if (st.cnt >= kWave) {
                wt_flush(st, cbuf, k_eff, sm);
                fl = thr_floor(st.thr);
                uint32_t keep = 0u;
#pragma unroll
                for (int i = TS::kE - 1; i >= 0; i--) keep = (keep << 1) | (v[i] >= fl ? 1u : 0u);
                bits &= keep;
            }
        }
    });
    if (st.cnt > 0) wt_flush(st, cbuf, k_eff, sm);
    sm.lists[w][lane] = st.lst;
    __syncthreads();
    if (w == 0) {
        uint64_t acc = sm.lists[0][lane];
#pragma unroll
        for (int j = 1; j < kWaves; j++) acc = wave_merge_top(acc, sm.lists[j][lane]);
        out->keys[lane] = acc;
    }
}

template <int DT, bool kAligned>
__device__ __forceinline__ void seg_greedy(const void* row, int64_t start, int64_t end, RowpassSmem& sm,
                           PartSlot* out) {
    using TS = TileShape<DT>;
    uint64_t best = 0ull;  // 0 = nothing seen yet
    float best_v = -INFINITY;
    stream_range<DT, kAligned>(row, start, end, [&](float (&v)[TS::kE], int64_t t0, bool full) __attribute__((always_inline)) {
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        if (vmax > best_v || best == 0ull) {
            // earliest valid element holding the tile maximum (ids ascend with
            // i); on a tie with best_v the earlier tile's element already wins
            uint64_t cand = 0ull;
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const bool valid = full || elem_id<DT>(t0, i) < end;
                if (cand == 0ull && valid && v[i] == vmax)
                    cand = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
            }
            if (cand > best) {
                best = cand;
                best_v = vmax;
            }
        }
    });
    const uint64_t r = block_max_u64(best, sm.red);
    if (threadIdx.x == 0) out->keys[0] = r;
}

// Full-vocab rows: per tile, every wave leaves {max, sum of exp((l - max)/T)}
// of the part it read (exp2 terms in fp32, the wave sum in fp64 over the
// fixed DPP tree).  The records are indexed by tile, so how the tiles were split
// over workgroups never changes the result.
template <int DT, bool kAligned>
__device__ __forceinline__ void seg_full(const void* row, int64_t start, int64_t end, float T,
                                         FullStat* rec) {
    using TS = TileShape<DT>;
    const float c = exp2_coef(T);
    const int w = wave_id();
    stream_range<DT, kAligned>(row, start, end, [&](float (&v)[TS::kE], int64_t t0, bool)
                                                    __attribute__((always_inline)) {
        // out-of-range elements read as -inf and add nothing
        float lm = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) lm = fmaxf(lm, v[i]);
        const float m = wave_max_f32(lm);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (m > -INFINITY) {
#pragma unroll
            for (int i = 0; i < TS::kE; i++) acc[i & 3] += fast_exp2((v[i] - m) * c);
        }
        const double s = wave_sum((double)((acc[0] + acc[1]) + (acc[2] + acc[3])));
        if (lane_id() == 0) {
            FullStat r;
            r.m = m;
            r.pad = 0.f;
            r.s = s;
            rec[(t0 / TS::kTile) * kWaves + w] = r;
        }
    });
}

// Nucleus rows: the piece's mass histogram over the unit's anchor window,
// added in LDS one token at a time (fixed-point, so exact in any order).
// The anchor is the largest of the row's first 64 vectors (64 kVec elements,
// fewer when V is smaller): every wave of every piece reads the same ones and
// gets the same value; the loads go out with the first tile's and are reduced
// once that tile has arrived.  Written out: the buckets from the
// piece max's bucket down to 2048 below it (lower ones weigh under e^-32 of
// the piece max), from an even bucket lo on, at the start of the slot; their
// range [lo, hi] in keys[1] of the record and the piece max in keys[0] (float
// bits).  A piece max above the window marks the unit for the second
// histogram pass.
template <int DT, bool kAligned>
__device__ __forceinline__ void seg_nuc(const void* row, int64_t start, int64_t end, int64_t V,
                                        float T, uint64_t* s_h, RowpassSmem& sm, PartSlot* out,
                                        FnUnit* fu, uint64_t* hout) {
    using TS = TileShape<DT>;
    constexpr int kVec = Elt<DT>::kVec;
    const float cb = bucket_coef(T);
    u32x4* h4 = reinterpret_cast<u32x4*>(s_h);
    for (int i = threadIdx.x; i < kNW / 2; i += kThreads) h4[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // The anchor's vectors: one range-checked 16-byte load per lane (vector
    // `lane`), issued after the barrier above (whose fence would wait for
    // it) and used once the first tile has arrived.
    const int n_av = V < (int64_t)kWave * kVec ? (int)V : kWave * kVec;
    const int nvec_av = n_av / kVec;
    u32x4 q_av = u32x4{0u, 0u, 0u, 0u};
    if constexpr (kAligned)
        q_av = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(row, (uint32_t)nvec_av * 16u),
                                                     lane_id() * 16, 0, 2 /* nt */);
    float lmax = -INFINITY, la = 0.f;
    bool first = true;
    stream_range<DT, kAligned>(row, start, end, [&](float (&v)[TS::kE], int64_t, bool)
                                                    __attribute__((always_inline)) {
        if (first) {
            first = false;
            const int lane = lane_id();
            float av[kVec];
            if constexpr (kAligned) {
                const uint32_t d[4] = {q_av.x, q_av.y, q_av.z, q_av.w};
#pragma unroll
                for (int e = 0; e < kVec; e++) {
                    float x;
                    if constexpr (DT == SV_F32)
                        x = __uint_as_float(d[e]);
                    else
                        x = (e & 1) ? bf16_hi(d[e >> 1]) : bf16_lo(d[e >> 1]);
                    av[e] = lane * kVec + e < n_av ? x : -INFINITY;
                }
                if (nvec_av * kVec < n_av) {  // wave-uniform: a vector straddles a short row's end
#pragma unroll
                    for (int e = 0; e < kVec; e++)
                        if (lane == nvec_av && nvec_av * kVec + e < n_av)
                            av[e] = load_one<DT>(row, nvec_av * kVec + e);
                }
            } else {
#pragma unroll
                for (int e = 0; e < kVec; e++) {
                    const int i = lane * kVec + e;
                    av[e] = i < n_av ? load_one<DT>(row, i) : -INFINITY;
                }
            }
            float m = av[0];
#pragma unroll
            for (int e = 1; e < kVec; e++) m = fmaxf(m, av[e]);
            la = wave_max_f32(m);
        }
        // elements past `end` read as -inf: t = -inf, outside the window.
        // Tokens outside it add 0 to the spare slot s_h[kNW] (no branch per
        // element).
#pragma unroll
        for (int i = 0; i < TS::kE; i++) {
            lmax = fmaxf(lmax, v[i]);
            const float t = nuc_t(v[i], la, cb);
            int bin;
            const uint64_t w = nuc_wfix_t(t, &bin);
            const bool in = nuc_in(t);
            atomicAdd((unsigned long long*)&s_h[in ? bin : kNW], (unsigned long long)(in ? w : 0ull));
        }
        // The running max is formed here, before the next tile's loads reuse
        // this tile's registers: left to the scheduler it was sunk to the end
        // of the loop, the next loads went to other registers, and the loop
        // copied them back after waiting for every outstanding load.
        asm volatile("" : "+v"(lmax));
    });
    const float pm = block_max_f32(lmax, sm.red);  // barriers
    const float tm = nuc_t(pm, la, cb);
    const int hi = nuc_in(tm) ? nuc_bin(tm) : (tm >= (float)kHalf ? kNW - 1 : -1);
    const int lo = (hi - 2048 > 0 ? hi - 2048 : 0) & ~1;  // even: pairs of buckets per store
    u32x4* o4 = reinterpret_cast<u32x4*>(hout);
    for (int i = (lo >> 1) + (int)threadIdx.x; i <= (hi >> 1); i += kThreads)
        o4[i - (lo >> 1)] = h4[i];
    if (threadIdx.x == 0) {
        out->keys[0] = (uint64_t)__float_as_uint(pm);
        out->keys[1] = ((uint64_t)(uint32_t)lo << 32) | (uint64_t)(uint32_t)hi;
        fu->la = la;  // the same value from every piece
        // t is monotone in l: the piece max is the token that would lie
        // highest above the window
        if (tm >= (float)kHalf) fu->rehist = 1;
    }
}

// ---- units no longer than one wave's share of a tile ----------------------
// A row of at most kWave kE tokens fits in one wave's loads.  A workgroup then
// works its units four at a time, one per wave, and each wave's record is its
// unit's whole record: no workgroup barrier and no merge of the waves' lists
// per unit (worked one at a time by the whole workgroup, such a unit left
// three waves with a quarter of the loads each and paid the barriers and the
// merge of four lists for a few kilobytes).  Nucleus units keep the
// workgroup-wide histogram.

// Lane l's vector j is vector j kWave + l of the row, so the lane's elements
// ascend in id; tokens at or past V read as -inf.
template <int DT>
__device__ __forceinline__ uint32_t wave_elem_id(int idx) {
    constexpr int kVec = Elt<DT>::kVec;
    int lane = lane_id();
    asm volatile("" : "+v"(lane));  // recomputed where used, not kept live
    return (uint32_t)(((idx / kVec) * kWave + lane) * kVec + idx % kVec);
}

template <int DT, bool kAligned>
__device__ __forceinline__ void load_wave_unit(const void* row, int V,
                                               float (&v)[TileShape<DT>::kE]) {
    constexpr int kVec = Elt<DT>::kVec;
    const int lane = lane_id();
    if constexpr (kAligned) {
        // whole vectors through range-checked buffer loads, the vector that
        // straddles V token by token
        const int nvec = V / kVec;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)nvec * 16u);
        RawTile r;
#pragma unroll
        for (int j = 0; j < kLoads; j++)
            r.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * kWave + lane) * 16, 0, 2 /* nt */);
        unpack_tile<DT>(r, v);
#pragma unroll
        for (int j = 0; j < kLoads; j++) {
            const int vi = j * kWave + lane;
#pragma unroll
            for (int e = 0; e < kVec; e++)
                if (vi * kVec + e >= V) v[j * kVec + e] = -INFINITY;
            if (vi == nvec && nvec * kVec < V) {
#pragma unroll
                for (int e = 0; e < kVec; e++)
                    if (vi * kVec + e < V) v[j * kVec + e] = load_one<DT>(row, vi * kVec + e);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLoads; j++) {
#pragma unroll
            for (int e = 0; e < kVec; e++) {
                const int i = (j * kWave + lane) * kVec + e;
                const float x = load_one<DT>(row, i < V ? i : V - 1);
                v[j * kVec + e] = i < V ? x : -INFINITY;
            }
        }
    }
}

// Greedy unit: the best (logit, lowest id) key.
template <int DT, bool kAligned>
__device__ __forceinline__ void wave_greedy(const void* row, int V, PartSlot* out) {
    using TS = TileShape<DT>;
    float v[TS::kE];
    load_wave_unit<DT, kAligned>(row, V, v);
    float vmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < TS::kE; i++) {
        const uint32_t id = wave_elem_id<DT>(i);
        if (best == 0ull && (int)id < V && v[i] == vmax) best = make_key(v[i], id);
    }
    const uint64_t r = wave_max_u64(best);
    if (lane_id() == 0) out->keys[0] = r;
}

// Top-k unit: the wave's top-64 list (seg_topk's selection on one tile, with
// no thresholds shared between waves: each wave has a unit of its own).
template <int DT, bool kAligned>
__device__ __forceinline__ void wave_topk(const void* row, int V, int k_eff, RowpassSmem& sm,
                                          PartSlot* out) {
    using TS = TileShape<DT>;
    static_assert(TS::kE <= 32, "candidate mask is 32 bits");
    const int lane = lane_id();
    uint64_t* cbuf = sm.cbuf[wave_id()];
    float v[TS::kE];
    load_wave_unit<DT, kAligned>(row, V, v);
    WaveTopk st;
    st.lst = 0ull;
    st.thr = 0ull;
    st.cnt = 0;
    {  // the k-th largest of the lanes' best keys bounds the unit's k-th key
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) {
            const uint32_t id = wave_elem_id<DT>(i);
            if (best == 0ull && (int)id < V && v[i] == vmax) best = make_key(v[i], id);
        }
        const uint64_t th = lane_value(wave_sort_desc(best), k_eff - 1);
        if (th > 0ull) st.thr = th - 1ull;
    }
    float fl = thr_floor(st.thr);
    uint32_t bits = 0u;
#pragma unroll
    for (int i = TS::kE - 1; i >= 0; i--)
        bits = (bits << 1) | (((int)wave_elem_id<DT>(i) < V && v[i] >= fl) ? 1u : 0u);
    while (__ballot(bits != 0u) != 0ull) {
        int total;
        const uint32_t c = (uint32_t)__popc(bits);
        const int excl = wave_excl_count(c, &total);
        int room = kCandBuf - (st.cnt + excl);
        room = room < 0 ? 0 : room;
        const int nw = (int)c < room ? (int)c : room;
        const int pos = st.cnt + excl;
        for (int j = 0; j < nw; j++) {
            const int i = __builtin_ctz(bits);
            bits &= bits - 1u;
            cbuf[pos + j] = make_raw(pick_elem(v, i), wave_elem_id<DT>(i));
        }
        st.cnt = st.cnt + total < kCandBuf ? st.cnt + total : kCandBuf;
        if (st.cnt >= kWave) {
            wt_flush(st, cbuf, k_eff, sm);
            fl = thr_floor(st.thr);
            uint32_t keep = 0u;
#pragma unroll
            for (int i = TS::kE - 1; i >= 0; i--) keep = (keep << 1) | (v[i] >= fl ? 1u : 0u);
            bits &= keep;
        }
    }
    if (st.cnt > 0) wt_flush(st, cbuf, k_eff, sm);
    out->keys[lane] = st.lst;
}

// Untruncated unit: {max, sum of exp2((l - max) c)} in the record of wave 0 of
// its one tile; the other waves' records are empty.
template <int DT, bool kAligned>
__device__ __forceinline__ void wave_full(const void* row, int V, float T, FullStat* rec) {
    using TS = TileShape<DT>;
    const float c = exp2_coef(T);
    float v[TS::kE];
    load_wave_unit<DT, kAligned>(row, V, v);
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < TS::kE; i++) lm = fmaxf(lm, v[i]);
    const float m = wave_max_f32(lm);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (m > -INFINITY) {
#pragma unroll
        for (int i = 0; i < TS::kE; i++) acc[i & 3] += fast_exp2((v[i] - m) * c);
    }
    const double s = wave_sum((double)((acc[0] + acc[1]) + (acc[2] + acc[3])));
    const int lane = lane_id();
    if (lane < kWaves) {
        FullStat r;
        r.m = lane == 0 ? m : -INFINITY;
        r.pad = 0.f;
        r.s = lane == 0 ? s : 0.0;
        rec[lane] = r;
    }
}

// Units [l0, l1) of position k (each one tile): four at a time, one per wave,
// then the nucleus units one at a time with the whole workgroup.
template <int DT, bool kAligned>
__device__ __forceinline__ void rowpass_short(const StepArgs& a, int k, const PosDesc& P, int l0,
                                              int l1, RowpassSmem& sm, uint64_t* s_h) {
    const int w = blockIdx.x;
    const int V = (int)a.V;
    for (int base = l0; base < l1; base += kWaves) {
        const int li = base + wave_id();
        if (li >= l1) break;
        int region;
        const int u = unit_at(a, k, P, li, &region);
        const int cls = a.force_full ? (int)CLS_FULL : region;
        if (cls == CLS_NUCLEUS) continue;
        const int b = unit_b(a, u, k), side = u & 1;
        const void* row = unit_row<DT>(a, b, side, unit_rowidx(a, u, b, k));
        PartSlot* out = a.parts + li + w;
        if (cls == CLS_GREEDY)
            wave_greedy<DT, kAligned>(row, V, out);
        else if (cls == CLS_TOPK)
            wave_topk<DT, kAligned>(row, V, a.rows[b].k_eff, sm, out);
        else
            wave_full<DT, kAligned>(row, V, a.rows[b].T, a.tstat + (int64_t)u * kWaves);
    }
    if (a.force_full || P.n_cls[CLS_NUCLEUS] == 0) return;
    for (int li = l0; li < l1; li++) {
        int region;
        const int u = unit_at(a, k, P, li, &region);
        if (region != CLS_NUCLEUS) continue;
        const int b = unit_b(a, u, k), side = u & 1;
        const void* row = unit_row<DT>(a, b, side, unit_rowidx(a, u, b, k));
        __syncthreads();  // LDS is reused from the previous unit
        seg_nuc<DT, kAligned>(row, 0, a.V, a.V, a.rows[b].T, s_h, sm, a.parts + li + w,
                              a.fn_unit + u, a.hist + (int64_t)(li + w) * kHistSlot);
    }
}

// The workgroups split the tiles of position k's units evenly (see
// flat_begin); each (unit, workgroup) piece leaves its record at slot
// li + blockIdx.x.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void rowpass_kernel(StepArgs a, int k) {
    using TS = TileShape<DT>;
    __shared__ RowpassSmem sm;
    __shared__ uint64_t s_h[kNW + 1];  // nucleus pieces (and a spare slot)
    const PosDesc P = a.pos[k];
    const int n = pos_units(P);
    const int64_t T = (int64_t)n * a.ntiles;
    const int w = blockIdx.x;
    const int Gr = row_grid(P, T, (int)gridDim.x);  // the workgroups taking part
    int64_t t = flat_begin(T, Gr, w);
    const int64_t t_end = flat_begin(T, Gr, w + 1);
    if (a.V <= (int64_t)kWave * TS::kE) {  // one tile per unit: t counts units
        rowpass_short<DT, kAligned>(a, k, P, (int)t, (int)t_end, sm, s_h);
        return;
    }
    while (t < t_end) {
        const int li = (int)(t / a.ntiles);
        const int64_t tu0 = t - (int64_t)li * a.ntiles;
        int64_t tu1 = tu0 + (t_end - t);
        if (tu1 > a.ntiles) tu1 = a.ntiles;
        // the class comes with the list region, so the first tile's loads
        // need not wait for the row's info
        int region;
        const int u = unit_at(a, k, P, li, &region);
        const int b = unit_b(a, u, k), side = u & 1;
        const int cls = a.force_full ? (int)CLS_FULL : region;
        const void* row = unit_row<DT>(a, b, side, unit_rowidx(a, u, b, k));
        const int64_t start = tu0 * TS::kTile;
        int64_t end = tu1 * TS::kTile;
        if (end > a.V) end = a.V;
        PartSlot* out = a.parts + li + w;
        if (cls == CLS_GREEDY)
            seg_greedy<DT, kAligned>(row, start, end, sm, out);
        else if (cls == CLS_TOPK)
            seg_topk<DT, kAligned>(row, start, end, a.rows[b].k_eff, sm, out);
        else if (cls == CLS_NUCLEUS)
            seg_nuc<DT, kAligned>(row, start, end, a.V, a.rows[b].T, s_h, sm, out, a.fn_unit + u,
                                  a.hist + (int64_t)(li + w) * kHistSlot);
        else
            seg_full<DT, kAligned>(row, start, end, a.rows[b].T,
                                   a.tstat + (int64_t)u * a.ntiles * kWaves);
        t += tu1 - tu0;
        __syncthreads();  // LDS is reused by the next piece
    }
}

}  // namespace sv
