// sv_rowpass.h — the streaming pass over logits rows (the HBM-bound step).
//
// One workgroup reads one segment of one logits row exactly once, in 16-byte
// coalesced vectors, and leaves a small record:
//   * greedy rows:   the best (logit, lowest id) key of the segment;
//   * top-k rows:    the segment's top-k keys, descending (k <= 64);
//   * full-vocab:    {segment max m, sum of exp((l - m) / T)} (online).
// Selection uses raw logits (the ranking does not depend on T > 0), so the
// candidate sets are exact; probabilities are formed later in fp64.
//
// Coalesced single reads follow the read-coalescing technique described on
// "Apple Silikon İçin Cihaz Üstü Çıkarımı Optimize Etme", section "Dikkat
// önbelleği okumalarını birleştirin" (neighbouring lanes ask for neighbouring
// bytes); the selection rule itself is deniz.in "Üç düzeltmeden sonra…",
// section "Kesme her iki tarafta eşleşmek zorunda" (same top_k on both sides).
#pragma once

#include "sv_device.h"

namespace sv {

struct TopkSmem {
    uint64_t list[kMaxTopK];
    uint64_t buf[kMergeBuf];
    uint64_t red[kWaves];
    uint64_t thr;    // k-th key of the merged list (0 until it holds k keys)
    uint64_t floor;  // lower bound from the segment's first tile
    int ncand;
    int nlist;
};

// Merge the candidate buffer into the running list (all threads call).
__device__ inline void topk_merge(TopkSmem& sm, int k_eff) {
    const int nc = sm.ncand < kCandCap ? sm.ncand : kCandCap;
    const int nl = sm.nlist;
    const int total = nc + nl;
    const int P = pow2_ceil(total < 2 ? 2 : total);
    for (int i = threadIdx.x; i < P; i += kThreads) {
        if (i >= nc) sm.buf[i] = (i < total) ? sm.list[i - nc] : 0ull;
    }
    __syncthreads();
    block_sort_desc(sm.buf, P);
    const int newn = total < k_eff ? total : k_eff;
    for (int i = threadIdx.x; i < newn; i += kThreads) sm.list[i] = sm.buf[i];
    __syncthreads();
    if (threadIdx.x == 0) {
        sm.nlist = newn;
        sm.thr = (newn == k_eff) ? sm.list[k_eff - 1] : 0ull;
        sm.ncand = 0;
    }
    __syncthreads();
}

// Logit below which no key can exceed `thr` (the id decides on equality).
__device__ __forceinline__ float thr_floor(uint64_t thr) {
    return ((uint32_t)(thr >> 32) < 0x007FFFFFu) ? -INFINITY : key_logit(thr);
}

template <int DT, bool kAligned>
__device__ void rowpass_topk(const void* row, int64_t start, int64_t end, int k_eff,
                             PartSlot* out) {
    using TS = TileShape<DT>;
    __shared__ TopkSmem sm;
    if (threadIdx.x == 0) {
        sm.ncand = 0;
        sm.nlist = 0;
        sm.thr = 0ull;
        sm.floor = 0ull;
    }
    __syncthreads();
    float v[TS::kE];
    for (int64_t t0 = start; t0 < end; t0 += TS::kTile) {
        const bool full = (t0 + TS::kTile <= end);
        const bool last = (t0 + TS::kTile >= end);
        load_tile<DT, kAligned>(row, t0, end, full, v);
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        uint64_t own_thr;
        if (t0 == start) {
            // Lower bound for the segment's k-th key: in each wave, the k-th
            // largest of the lanes' best keys is reached by k distinct
            // elements, so the segment's k-th key is at least the largest of
            // these per-wave values.  Keys below it are never candidates.
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const int64_t id = elem_id<DT>(t0, i);
                if (id < end && v[i] == vmax && best == 0ull) best = make_key(v[i], (uint32_t)id);
            }
            const uint64_t sorted = wave_sort_desc(best);
            const uint64_t theta = __shfl(sorted, k_eff - 1, kWave);
            if (threadIdx.x % kWave == 0) sm.red[threadIdx.x / kWave] = theta;
            __syncthreads();
            uint64_t th = sm.red[0];
#pragma unroll
            for (int w = 1; w < kWaves; w++) th = sm.red[w] > th ? sm.red[w] : th;
            own_thr = th > 0ull ? th - 1ull : 0ull;
            __syncthreads();
            if (threadIdx.x == 0) sm.floor = own_thr;
        } else {
            own_thr = sm.thr > sm.floor ? sm.thr : sm.floor;
        }
        uint32_t pend = 0u;
        {
            const float tf = thr_floor(own_thr);
            if (vmax >= tf) {
#pragma unroll
                for (int i = 0; i < TS::kE; i++) {
                    const int64_t id = elem_id<DT>(t0, i);
                    if (id < end && v[i] >= tf && make_key(v[i], (uint32_t)id) > own_thr)
                        pend |= (1u << i);
                }
            }
        }
        for (;;) {
            const uint64_t thr = own_thr > sm.thr ? own_thr : sm.thr;
            uint32_t keep = 0u;
            if (pend) {
                // static indices keep v[] in registers
#pragma unroll
                for (int i = 0; i < TS::kE; i++) {
                    if (!(pend & (1u << i))) continue;
                    const uint64_t key = make_key(v[i], (uint32_t)elem_id<DT>(t0, i));
                    if (key <= thr) continue;
                    const int slot = atomicAdd(&sm.ncand, 1);
                    if (slot < kCandCap)
                        sm.buf[slot] = key;
                    else
                        keep |= (1u << i);
                }
            }
            pend = keep;
            __syncthreads();
            const int nc = sm.ncand;
            const bool over = nc > kCandCap;
            if (nc > 0 && (over || last || nc >= kCandCap / 2)) topk_merge(sm, k_eff);
            __syncthreads();
            if (!over) break;
        }
    }
    if (sm.ncand > 0) topk_merge(sm, k_eff);
    for (int i = threadIdx.x; i < kMaxTopK; i += kThreads)
        out->keys[i] = (i < sm.nlist) ? sm.list[i] : 0ull;
}

template <int DT, bool kAligned>
__device__ void rowpass_greedy(const void* row, int64_t start, int64_t end, PartSlot* out) {
    using TS = TileShape<DT>;
    __shared__ uint64_t red[kWaves];
    float v[TS::kE];
    uint64_t best = 0ull;  // 0 = nothing seen yet
    float best_v = -INFINITY;
    for (int64_t t0 = start; t0 < end; t0 += TS::kTile) {
        const bool full = (t0 + TS::kTile <= end);
        load_tile<DT, kAligned>(row, t0, end, full, v);
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        if (vmax > best_v || best == 0ull) {
            // earliest valid element holding the tile maximum (ids ascend with i);
            // on a tie with best_v the earlier tile's element already wins
            uint64_t cand = 0ull;
#pragma unroll
            for (int i = 0; i < TS::kE; i++) {
                const int64_t id = elem_id<DT>(t0, i);
                if (cand == 0ull && id < end && v[i] == vmax) cand = make_key(v[i], (uint32_t)id);
            }
            if (cand > best) {
                best = cand;
                best_v = vmax;
            }
        }
    }
    const uint64_t r = block_max_u64(best, red);
    if (threadIdx.x == 0) out->keys[0] = r;
}

// (m, s) pairs: s = sum of exp((l - m) / T).  Combining is exact up to one
// fp64 rounding per term; the fixed xor-tree keeps it deterministic.
__device__ __forceinline__ void ms_combine(float& m, double& s, float m2, double s2, double invT) {
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) {
        m = mm;
        s = 0.0;
        return;
    }
    const double a = (m == mm) ? s : s * exp(((double)m - (double)mm) * invT);
    const double b = (m2 == mm) ? s2 : s2 * exp(((double)m2 - (double)mm) * invT);
    m = mm;
    s = a + b;
}

template <int DT, bool kAligned>
__device__ void rowpass_full(const void* row, int64_t start, int64_t end, float T, PartSlot* out) {
    using TS = TileShape<DT>;
    __shared__ float red_m[kWaves];
    __shared__ double red_s[kWaves];
    const double invT = 1.0 / (double)T;
    float c = (float)(1.4426950408889634 / (double)T);
    c = fminf(c, 3.0e38f);
    float v[TS::kE];
    float m = -INFINITY;
    double s = 0.0;
    for (int64_t t0 = start; t0 < end; t0 += TS::kTile) {
        const bool full = (t0 + TS::kTile <= end);
        load_tile<DT, kAligned>(row, t0, end, full, v);
        float vmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < TS::kE; i++) vmax = fmaxf(vmax, v[i]);
        if (vmax > m) {
            s = (m == -INFINITY) ? 0.0 : s * exp(((double)m - (double)vmax) * invT);
            m = vmax;
        }
        if (m > -INFINITY) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < TS::kE; i++) acc[i & 3] += exp2f((v[i] - m) * c);
            s += (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const double s2 = __shfl_xor(s, o, kWave);
        ms_combine(m, s, m2, s2, invT);
    }
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    if (lane == 0) {
        red_m[w] = m;
        red_s[w] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = red_m[0];
        double ss = red_s[0];
        for (int i = 1; i < kWaves; i++) ms_combine(mm, ss, red_m[i], red_s[i], invT);
        FullStat* fs = reinterpret_cast<FullStat*>(out);
        fs->m = mm;
        fs->pad = 0.f;
        fs->s = ss;
    }
}

// grid.x = B * 2 * nseg; block -> (row b, side, segment).  side 0 = target
// row k, side 1 = draft row k.  Rows not live at position k exit at once.
template <int DT, bool kAligned>
__global__ __launch_bounds__(kThreads) void rowpass_kernel(
    const void* __restrict__ target, const void* __restrict__ draft, int64_t t_stride,
    int64_t d_stride, int K, int V, int k, int nseg, int tiles_per_seg,
    const RowInfo* __restrict__ rows, PartSlot* __restrict__ parts) {
    using TS = TileShape<DT>;
    const int bid = blockIdx.x;
    const int seg = bid % nseg;
    const int side = (bid / nseg) & 1;
    const int b = bid / (2 * nseg);
    const RowInfo& ri = rows[b];
    const int status = ri.status, L = ri.L, cls = ri.cls;
    if (status != ST_LIVE || k > L) return;
    if (side == 1 && (cls == CLS_GREEDY || k >= L)) return;
    const char* base;
    if (side == 0)
        base = static_cast<const char*>(target) +
               ((int64_t)b * (K + 1) + k) * t_stride * Elt<DT>::kSize;
    else
        base = static_cast<const char*>(draft) + ((int64_t)b * K + k) * d_stride * Elt<DT>::kSize;
    const int64_t start = (int64_t)seg * tiles_per_seg * TS::kTile;
    int64_t end = start + (int64_t)tiles_per_seg * TS::kTile;
    if (end > V) end = V;
    PartSlot* out = parts + ((int64_t)b * 2 + side) * nseg + seg;
    if (cls == CLS_GREEDY)
        rowpass_greedy<DT, kAligned>(base, start, end, out);
    else if (cls == CLS_TOPK)
        rowpass_topk<DT, kAligned>(base, start, end, ri.k_eff, out);
    else
        rowpass_full<DT, kAligned>(base, start, end, ri.T, out);
}

}  // namespace sv
