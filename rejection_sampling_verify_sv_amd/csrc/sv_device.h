// sv_device.h — device-side types and helpers shared by the verify kernels.
//
// Layout conventions (gfx950, wave64):
//   * one workgroup = 256 threads = 4 waves;
//   * a "tile" is what one workgroup reads in one step: every thread issues
//     kLoads 16-byte loads, consecutive lanes read consecutive 16-byte vectors
//     (fully coalesced), so a tile is 16 KiB of logits (4096 fp32 or 8192 bf16);
//     tiles are double-buffered, so two tiles per workgroup are in flight
//     (a workgroup streaming a whole row alone keeps more, see TileRing);
//   * a "unit" is one logits row to stream: (batch row b, side), side 0 = the
//     target row, side 1 = the draft row of the current position;
//   * units live at a position are listed on the device, and their tiles are
//     split evenly over a fixed grid of workgroups, so every position keeps the
//     256 compute units equally busy even after most rows have stopped.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTopK = SV_MAX_TOP_K;
constexpr int kLoads = 4;          // 16-byte loads per thread per tile
constexpr int kGrid = 1024;        // most workgroups of a streaming launch (record slots)
constexpr int kCandBuf = 128;      // per-wave candidate buffer (top-k select)

enum RowClass : int32_t {
    CLS_GREEDY = 0,
    CLS_TOPK = 1,
    CLS_FULL = 2,     // no top_k, no top_p cut: softmax over all V
    CLS_NUCLEUS = 3,  // no top_k, top_p < 1 over all V
    CLS_ERROR = -1,
    CLS_UNSUP = -2,
};

enum RowStatus : int32_t { ST_LIVE = 0, ST_DONE = 1, ST_SAMPLE = 2, ST_ERROR = 3 };
enum Need : int32_t { NEED_NONE = 0, NEED_RESID = 1, NEED_BONUS = 2 };

// Per-row bookkeeping kept in the workspace (112 bytes).  A verify step walks
// positions 0..L of a chain of drafts; a tree verify walks from node 0 to an
// accepted child at every level (then `node` names the node whose rows the
// current level reads, and `acc` the level).
struct RowInfo {
    int32_t cls, L, status, acc;
    int32_t kpos, need, k_eff, node;  // kpos: row index of the final draw (position or node)
    float T, top_p;
    int32_t li_t, li_d;      // index of the target / draft unit in its class region at the current position
    double mt, zt, md, zd;   // full-vocab stats (max, normaliser) at position kpos
    uint64_t tau_t, tau_d;   // nucleus rows: key of the last kept token
    int32_t rounds;          // tree, full-vocab rows: children rejected at the current node
    int32_t nxt;             // tree, full-vocab rows: the next child to test (-1: none)
    int32_t kids;            // tree: the current node has children (its draft row is listed)
    int32_t pad;
};
static_assert(sizeof(RowInfo) == 112, "RowInfo layout");

// Children per node a tree verify serves on full-vocab rows (each rejected
// child there costs a pass over the node's two rows); top-k and greedy rows
// take any number.
constexpr int kMaxKids = 64;

// Work counters of one position.  The units to stream are listed in one
// region per row class (greedy, top-k, untruncated, nucleus), laid end to end
// in that order, so that neighbouring workgroups of the row pass mostly run
// the same code (mixed classes on one compute unit measurably slow it).
constexpr int kNumCls = 4;
static_assert(CLS_GREEDY == 0 && CLS_TOPK == 1 && CLS_FULL == 2 && CLS_NUCLEUS == 3,
              "row classes index the unit regions");
struct PosDesc {
    int32_t n_cls[kNumCls];  // units listed per class region
    int32_t n_sample;        // rows whose final draw streams their rows (final slot only)
    int32_t n_pick;          // rows whose final draw takes its masses from the row pass's
                             // records (untruncated bonus draws; final slot only)
    int32_t pad[2];
};
__host__ __device__ __forceinline__ int pos_units(const PosDesc& p) {
    return p.n_cls[0] + p.n_cls[1] + p.n_cls[2] + p.n_cls[3];
}
// Index in the concatenated list of entry j of class c's region.
__device__ __forceinline__ int unit_index(const PosDesc& p, int c, int j) {
    int s = 0;
    for (int i = 0; i < c; i++) s += p.n_cls[i];
    return s + j;
}

// One segment's result: a descending top-k key list (zero-padded), or the
// best key of a greedy segment in keys[0].
struct PartSlot {
    uint64_t keys[kMaxTopK];
};

// Full-vocab rows: {max, sum of exp((l - max) / T)} of the part of one tile
// that one wave reads.  Records are laid out per (row, side, tile, wave), so
// the order in which they are combined never depends on how the tiles were
// split over workgroups.
struct FullStat {
    float m;
    float pad;
    double s;
};

// 2^x by the hardware exp2 (about 1 ulp; results below 2^-126 may flush to
// zero, far below anything these sums can resolve).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp(x / T) = exp2(x * c) with c = log2(e) / T (clamped so that c is finite).
__host__ __device__ __forceinline__ float exp2_coef(float T) {
    const float c = (float)(1.4426950408889634 / (double)T);
    return c < 3.0e38f ? c : 3.0e38f;
}

// ---- masses for the full-vocab nucleus cut ---------------------------------
// A nucleus unit is measured against an anchor logit la: the largest of the
// row's first 64 vectors (every piece of the row pass reads them and gets the
// same value), or the row max on a second pass (below).  Token l sits at
// t = (l - la) 64 / T, its weight relative to the anchor is exp(t / 64), and
// it falls into bucket floor(t) + kHalf of a window of kNW buckets (slices of
// 1/64 in (l - la) / T; a higher logit never lands in a lower bucket).
// Within bucket b a weight is scale_b w_rel with
// scale_b = exp((b - kHalf + 1) / 64) and w_rel = exp((frac(t) - 1) / 64) in
// (0.984, 1], the latter in 31-bit fixed point, so a bucket's mass is scale_b
// times an exact integer whatever the order of the additions.
//   * t < -kHalf: at least 32 T below the anchor, hence below the row max;
//     the weight is under e^-32 of the max's and the token is dropped;
//   * t >= kHalf: the row max lies far above the anchor; the unit is then
//     histogrammed again, anchored at its row max (where t <= 0).
constexpr int kNW = 4096;
constexpr int kHalf = kNW / 2;
constexpr float kBucketScale = 64.0f;
constexpr float kLog2e64 = 0.022542110013490055f;  // log2(e) / 64
constexpr int kCollectCap = 4096;   // boundary-bucket tokens resolved in LDS per unit
// A row-pass piece writes out the buckets from its max's bucket down to 2048
// below it (the lower ones weigh under e^-32 of the piece max), starting at an
// even bucket: at most 2050 of them, stored from the slot's start.
constexpr int kHistSlot = 2056;
constexpr double kUnfix = 1.0 / 2147483648.0;    // 2^-31, the weights' fixed-point unit

// Bucket scale 64 / T, clamped finite like exp2_coef.
__host__ __device__ __forceinline__ float bucket_coef(float T) {
    const float c = kBucketScale / T;
    return c < 3.0e38f ? c : 3.0e38f;
}

// Window coordinate of logit l (NaN when l or la is NaN, or both are -inf).
__device__ __forceinline__ float nuc_t(float l, float la, float cb) { return (l - la) * cb; }
// t lies in the window (false for NaN).
__device__ __forceinline__ bool nuc_in(float t) {
    return t >= -(float)kHalf && t < (float)kHalf;
}
// Bucket of an in-window coordinate.
__device__ __forceinline__ int nuc_bin(float t) { return (int)floorf(t) + kHalf; }

// floor(w_rel 2^31) for w_rel = exp2((fr - 1) log2(e) / 64), fr = frac(t) in
// [0, 1): below 2^31, so one 32-bit conversion gives it exactly; sums of up
// to 2^33 of them fit 64 bits.
__device__ __forceinline__ uint64_t nuc_wrel(float fr) {
    const float w = fast_exp2(fmaf(fr, kLog2e64, -kLog2e64));
    return (uint64_t)(uint32_t)(w * 2147483648.0f);
}
// Fixed-point weight of an in-window coordinate t, and its bucket.
__device__ __forceinline__ uint64_t nuc_wfix_t(float t, int* bin) {
    const float f = floorf(t);
    *bin = (int)f + kHalf;
    return nuc_wrel(t - f);
}
// Bucket of any non-NaN logit: -1 below the window, kNW above it.  Never
// decreases as l grows.
__device__ __forceinline__ int nuc_gbin(float l, float la, float cb) {
    const float t = nuc_t(l, la, cb);
    return nuc_in(t) ? nuc_bin(t) : (t < 0.f ? -1 : kNW);
}
// The float with ranking image o (the inverse of ord32 on non-NaN values).
__device__ __forceinline__ float ord_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// scale_b = exp((b - kHalf + 1) / 64), the weight of bucket b's upper edge
// relative to the anchor, as a table built at compile time: e^(1/64) from its
// Taylor series (20 terms, far past double precision), then repeated
// products outward from scale_{kHalf-1} = 1 (at most 2048 roundings: the
// relative error stays below 1e-12).
struct NucScaleTable {
    double v[kNW];
    constexpr NucScaleTable() : v() {
        double e = 1.0, term = 1.0;
        for (int i = 1; i < 20; i++) {
            term = term / (64.0 * i);
            e += term;
        }
        const double ie = 1.0 / e;
        v[kHalf - 1] = 1.0;
        for (int b = kHalf; b < kNW; b++) v[b] = v[b - 1] * e;
        for (int b = kHalf - 2; b >= 0; b--) v[b] = v[b + 1] * ie;
    }
};
__device__ constexpr NucScaleTable kNucScale{};
__device__ __forceinline__ double nuc_scale(int b) { return kNucScale.v[b]; }

// Per (row, side) state of the nucleus cut at the current position; masses
// are relative to the anchor (a token weighs exp(t / 64)).
struct FnUnit {
    double S;         // kept mass
    uint64_t tau;     // key of the last kept token
    float la;         // anchor logit
    int32_t status;   // 0 ok, 1 no boundary found (not reached), 2 no finite logit
    int32_t rehist;   // set by the row pass: a token lies above the window
};

// Cross-workgroup hand-offs inside one launch.  The data another workgroup
// will read is stored at device scope, which writes it through to the point
// where the caches of all compute units agree; the writer then waits for its
// stores to complete (dev_stores_done) before it signals with a device-scope
// atomic, and the reader, having seen the signal, loads at device scope.  The
// stores being written through, no cache-wide write-back (what a release
// fence would add) is needed.
template <class T>
__device__ __forceinline__ void dev_store(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T dev_load(T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory operation this wave issued has completed.
__device__ __forceinline__ void dev_stores_done() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void fn_put_status(FnUnit* f, int32_t st) { dev_store(&f->status, st); }
__device__ __forceinline__ void fn_put_la(FnUnit* f, float la) {
    dev_store(reinterpret_cast<int32_t*>(&f->la), __float_as_int(la));
}
__device__ __forceinline__ void fn_put_cut(FnUnit* f, uint64_t tau, double S) {
    dev_store(&f->tau, tau);
    dev_store(reinterpret_cast<uint64_t*>(&f->S), (uint64_t)__double_as_longlong(S));
}

// ---- element types and tiles ----------------------------------------------
template <int DT>
struct Elt;
template <>
struct Elt<SV_F32> {
    static constexpr int kVec = 4;
    static constexpr int kSize = 4;
};
template <>
struct Elt<SV_BF16> {
    static constexpr int kVec = 8;
    static constexpr int kSize = 2;
};

template <int DT>
struct TileShape {
    static constexpr int kVec = Elt<DT>::kVec;
    static constexpr int kE = kLoads * kVec;      // elements per thread
    static constexpr int kTile = kThreads * kE;   // elements per tile
};

// ---- ranking key ---------------------------------------------------------
// key = (order-preserving image of the logit) << 32 | (0xFFFFFFFF - id):
// a larger key is a higher logit, and among equal logits the lower id.
// -0.0 is folded onto +0.0 so the two compare equal, as they do in fp64.
// Key 0 is below every real token (the image of -inf is 0x007FFFFF).
__device__ __forceinline__ uint32_t ord32(float f) {
    uint32_t b = __float_as_uint(f);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float f, uint32_t id) {
    return ((uint64_t)ord32(f) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ float key_logit(uint64_t k) {
    uint32_t o = (uint32_t)(k >> 32);
    uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(b);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

// Logit below which no key can exceed `thr` (the id decides on equality).
__device__ __forceinline__ float thr_floor(uint64_t thr) {
    return ((uint32_t)(thr >> 32) < 0x007FFFFFu) ? -INFINITY : key_logit(thr);
}

// ---- loads ---------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RawTile {
    u32x4 q[kLoads];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t i) {
    if constexpr (DT == SV_F32) {
        return static_cast<const float*>(row)[i];
    } else {
        uint32_t h = static_cast<const uint16_t*>(row)[i];
        return __uint_as_float(h << 16);
    }
}

// Issue the 16-byte loads of one full tile (row 16-byte aligned).
template <int DT>
__device__ __forceinline__ void issue_tile(const void* row, int64_t t0, RawTile& r) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(row) +
                                                    t0 * Elt<DT>::kSize);
#pragma unroll
    for (int j = 0; j < kLoads; j++)
        r.q[j] = __builtin_nontemporal_load(p + j * kThreads + (int)threadIdx.x);
}

template <int DT>
__device__ __forceinline__ void unpack_tile(const RawTile& r, float (&v)[TileShape<DT>::kE]) {
#pragma unroll
    for (int j = 0; j < kLoads; j++) {
        if constexpr (DT == SV_F32) {
            v[j * 4 + 0] = __uint_as_float(r.q[j].x);
            v[j * 4 + 1] = __uint_as_float(r.q[j].y);
            v[j * 4 + 2] = __uint_as_float(r.q[j].z);
            v[j * 4 + 3] = __uint_as_float(r.q[j].w);
        } else {
            v[j * 8 + 0] = bf16_lo(r.q[j].x);
            v[j * 8 + 1] = bf16_hi(r.q[j].x);
            v[j * 8 + 2] = bf16_lo(r.q[j].y);
            v[j * 8 + 3] = bf16_hi(r.q[j].y);
            v[j * 8 + 4] = bf16_lo(r.q[j].z);
            v[j * 8 + 5] = bf16_hi(r.q[j].z);
            v[j * 8 + 6] = bf16_lo(r.q[j].w);
            v[j * 8 + 7] = bf16_hi(r.q[j].w);
        }
    }
}

// threadIdx.x behind an empty asm: values derived from it are recomputed
// where used instead of being hoisted into registers that stay live across
// the whole streaming loop.
__device__ __forceinline__ int tid_opaque() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Element-wise load of a tile; elements at or past `end` read as -inf.  The
// index is clamped instead of branched on, so every load is issued before the
// first wait.  Requires start < end.
template <int DT>
__device__ __forceinline__ void load_tile_partial(const void* row, int64_t start, int64_t end,
                                                  float (&v)[TileShape<DT>::kE]) {
    constexpr int kVec = Elt<DT>::kVec;
#pragma unroll
    for (int j = 0; j < kLoads; j++) {
#pragma unroll
        for (int e = 0; e < kVec; e++) {
            const int64_t i = start + (int64_t)(j * kThreads + (int)threadIdx.x) * kVec + e;
            const float x = load_one<DT>(row, i < end ? i : end - 1);
            v[j * kVec + e] = i < end ? x : -INFINITY;
        }
    }
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): loads past
// the end return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Last, partial tile of a 16-byte aligned row: whole vectors below `end` come
// in with 16-byte buffer loads (range-checked, so nothing past the last whole
// vector is read), the few elements of a vector that straddles `end` one by
// one; elements at or past `end` read as -inf.  Requires start < end <=
// start + tile.
template <int DT>
__device__ __forceinline__ void load_tile_tail(const void* row, int64_t start, int64_t end,
                                               float (&v)[TileShape<DT>::kE]) {
    constexpr int kVec = Elt<DT>::kVec;
    const int n = (int)(end - start);
    const int nvec = n / kVec;
    const char* base = static_cast<const char*>(row) + start * Elt<DT>::kSize;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)nvec * 16u);
    RawTile r;
    const int tid = tid_opaque();
#pragma unroll
    for (int j = 0; j < kLoads; j++)
        r.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * kThreads + tid) * 16, 0, 2 /* nt */);
    unpack_tile<DT>(r, v);
#pragma unroll
    for (int j = 0; j < kLoads; j++) {
        const int vi = j * kThreads + tid;
#pragma unroll
        for (int e = 0; e < kVec; e++)
            if (vi * kVec + e >= n) v[j * kVec + e] = -INFINITY;
        if (vi == nvec && nvec * kVec < n) {  // the straddling vector
#pragma unroll
            for (int e = 0; e < kVec; e++)
                if (vi * kVec + e < n) v[j * kVec + e] = load_one<DT>(row, start + vi * kVec + e);
        }
    }
}

// Id of element v[idx] of the tile starting at t0: the thread's elements are
// in ascending id order.
template <int DT>
__device__ __forceinline__ int64_t elem_id(int64_t start, int idx) {
    constexpr int kVec = Elt<DT>::kVec;
    const int j = idx / kVec, e = idx % kVec;
    return start + (int64_t)(j * kThreads + tid_opaque()) * kVec + e;
}

// Stream the elements [start, end) of a row (start tile-aligned) through
// body(v, t0, full).  Full tiles are double-buffered: the loads of tile t+1
// are in flight while tile t is processed, and the compiler's wait before a
// tile is used only drains the older of the two buffers.  The ragged tail of
// an aligned row comes in through range-checked buffer loads; every tile of a
// row that is not 16-byte aligned is loaded element by element.  `body` must not contain workgroup barriers (they would
// drain the loads).
template <int DT, bool kAligned, class Body>
__device__ __forceinline__ void stream_range(const void* row, int64_t start, int64_t end,
                                             Body&& body) {
    using TS = TileShape<DT>;
    float v[TS::kE];
    int64_t t0 = start;
    if constexpr (kAligned) {
        const int64_t full_end = start + ((end - start) / TS::kTile) * TS::kTile;
        if (t0 < full_end) {
            // Counted pairs with a single exit keep the loop free of dead
            // back edges, which would otherwise force a full drain of the
            // outstanding loads at the loop head.  After an even count the
            // last prefetch re-reads the final tile and is dropped.
            const int64_t nt = (full_end - t0) / TS::kTile;
            const int64_t last = full_end - TS::kTile;
            RawTile A, B;
            issue_tile<DT>(row, t0, A);
            for (int64_t p = nt >> 1; p > 0; --p) {
                issue_tile<DT>(row, t0 + TS::kTile, B);
                __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the wait
                unpack_tile<DT>(A, v);
                body(v, t0, true);
                const int64_t tn = t0 + 2 * TS::kTile;
                issue_tile<DT>(row, tn <= last ? tn : last, A);
                __builtin_amdgcn_sched_barrier(0);
                unpack_tile<DT>(B, v);
                body(v, t0 + TS::kTile, true);
                t0 += 2 * TS::kTile;
            }
            if (nt & 1) {
                unpack_tile<DT>(A, v);
                body(v, t0, true);
                t0 += TS::kTile;
            }
        }
    }
    while (t0 < end) {
        if constexpr (kAligned)
            load_tile_tail<DT>(row, t0, end, v);
        else
            load_tile_partial<DT>(row, t0, end, v);
        body(v, t0, t0 + TS::kTile <= end);
        t0 += TS::kTile;
    }
}

// Elements [start, end) of a row (start tile-aligned) streamed by one
// workgroup, kDepth full tiles in flight.  A workgroup working alone is bound
// by the latency of its loads, not by HBM, so it keeps more of them
// outstanding than the double buffer of stream_range.  start() issues the
// first tiles and may run well before run(): the loads then overlap whatever
// the workgroup does in between.  run() covers the same ground as
// stream_range (full tiles, then the ragged tail); `body` must not contain
// barriers.
template <int DT, bool kAligned, int kDepth>
struct TileRing {
    using TS = TileShape<DT>;
    RawTile r[kDepth];
    int64_t nt;  // full tiles streamed through the ring

    __device__ __forceinline__ void start(const void* row, int64_t start, int64_t end) {
        nt = kAligned ? (end - start) / TS::kTile : 0;
        if (nt > 0) {
#pragma unroll
            for (int j = 0; j < kDepth; j++)
                issue_tile<DT>(row, start + (j < nt ? j : nt - 1) * TS::kTile, r[j]);
        } else {
            // defined on every path: buffers left undefined here were seen
            // to be kept live (as copies of an earlier use) across a
            // caller's surrounding loop
#pragma unroll
            for (int j = 0; j < kDepth; j++)
#pragma unroll
                for (int q = 0; q < kLoads; q++) r[j].q[q] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Counted rounds with one exit, as in stream_range; prefetches past the
    // last full tile re-read it and are dropped.
    template <class Body>
    __device__ __forceinline__ void run(const void* row, int64_t start, int64_t end, Body&& body) {
        float v[TS::kE];
        int64_t t0 = start;
        if (nt > 0) {
            const int64_t last = start + (nt - 1) * TS::kTile;
            for (int64_t p = nt / kDepth; p > 0; --p) {
#pragma unroll
                for (int j = 0; j < kDepth; j++) {
                    unpack_tile<DT>(r[j], v);
                    body(v, t0 + j * TS::kTile, true);
                    const int64_t tn = t0 + (kDepth + j) * TS::kTile;
                    issue_tile<DT>(row, tn <= last ? tn : last, r[j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                t0 += kDepth * TS::kTile;
            }
            const int rem = (int)(nt % kDepth);
#pragma unroll
            for (int j = 0; j < kDepth - 1; j++) {
                if (j < rem) {
                    unpack_tile<DT>(r[j], v);
                    body(v, t0, true);
                    t0 += TS::kTile;
                }
            }
        }
        while (t0 < end) {
            if constexpr (kAligned)
                load_tile_tail<DT>(row, t0, end, v);
            else
                load_tile_partial<DT>(row, t0, end, v);
            body(v, t0, t0 + TS::kTile <= end);
            t0 += TS::kTile;
        }
    }
};

// Same as stream_range over two rows in lockstep (the second may be null):
// body(va, vb, t0, full); vb is all -inf when rb is null.
template <int DT, bool kAligned, class Body>
__device__ __forceinline__ void stream_range2(const void* ra, const void* rb, int64_t start,
                                              int64_t end, Body&& body) {
    using TS = TileShape<DT>;
    float va[TS::kE], vb[TS::kE];
#pragma unroll
    for (int i = 0; i < TS::kE; i++) vb[i] = -INFINITY;
    int64_t t0 = start;
    const void* rb2 = rb ? rb : ra;  // loads stay unconditional; vb is ignored then
    if constexpr (kAligned) {
        const int64_t full_end = start + ((end - start) / TS::kTile) * TS::kTile;
        if (t0 < full_end) {
            const int64_t nt = (full_end - t0) / TS::kTile;
            const int64_t last = full_end - TS::kTile;
            RawTile A, A2, B, B2;
            issue_tile<DT>(ra, t0, A);
            issue_tile<DT>(rb2, t0, A2);
            for (int64_t p = nt >> 1; p > 0; --p) {
                issue_tile<DT>(ra, t0 + TS::kTile, B);
                issue_tile<DT>(rb2, t0 + TS::kTile, B2);
                __builtin_amdgcn_sched_barrier(0);
                unpack_tile<DT>(A, va);
                if (rb) unpack_tile<DT>(A2, vb);
                body(va, vb, t0, true);
                const int64_t tn = t0 + 2 * TS::kTile;
                issue_tile<DT>(ra, tn <= last ? tn : last, A);
                issue_tile<DT>(rb2, tn <= last ? tn : last, A2);
                __builtin_amdgcn_sched_barrier(0);
                unpack_tile<DT>(B, va);
                if (rb) unpack_tile<DT>(B2, vb);
                body(va, vb, t0 + TS::kTile, true);
                t0 += 2 * TS::kTile;
            }
            if (nt & 1) {
                unpack_tile<DT>(A, va);
                if (rb) unpack_tile<DT>(A2, vb);
                body(va, vb, t0, true);
                t0 += TS::kTile;
            }
        }
    }
    while (t0 < end) {
        if constexpr (kAligned) {
            load_tile_tail<DT>(ra, t0, end, va);
            if (rb) load_tile_tail<DT>(rb, t0, end, vb);
        } else {
            load_tile_partial<DT>(ra, t0, end, va);
            if (rb) load_tile_partial<DT>(rb, t0, end, vb);
        }
        body(va, vb, t0, t0 + TS::kTile <= end);
        t0 += TS::kTile;
    }
}

// ---- even split of a list's tiles over the workgroups ----------------------
// The n units of a list are laid end to end, ntiles tiles each, and
// workgroup w of G streams tiles [w*T/G, (w+1)*T/G) of that concatenation
// (T = n*ntiles), so every workgroup reads the same amount.  A workgroup can
// cover the end of one unit and the start of the next; it leaves one record
// per (unit u, workgroup w) piece, at slot u + w (unique because both grow
// along the concatenation), so n + G slots suffice.
// Only min(G, T) workgroups take part, so every taking part owns a tile.
__host__ __device__ __forceinline__ int flat_active(int64_t T, int G) {
    return (int)(T < (int64_t)G ? T : (int64_t)G);
}
__host__ __device__ __forceinline__ int64_t flat_begin(int64_t T, int G, int w) {
    const int Ga = flat_active(T, G);
    return w < Ga ? ((int64_t)w * T) / Ga : T;
}
// Workgroup that streams tile t (0 <= t < T).
__host__ __device__ __forceinline__ int flat_owner(int64_t t, int64_t T, int G) {
    const int Ga = flat_active(T, G);
    return (int)(((t + 1) * (int64_t)Ga - 1) / T);
}

// The row pass gives every workgroup taking part at least kRowMinTiles tiles
// (when the position has that many) unless all its units are untruncated:
// with few units, a unit split over one workgroup per tile leaves dozens of
// records that the decision merges one after another (a top-k list, a best
// key or a histogram per piece), and every piece pays its own start (the
// first tiles of a top-k piece are the costly ones).  Untruncated units keep
// per-tile records whatever the split, so they keep one tile per workgroup.
// With at most one unit per workgroup and pieces of at least 2 kRowMinTiles
// tiles, the workgroups taking part are a multiple of the unit count when
// that keeps at least 5/8 of them: every unit then gets the same number of
// workgroups, each streaming a part of one unit only (the even split's
// boundaries fall on unit boundaries), so no workgroup pays for the start and
// end of a second piece.  Measured on the 1024-row mix: 330 units on 990
// workgroups took 46 us against 50.5, 715 units on 715 workgroups (one unit
// each) 82 against 87 on all 1024; at 4-tile pieces, as in small batches,
// there was no gain.
constexpr int kRowMinTiles = 4;
__host__ __device__ __forceinline__ int row_grid(const PosDesc& P, int64_t T, int G) {
    const int n = pos_units(P);
    if (P.n_cls[CLS_FULL] == n) return flat_active(T, G);
    const int64_t g = (T + kRowMinTiles - 1) / kRowMinTiles;
    const int Gm = (int)(g < (int64_t)G ? (g > 0 ? g : 1) : (int64_t)G);
    if (n > 0 && n <= G && T >= (int64_t)Gm * 2 * kRowMinTiles) {
        const int64_t cap = (T / n) / kRowMinTiles;  // pieces of at least kRowMinTiles tiles
        const int64_t per = (int64_t)(G / n) < cap ? (int64_t)(G / n) : cap;
        // short units that alone give every compute unit a workgroup (a
        // quarter of the resident grid) are not split at all: their pieces'
        // fixed costs (first tiles, flush, record) outweigh the streaming
        // (64-row greedy mix, 448 units of 19 tiles: 67.2 -> 65.0 us per
        // step; units of 38 tiles kept their split, which measured better)
        if (per > 1 && (int64_t)n * 4 >= (int64_t)G && T < (int64_t)n * 8 * kRowMinTiles) return n;
        if (per >= 1 && (int64_t)n * per * 8 >= (int64_t)Gm * 5) return (int)(n * per);
    }
    return Gm;
}

// Record slots [first, first + count) of unit li (index in position P's
// list), from the row pass of G workgroups.
struct RecRange {
    int first, count;
};
__host__ __device__ __forceinline__ RecRange unit_records(const PosDesc& P, int li, int ntiles,
                                                           int G) {
    const int64_t T = (int64_t)pos_units(P) * ntiles;
    const int Gr = row_grid(P, T, G);
    const int w0 = flat_owner((int64_t)li * ntiles, T, Gr);
    const int w1 = flat_owner((int64_t)(li + 1) * ntiles - 1, T, Gr);
    RecRange r;
    r.first = li + w0;
    r.count = w1 - w0 + 1;
    return r;
}

// ---- wave / block helpers -------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x / kWave); }

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// Exclusive prefix over the wave of a per-lane count c < 64 (bit planes
// through ballots, no LDS); *total gets the wave sum.
__device__ __forceinline__ int wave_excl_count(uint32_t c, int* total) {
    int excl = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 6; bit++) {
        const uint64_t m = __ballot((c >> bit) & 1u);
        const uint32_t below =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        excl += (int)below << bit;
        tot += __popcll(m) << bit;
    }
    *total = tot;
    return excl;
}

// Relaxed atomic LDS accesses for values other waves update concurrently:
// always re-read (never cached in registers), and kept in the LDS address
// space so they wait on the LDS counter only, not on outstanding HBM loads.
typedef __attribute__((address_space(3))) uint64_t lds_u64;
__device__ __forceinline__ uint64_t lds_load_relaxed(const uint64_t* p) {
    return __atomic_load_n((const lds_u64*)p, __ATOMIC_RELAXED);
}
__device__ __forceinline__ void lds_store_relaxed(uint64_t* p, uint64_t v) {
    __atomic_store_n((lds_u64*)p, v, __ATOMIC_RELAXED);
}

// Order this wave's LDS accesses (writes by some lanes, reads by others).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- lane exchanges without LDS ------------------------------------------
// xor_lane<S>(v) is v of lane (lane ^ S), S a power of two below 64.  Inside
// a row of 16 lanes DPP does it: S = 1, 2 are quad permutations, S = 8 is a
// rotation by 8, and S = 4 takes two rotations (by 4 and by 12), each written
// only to the quads (DPP banks) whose partner it reaches.  Across rows the
// gfx950 permlane swaps exchange the odd rows (S = 16) or the upper half
// (S = 32) of one register with the even rows / lower half of another; given
// v twice, every lane ends holding the values of both lanes of its pair, the
// lower lane's in the first result and the higher lane's in the second.
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "stride");
    const int iv = (int)v;
    if constexpr (S == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0xb1, 0xf, 0xf, false);  // [1,0,3,2]
    } else if constexpr (S == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0x4e, 0xf, 0xf, false);  // [2,3,0,1]
    } else if constexpr (S == 4) {
        // row_ror:4 reads lane i - 4 (quads 1, 3), row_ror:12 lane i + 4 (quads 0, 2)
        const int t = __builtin_amdgcn_update_dpp(iv, iv, 0x124, 0xf, 0xa, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(t, iv, 0x12c, 0xf, 0x5, false);
    } else if constexpr (S == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(iv, iv, 0x128, 0xf, 0xf, false);  // row_ror:8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? (uint32_t)r[0] : (uint32_t)r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? (uint32_t)r[0] : (uint32_t)r[1];
    }
}
template <int S>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v) {
    const uint32_t lo = xor_lane<S>((uint32_t)v), hi = xor_lane<S>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
// Wave-wide max / min of an int; every lane gets the result.
__device__ __forceinline__ int wave_max_i32(int v) {
    int w;
    w = (int)xor_lane<1>((uint32_t)v);  v = w > v ? w : v;
    w = (int)xor_lane<2>((uint32_t)v);  v = w > v ? w : v;
    w = (int)xor_lane<4>((uint32_t)v);  v = w > v ? w : v;
    w = (int)xor_lane<8>((uint32_t)v);  v = w > v ? w : v;
    w = (int)xor_lane<16>((uint32_t)v); v = w > v ? w : v;
    w = (int)xor_lane<32>((uint32_t)v); v = w > v ? w : v;
    return v;
}
__device__ __forceinline__ int wave_min_i32(int v) { return -wave_max_i32(-v); }
// v of lane 63 - lane: mirror inside rows (row_mirror), then swap rows and halves.
__device__ __forceinline__ uint64_t wave_reverse(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(v >> 32), (int)(v >> 32), 0x140, 0xf, 0xf,
                                               false);
    const uint64_t m = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    return xor_lane<32>(xor_lane<16>(m));
}
// v of lane i for a wave-uniform i (scalar reads, no LDS).
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int i) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)v, i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), i);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double lane_value(double v, int i) {
    return __longlong_as_double((long long)lane_value((uint64_t)__double_as_longlong(v), i));
}

// 64-bit DPP move (two 32-bit moves); lanes whose source lies outside the
// pattern, or outside the rows of kRowMask, read 0.
template <int kCtrl, int kRowMask, class T>
__device__ __forceinline__ T dpp_zero(T v) {
    static_assert(sizeof(T) == 8, "64-bit values");
    uint64_t u;
    __builtin_memcpy(&u, &v, 8);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, kCtrl, kRowMask, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), kCtrl, kRowMask, 0xf, false);
    const uint64_t r = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    T o;
    __builtin_memcpy(&o, &r, 8);
    return o;
}
// Inclusive prefix sum over the wave (lane i gets lanes 0..i) in one fixed
// order: inside each row of 16 by shifts of 1, 2, 4 and 8 lanes
// (row_shr), then the totals of rows 0 and 2 added into rows 1 and 3
// (row_bcast:15) and the total of rows 0-1 into rows 2 and 3 (row_bcast:31).
template <class T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    v += dpp_zero<0x111, 0xf>(v);
    v += dpp_zero<0x112, 0xf>(v);
    v += dpp_zero<0x114, 0xf>(v);
    v += dpp_zero<0x118, 0xf>(v);
    v += dpp_zero<0x142, 0xa>(v);
    v += dpp_zero<0x143, 0xc>(v);
    return v;
}
// v of lane i - 1, 0 in lane 0 (wave_shr:1).
template <class T>
__device__ __forceinline__ T wave_shift_up1(T v) {
    return dpp_zero<0x138, 0xf>(v);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t w;
    w = xor_lane<1>(v);  v = w > v ? w : v;
    w = xor_lane<2>(v);  v = w > v ? w : v;
    w = xor_lane<4>(v);  v = w > v ? w : v;
    w = xor_lane<8>(v);  v = w > v ? w : v;
    w = xor_lane<16>(v); v = w > v ? w : v;
    w = xor_lane<32>(v); v = w > v ? w : v;
    return v;
}

// One compare-exchange stage of a bitonic network: lanes (i, i ^ kStride)
// order their pair descending inside blocks of kSize lanes whose bit kSize
// is clear and ascending in the others (flipped when kDesc is false; at
// kSize = 64 every block is the first one).
template <bool kDesc, int kSize, int kStride>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t v, int lane) {
    const uint64_t o = xor_lane<kStride>(v);
    const bool first_block = (lane & kSize) == 0;
    const bool lower = (lane & kStride) == 0;
    const bool keep_max = (lower == first_block) == kDesc;
    return keep_max ? (o > v ? o : v) : (o < v ? o : v);
}
template <bool kDesc, int kSize, int kStride>
__device__ __forceinline__ uint64_t bitonic_from(uint64_t v, int lane) {
    v = bitonic_stage<kDesc, kSize, kStride>(v, lane);
    if constexpr (kStride > 1) return bitonic_from<kDesc, kSize, kStride / 2>(v, lane);
    else if constexpr (kSize < kWave) return bitonic_from<kDesc, kSize * 2, kSize>(v, lane);
    else return v;
}
// Bitonic sort of one u64 per lane across a wave: descending (lane 0 the
// largest) or ascending.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
    return bitonic_from<true, 2, 1>(v, lane_id());
}
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t v) {
    return bitonic_from<false, 2, 1>(v, lane_id());
}

// Top 64 of a descending and an ascending 64-list (one entry per lane),
// descending: max(a_j, b_j) holds the 64 largest of the union as a bitonic
// sequence, which six half-cleaner stages sort.
template <int kStride>
__device__ __forceinline__ uint64_t half_clean_desc(uint64_t v, int lane) {
    const uint64_t o = xor_lane<kStride>(v);
    const bool lower = (lane & kStride) == 0;
    v = lower ? (o > v ? o : v) : (o < v ? o : v);
    if constexpr (kStride > 1) return half_clean_desc<kStride / 2>(v, lane);
    else return v;
}
__device__ __forceinline__ uint64_t wave_merge_top_asc(uint64_t a, uint64_t b_asc) {
    return half_clean_desc<kWave / 2>(a > b_asc ? a : b_asc, lane_id());
}
// The same for two descending lists.
__device__ __forceinline__ uint64_t wave_merge_top(uint64_t a, uint64_t b) {
    return wave_merge_top_asc(a, wave_reverse(b));
}

// ---- wave reductions on the DPP network (no LDS round trips) --------------
// The steps combine lanes pairwise inside quads, then rows of 16 (rotations),
// then broadcast row results up the wave; lane 63 ends with the full result,
// which readlane hands to every lane.  Lanes whose DPP source does not exist
// see the identity.  The order of the combination is fixed, so results are
// deterministic.  Every lane of the wave must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float identity, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v),
                                                      kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ double dpp_move(double identity, double v) {
    const int64_t iv = __double_as_longlong(v), io = __double_as_longlong(identity);
    const int lo = __builtin_amdgcn_update_dpp((int)io, (int)iv, kCtrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(io >> 32), (int)(iv >> 32), kCtrl, 0xf, 0xf,
                                               false);
    return __longlong_as_double((int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ float readlane63(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double readlane63(double v) {
    const int64_t iv = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)iv, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(iv >> 32), 63);
    return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float wave_max_f32(float v) {
    const float id = -INFINITY;
    v = fmaxf(v, dpp_move<0xb1>(id, v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_move<0x4e>(id, v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_move<0x124>(id, v));  // row_ror:4
    v = fmaxf(v, dpp_move<0x128>(id, v));  // row_ror:8
    v = fmaxf(v, dpp_move<0x142>(id, v));  // row_bcast:15
    v = fmaxf(v, dpp_move<0x143>(id, v));  // row_bcast:31
    return readlane63(v);
}
template <class F>
__device__ __forceinline__ F wave_sum(F v) {
    const F id = (F)0;
    v += dpp_move<0xb1>(id, v);
    v += dpp_move<0x4e>(id, v);
    v += dpp_move<0x124>(id, v);
    v += dpp_move<0x128>(id, v);
    v += dpp_move<0x142>(id, v);
    v += dpp_move<0x143>(id, v);
    return readlane63(v);
}

// Block-wide max of a u64; every thread gets the result.  `tmp` holds kWaves.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* tmp) {
    v = wave_max_u64(v);
    __syncthreads();
    if (lane_id() == 0) tmp[wave_id()] = v;
    __syncthreads();
    uint64_t r = tmp[0];
#pragma unroll
    for (int i = 1; i < kWaves; i++) r = tmp[i] > r ? tmp[i] : r;
    return r;
}

// Block-wide max of a float; every thread gets the result.  `tmp` holds kWaves.
__device__ __forceinline__ float block_max_f32(float v, uint64_t* tmp) {
    v = wave_max_f32(v);
    __syncthreads();
    if (lane_id() == 0) tmp[wave_id()] = (uint64_t)__float_as_uint(v);
    __syncthreads();
    float r = __uint_as_float((uint32_t)tmp[0]);
#pragma unroll
    for (int i = 1; i < kWaves; i++) r = fmaxf(r, __uint_as_float((uint32_t)tmp[i]));
    return r;
}

// Block-wide exclusive prefix sum of one double per thread (fixed order).
template <class T>
__device__ inline T block_exclusive_scan(T v, T* tmp /* kWaves */, T* total) {
    const int lane = lane_id(), w = wave_id();
    const T incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == kWave - 1) tmp[w] = incl;
    __syncthreads();
    T off = 0, tot = 0;
    for (int i = 0; i < kWaves; i++) {
        if (i < w) off += tmp[i];
        tot += tmp[i];
    }
    *total = tot;
    return off + incl - v;
}

// N block-wide exclusive prefix sums at once over a block of kW waves (one
// barrier pair): excl[j] and tot[j] are what block_exclusive_scan gives for
// v[j], bit for bit, at kW = kWaves.
template <int N, int kW = kWaves>
__device__ inline void block_exclusive_scan_n(const double (&v)[N], double* tmp /* N * kW */,
                                              double (&excl)[N], double (&tot)[N]) {
    const int lane = lane_id(), w = wave_id();
    double incl[N];
#pragma unroll
    for (int j = 0; j < N; j++) incl[j] = wave_incl_scan(v[j]);
    __syncthreads();
    if (lane == kWave - 1)
#pragma unroll
        for (int j = 0; j < N; j++) tmp[j * kW + w] = incl[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; j++) {
        double off = 0, t = 0;
        for (int i = 0; i < kW; i++) {
            if (i < w) off += tmp[j * kW + i];
            t += tmp[j * kW + i];
        }
        tot[j] = t;
        excl[j] = off + incl[j] - v[j];
    }
}

// Bitonic sort (descending) of n = power of two u64 keys in LDS.
__device__ inline void block_sort_desc(uint64_t* s, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n >> 1); i += kThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = s[lo], b = s[hi];
                if ((a < b) == desc) {
                    s[lo] = b;
                    s[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---- arguments shared by the step kernels ---------------------------------
// Per-row description of the four distributions of the acceptance
// statistics (sv_stats.h): with e = exp((l - m) / T) on each side, the
// untruncated probability is e * iz and the truncated one [key >= tau] e * kap.
struct StatDesc {
    uint64_t tau_t, tau_d;
    double kap_t, kap_d, iz_t, iz_d;
    float m_t, m_d, c;
    int32_t pad;
};

struct StepArgs {
    const void* target;
    const void* draft;
    int64_t t_stride, d_stride;
    int B, K, V, ntiles;
    int t_rows, d_rows;    // rows per batch entry in each tensor (K + 1 and K for a verify step)
    int stats;             // 1: acceptance statistics instead of a verify step (sv_stats.h)
    int force_full;        // row pass: every unit as an untruncated one
    int g_row;             // grid of the row pass (its records are laid out by it)
    const int32_t* tokens;
    const float* uniforms;
    RowInfo* rows;
    PartSlot* parts;       // piece records of the current position (slot u + w)
    FullStat* tstat;       // [2B][ntiles][kWaves] full-vocab row stats of the current position
    double2* chunks;       // [B][ntiles][kWaves] draw masses (one chunk = one tile)
    int32_t* out_tokens;
    int32_t* out_acc;
    double* diag;
    PosDesc* pos;          // [K+2]: positions 0..K, then the final draw
    int32_t* ulist;        // [K+1][kNumCls][2B] units to stream per position and class
    int32_t* slist;        // [B] rows that draw over the full vocabulary at the end
    FnUnit* fn_unit;       // [2B] nucleus cut of the current position
    uint64_t* hist;        // [units + kGrid][kHistSlot] nucleus histograms of the row pass, slot u + w
    uint64_t* fn_keys;     // [kGrid / 2][kCollectCap] boundary keys of a unit whose cut is split
    int32_t* fn_sync;      // [kGrid / 2][2] per split unit: workgroups arrived, keys reserved
    int32_t* fn_row;       // [B] nucleus units of the row whose cut is complete
    const StepArgs* self;  // a copy of these arguments in device memory (written by the plan)
    StatDesc* sdesc;       // [B] acceptance statistics: the rows' distributions
    double* srec;          // [B][ntiles][kWaves][4] acceptance statistics: partial sums
    double* sout;          // [B][4] acceptance statistics: the result
    // tree verify (tree = 1): node c >= 1 has token tokens[b][c-1] and parent
    // parents[b][c-1] < c; rows are indexed by node
    int tree;
    const int32_t* parents;
    int32_t* out_path;     // [B][K+1] accepted nodes, or null
    double* wchain;        // [B][kMaxKids] masses of the residuals after each rejected child
    int32_t* tlist;        // [kMaxKids][B] full-vocab rows in each child round of a level
    int32_t* tcount;       // [K+1][kMaxKids] their numbers, per level and round
    int32_t* nscr;         // [B][K+1] per-node scratch of the plan (depths, child counts)
    int max_depth, max_kids;  // the tree's bounds: levels after 0, children per node
    // merged launch: the positions d0..K of the rows still live are streamed
    // by one row pass and decided by one cut/decide launch that walks them in
    // order (d0 = 0: the whole step, a dense step; d0 = K + 1: none, one
    // launch pair per position); a unit's code there carries its position,
    // (b (K + 1 - d0) + k - d0) 2 + side
    int d0;
    int ustride;           // entries per class region of a position's unit list
    int32_t* dli;          // dense: [B][K+1][2] index of each unit in its class region
};

// A dense step serves batches whose units over all positions number at most
// kDenseUnits: there the K launch pairs a position-by-position step needs
// cost more than the rows it need not read (section on small batches in the
// design notes: the launches of a position take tens of microseconds, a row
// a fraction of one).
constexpr int kDenseUnits = 1024;
__host__ __device__ __forceinline__ bool dense_eligible(int64_t B, int64_t K) {
    return 2 * B * (K + 1) <= kDenseUnits;
}
// Larger batches merge their last positions: the launch pair of each position
// before d0, then one pair for positions d0..K of the rows still live, with d0
// the earliest position (from 1, leaving at least two positions to merge)
// whose largest possible list, B (2 (K - d0) + 1) units, fits kMergeUnits.
// The merged launch also streams the later positions of rows that reject at
// an earlier one of them; a launch pair costs about as much as streaming a
// few hundred rows, and rows that reach the last positions are the fewer the
// lower the acceptance, so the budget keeps that waste small against the
// launches it saves.  K + 1: no merged launch.
constexpr int kMergeUnits = 3072;
__host__ __device__ __forceinline__ int merge_start(int64_t B, int64_t K) {
    if (dense_eligible(B, K)) return 0;
    for (int64_t d0 = 1; d0 < K; d0++)
        if (B * (2 * (K - d0) + 1) <= kMergeUnits) return (int)d0;
    return (int)K + 1;
}

// Unit codes: b 2 + side in the launch of a position before d0 (the position
// is the launch's), 2B + (b (K + 1 - d0) + k - d0) 2 + side in the merged
// launch after such launches (no 2B in a dense step).  Per-unit state (the
// untruncated records, the nucleus cut) is indexed by the code, so the merged
// launch's codes lie past those of the earlier launches: the records of a row
// that stopped before d0 outlive the merged launch, and the merged units that
// the decisions before d0 list (clearing their state) touch no unit those
// decisions' launch is still cutting.
__device__ __forceinline__ int merged_base(const StepArgs& a) { return a.d0 > 0 ? 2 * a.B : 0; }
__device__ __forceinline__ int unit_code(const StepArgs& a, int b, int k, int side) {
    return k >= a.d0 ? merged_base(a) + (b * (a.K + 1 - a.d0) + (k - a.d0)) * 2 + side
                     : b * 2 + side;
}
// Row of unit u in the launch of position k.
__device__ __forceinline__ int unit_b(const StepArgs& a, int u, int k) {
    return k >= a.d0 ? ((u - merged_base(a)) >> 1) / (a.K + 1 - a.d0) : u >> 1;
}
// Position of unit u in the launch of position k.
__device__ __forceinline__ int unit_pos(const StepArgs& a, int u, int k) {
    return k >= a.d0 ? a.d0 + ((u - merged_base(a)) >> 1) % (a.K + 1 - a.d0) : k;
}
// Row index (within its batch entry's rows) that unit u of row b streams in
// the launch of position / level k.
__device__ __forceinline__ int unit_rowidx(const StepArgs& a, int u, int b, int k) {
    if (k >= a.d0) return unit_pos(a, u, k);
    return a.tree ? a.rows[b].node : k;
}

// Row index (within batch entry b's rows) read at position / level k: the
// position itself in a verify step, the row's current node in a tree verify.
__device__ __forceinline__ int row_at(const StepArgs& a, int b, int k) {
    return a.tree ? a.rows[b].node : k;
}

template <int DT>
__device__ __forceinline__ const void* unit_row(const StepArgs& a, int b, int side, int k) {
    if (side == 0)
        return static_cast<const char*>(a.target) +
               ((int64_t)b * a.t_rows + k) * a.t_stride * Elt<DT>::kSize;
    return static_cast<const char*>(a.draft) +
           ((int64_t)b * a.d_rows + k) * a.d_stride * Elt<DT>::kSize;
}

// The nucleus units of position k (their class region) and their number.
__device__ __forceinline__ const int32_t* nuc_list(const StepArgs& a, int k) {
    return a.ulist + ((int64_t)k * kNumCls + CLS_NUCLEUS) * a.ustride;
}

// Unit at index li of position k's concatenated list; *cls: its class
// region, which is the class of the unit's row.
__device__ __forceinline__ int32_t unit_at(const StepArgs& a, int k, const PosDesc& p, int li,
                                           int* cls) {
    int c = 0;
    while (c < kNumCls - 1 && li >= p.n_cls[c]) li -= p.n_cls[c++];
    *cls = c;
    return a.ulist[((int64_t)k * kNumCls + c) * a.ustride + li];
}

}  // namespace sv
