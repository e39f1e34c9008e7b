// sv_verify.hip — host side of the C ABI declared in include/sv.h.
//
// Launch sequence for one verify step (all on the caller's stream, no host
// synchronisation, no device reads on the host):
//   plan_kernel                   one workgroup: zero the work counters,
//                                 classify rows, initialise outputs, list the
//                                 units of position 0
//   for k = 0 .. K:
//     rowpass_kernel<k>           stream the units live at position k
//     cut_decide_kernel<k>        exact top_p cut of full-vocab nucleus rows
//                                 from the histograms the row pass left (one
//                                 or, few units, several workgroups per
//                                 unit); accept / reject / draw for every
//                                 live row; list the units of k+1
//   sample_sums_kernel            full-vocab rows: per-chunk draw masses
//   sample_pick_kernel            full-vocab rows: the drawn token
// Positions after a row's first rejection are never read (the first
// rejection ends the row: tinycto.tv "Spekülatif Kod Çözme…", section
// "1. Temel Çalışma Mekanizması").
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sv.h"
#include "sv_decide.h"
#include "sv_device.h"
#include "sv_nucleus.h"
#include "sv_rowpass.h"
#include "sv_sample.h"
#include "sv_stats.h"
#include "sv_tree.h"

namespace {

using namespace sv;

constexpr int kMaxDraft = 1024;

struct Plan {
    int tile, ntiles, ustride;
    size_t off_rows, off_pos, off_ulist, off_slist, off_parts, off_tstat, off_chunks,
        off_fnu, off_hist, off_fnkeys, off_fnsync, off_fnrow, off_self, off_sdesc, off_srec, off_status,
        off_wchain, off_tlist, off_tcount, off_nscr, off_dli, bytes;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan* p) {
    if (B <= 0 || K < 0 || V < 2 || (dtype != SV_F32 && dtype != SV_BF16)) return false;
    if (K > kMaxDraft || (int64_t)B * (K + 1) > 0x3FFFFFFFll || V > 0x7FFFFFFF - (1 << 16))
        return false;
    p->tile = (dtype == SV_F32) ? TileShape<SV_F32>::kTile : TileShape<SV_BF16>::kTile;
    p->ntiles = (V + p->tile - 1) / p->tile;
    // units one launch lists: two per row, or two per row and position in
    // the merged launch (the automatic mode's, which needs the most); unit
    // codes: those, and the 2B of the launches before a merged one
    const int d0 = merge_start(B, K);
    const size_t units = (size_t)B * 2 * (size_t)(d0 <= K ? K + 1 - d0 : 1);
    const size_t codes = units + (d0 >= 1 && d0 <= K ? (size_t)B * 2 : 0);
    const size_t slots = units + kGrid;  // record slot u + w of a (unit, workgroup) piece
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    p->off_rows = take(sizeof(RowInfo) * (size_t)B);
    p->off_pos = take(sizeof(PosDesc) * (size_t)(K + 2));
    p->ustride = (int)units;  // entries per class region of a position's list
    p->off_ulist = take(sizeof(int32_t) * units * kNumCls * (size_t)(K + 1));
    p->off_slist = take(sizeof(int32_t) * (size_t)B);
    p->off_parts = take(sizeof(PartSlot) * slots);
    p->off_tstat = take(sizeof(FullStat) * codes * p->ntiles * kWaves);
    p->off_chunks = take(sizeof(double2) * (size_t)B * p->ntiles * kWaves);
    p->off_fnu = take(sizeof(FnUnit) * codes);
    p->off_hist = take(sizeof(uint64_t) * slots * kHistSlot);
    // split nucleus units: their index in a launch's list is below
    // min(units, kGrid / 2)
    const size_t split_rows = units < (size_t)kGrid / 2 ? units : (size_t)kGrid / 2;
    p->off_fnkeys = take(sizeof(uint64_t) * split_rows * kCollectCap);
    p->off_fnsync = take(sizeof(int32_t) * 2 * split_rows);
    p->off_fnrow = take(sizeof(int32_t) * (size_t)B);
    p->off_self = take(sizeof(StepArgs));
    p->off_sdesc = take(sizeof(StatDesc) * (size_t)B);  // sv_accept_stats
    p->off_srec = take(sizeof(double) * 4 * (size_t)B * p->ntiles * kWaves);
    p->off_status = take(sizeof(int32_t) * (size_t)B);  // sv_sample without out_status
    // sv_verify_tree: residual masses and child-round lists of full-vocab
    // rows, per-node scratch of the plan
    p->off_wchain = take(sizeof(double) * (size_t)B * kMaxKids);
    p->off_tlist = take(sizeof(int32_t) * (size_t)kMaxKids * B);
    p->off_tcount = take(sizeof(int32_t) * (size_t)(K + 1) * kMaxKids);
    p->off_nscr = take(sizeof(int32_t) * (size_t)B * (K + 1));
    p->off_dli = take(sizeof(int32_t) * codes);  // merged launch: list index of each unit
    p->bytes = off;
    return true;
}

thread_local char g_hip_msg[256];

int hip_fail(hipError_t e) {
    snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error: %s", hipGetErrorString(e));
    return SV_EHIP;
}

// Launch order of one step; sv_launch_count / sv_launch_name describe it:
// the plan, a launch pair per position before the merge start d0 and one for
// the merged positions (a dense step: d0 = 0, one pair in all), the draws.
constexpr int kPre = 1;
constexpr int kPerPos = 2;
const char* const kPreNames[kPre] = {"plan"};
const char* const kPosNames[kPerPos] = {"rowpass", "cut_decide"};
// The merge start of a step of this shape in this mode (K + 1: none); -1
// when the mode is not served for the shape.
int step_d0(int B, int K, int mode) {
    if (mode == SV_STEP_POSITIONS) return K + 1;
    if (mode == SV_STEP_DENSE) return dense_eligible(B, K) ? 0 : -1;
    if (mode == SV_STEP_AUTO) return merge_start(B, K);
    return -1;
}
// Launch pairs of a step with merge start d0.
int pairs(int K, int d0) { return (d0 < K ? d0 : K) + 1; }
int launch_count(int B, int K, int mode) {
    const int d0 = step_d0(B, K, mode);
    return d0 < 0 ? 0 : kPre + kPerPos * pairs(K, d0) + 2;
}

const char* launch_name(int B, int K, int mode, int i) {
    if (i < 0 || i >= launch_count(B, K, mode)) return nullptr;
    if (i < kPre) return kPreNames[i];
    const int np = pairs(K, step_d0(B, K, mode));
    if (i < kPre + kPerPos * np) return kPosNames[(i - kPre) % kPerPos];
    return (i == kPre + kPerPos * np) ? "sample_sums" : "sample_pick";
}

// The streaming kernels split their tiles evenly over the grid, so the grid
// is one resident wave of workgroups: compute units x workgroups each unit
// holds at the kernel's register and LDS use (at most kGrid, the record
// slots reserved per position).  A second, partial wave would double the
// time of the workgroups in it.
struct Grids {
    unsigned rowpass, cut, sums, stats;
};

template <class Kern>
unsigned resident_grid(Kern kernel, int cus) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const long g = (long)cus * per_cu;
    return (unsigned)(g < kGrid ? g : kGrid);
}

constexpr int kMaxDevices = 64;

template <int DT, bool kAligned>
int grids_for_device(Grids* out) {
    static std::mutex mu;
    static Grids cache[kMaxDevices];
    static bool have[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < kMaxDevices && have[dev]) {
        *out = cache[dev];
        return SV_OK;
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (cus < 1) cus = 1;
    Grids g;
    g.rowpass = resident_grid(rowpass_kernel<DT, kAligned>, cus);
    g.cut = resident_grid(cut_decide_kernel<DT, kAligned>, cus);
    g.sums = resident_grid(sample_sums_kernel<DT, kAligned>, cus);
    g.stats = resident_grid(stats_stream_kernel<DT, kAligned>, cus);
    (void)hipGetLastError();
    if (dev >= 0 && dev < kMaxDevices) {
        cache[dev] = g;
        have[dev] = true;
    }
    *out = g;
    return SV_OK;
}

// The streaming launches take at most one workgroup per tile of their largest
// possible list: workgroups past that find no work, and a small batch would
// otherwise start hundreds of them, all reading the same list descriptor
// (which delays the few that work by several microseconds).
unsigned stream_grid(unsigned resident, int64_t units, int ntiles) {
    const int64_t t = units * (int64_t)ntiles;
    return (unsigned)(t < (int64_t)resident ? (t > 0 ? t : 1) : (int64_t)resident);
}

// ev (optional, launch_count+1 events): ev[i] is recorded just before launch
// i and ev[launch_count] after the last launch.
template <int DT, bool kAligned>
int launch_all(const int32_t* draft_len, const sv_sampler_params* params, StepArgs a,
               hipStream_t st, hipEvent_t const* ev) {
    Grids g;
    const int rc = grids_for_device<DT, kAligned>(&g);
    if (rc != SV_OK) return rc;
    // units of one row-pass launch: two per row and position in the merged one
    const unsigned grow = stream_grid(
        g.rowpass, (int64_t)2 * a.B * (a.d0 <= a.K ? a.K + 1 - a.d0 : 1), a.ntiles);
    const unsigned gsums = stream_grid(g.sums, a.B, a.ntiles);
    a.g_row = (int)grow;
    int n = 0;
    auto mark = [&]() {
        if (ev) (void)hipEventRecord(ev[n], st);
        n++;
    };
    const int B = a.B;
    // cut_decide: up to kMaxSplit workgroups per nucleus unit
    const unsigned cut_cap = (unsigned)(2 * B * kMaxSplit < kGrid ? 2 * B * kMaxSplit : kGrid);
    const unsigned cut_grid = g.cut < cut_cap ? g.cut : cut_cap;
    const unsigned row_grid = (unsigned)(B < kGrid ? B : kGrid);
    mark();
    plan_kernel<<<plan_grid(a.B, a.K, a.tree, a.d0), kPlanThreads, 0, st>>>(a, draft_len, params);
    for (int k = 0; k <= (a.d0 < a.K ? a.d0 : a.K); k++) {
        mark();
        rowpass_kernel<DT, kAligned><<<grow, kThreads, 0, st>>>(a, k);
        mark();
        cut_decide_kernel<DT, kAligned><<<cut_grid, kThreads, 0, st>>>(a, k);
    }
    mark();
    sample_sums_kernel<DT, kAligned><<<gsums, kThreads, 0, st>>>(a, a.slist,
                                                                &a.pos[a.K + 1].n_sample);
    mark();
    sample_pick_kernel<DT, kAligned><<<row_grid, kPickThreads, 0, st>>>(a);
    mark();
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

// Tree verify: per level the row pass and the cut / decisions, then the
// child rounds of full-vocab rows (sv_tree.h); the final draws at the end.
template <int DT, bool kAligned>
int launch_tree(const int32_t* n_cand, const sv_sampler_params* params, StepArgs a,
                hipStream_t st) {
    Grids g;
    const int rc = grids_for_device<DT, kAligned>(&g);
    if (rc != SV_OK) return rc;
    const unsigned grow = stream_grid(g.rowpass, (int64_t)2 * a.B, a.ntiles);
    const unsigned gsums = stream_grid(g.sums, a.B, a.ntiles);
    a.g_row = (int)grow;
    const int B = a.B;
    const unsigned cut_cap = (unsigned)(2 * B * kMaxSplit < kGrid ? 2 * B * kMaxSplit : kGrid);
    const unsigned cut_grid = g.cut < cut_cap ? g.cut : cut_cap;
    const unsigned row_grid = (unsigned)(B < kGrid ? B : kGrid);
    const unsigned wave_grid = (unsigned)((B + kWaves - 1) / kWaves);
    plan_kernel<<<plan_grid(a.B, a.K, a.tree, a.d0), kPlanThreads, 0, st>>>(a, n_cand, params);
    for (int k = 0; k <= a.max_depth; k++) {
        rowpass_kernel<DT, kAligned><<<grow, kThreads, 0, st>>>(a, k);
        cut_decide_kernel<DT, kAligned><<<cut_grid, kThreads, 0, st>>>(a, k);
        for (int j = 1; j < a.max_kids; j++) {
            sample_sums_kernel<DT, kAligned><<<gsums, kThreads, 0, st>>>(
                a, a.tlist + (int64_t)j * B, a.tcount + k * kMaxKids + j);
            tree_round_kernel<DT><<<wave_grid, kThreads, 0, st>>>(a, k, j);
        }
    }
    sample_sums_kernel<DT, kAligned><<<gsums, kThreads, 0, st>>>(a, a.slist,
                                                                &a.pos[a.K + 1].n_sample);
    sample_pick_kernel<DT, kAligned><<<row_grid, kPickThreads, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

// Acceptance statistics of one position (sv_stats.h): the row pass, the
// nucleus cut (no decisions), the row pass again with every unit
// untruncated, then the statistics.
template <int DT, bool kAligned>
int launch_stats(const sv_sampler_params* params, StepArgs a, hipStream_t st) {
    Grids g;
    const int rc = grids_for_device<DT, kAligned>(&g);
    if (rc != SV_OK) return rc;
    a.g_row = (int)g.rowpass;
    const int B = a.B;
    const unsigned cut_cap = (unsigned)(2 * B * kMaxSplit < kGrid ? 2 * B * kMaxSplit : kGrid);
    const unsigned cut_grid = g.cut < cut_cap ? g.cut : cut_cap;
    const unsigned row_groups = (unsigned)((B + kWaves - 1) / kWaves);
    plan_kernel<<<plan_grid(a.B, a.K, a.tree, a.d0), kPlanThreads, 0, st>>>(a, nullptr, params);
    rowpass_kernel<DT, kAligned><<<g.rowpass, kThreads, 0, st>>>(a, 0);
    cut_decide_kernel<DT, kAligned><<<cut_grid, kThreads, 0, st>>>(a, 0);
    StepArgs full = a;
    full.force_full = 1;
    rowpass_kernel<DT, kAligned><<<g.rowpass, kThreads, 0, st>>>(full, 0);
    stats_prep_kernel<DT><<<row_groups, kThreads, 0, st>>>(a);
    stats_stream_kernel<DT, kAligned><<<g.stats, kThreads, 0, st>>>(a);
    stats_reduce_kernel<<<row_groups, kThreads, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

// Sustainable streaming-read rate: the row pass's tiling (16-byte coalesced
// non-temporal loads, double-buffered tiles, the tiles split evenly over one
// resident wave of workgroups) with nothing per element but a max, so that
// the loads stay live.  Each workgroup folds its maximum (as raw bits, any
// data will do) into *out.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const void* data, int64_t n,
                                                               uint32_t* out) {
    using TS = TileShape<SV_F32>;
    const int64_t T = (n + TS::kTile - 1) / TS::kTile;
    const int64_t t0 = flat_begin(T, (int)gridDim.x, (int)blockIdx.x);
    const int64_t t1 = flat_begin(T, (int)gridDim.x, (int)blockIdx.x + 1);
    if (t0 >= t1) return;
    const int64_t end = t1 * TS::kTile < n ? t1 * TS::kTile : n;
    float m = -INFINITY;
    stream_range<SV_F32, true>(data, t0 * TS::kTile, end,
                               [&](float (&v)[TS::kE], int64_t, bool) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TS::kE; i++) m = fmaxf(m, v[i]);
    });
    __shared__ uint64_t s_red[kWaves];
    const float r = block_max_f32(m, s_red);
    if (threadIdx.x == 0) atomicMax(out, __float_as_uint(r));
}

}  // namespace

extern "C" int sv_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream) {
    if (!data || !out || bytes == 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(data) % 16 != 0 || bytes / 4 > (size_t)INT64_MAX)
        return SV_EINVAL;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_read_kernel, kThreads, 0);
    if (e != hipSuccess) return hip_fail(e);
    const long g = (long)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    hipStream_t st = static_cast<hipStream_t>(stream);
    stream_read_kernel<<<(unsigned)(g < kGrid ? g : kGrid), kThreads, 0, st>>>(
        data, (int64_t)(bytes / 4), out);
    e = hipGetLastError();
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

extern "C" size_t sv_workspace_bytes(int32_t batch, int32_t max_draft, int32_t vocab,
                                     int32_t dtype) {
    Plan p;
    return make_plan(batch, max_draft, vocab, dtype, &p) ? p.bytes : 0;
}

// The tree of a tree verify (null for a verify step).
struct TreeIn {
    const int32_t* parents;
    int32_t* out_path;
    int max_depth, max_kids;
};

static int verify_impl(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_len,
                       const sv_sampler_params* sampler_params, const float* uniforms,
                       int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg,
                       hipEvent_t const* ev, const TreeIn* tree = nullptr) {
    if (!cfg || !target_logits || !sampler_params || !uniforms || !out_tokens || !out_accept_len)
        return SV_EINVAL;
    const int32_t B = cfg->batch, K = cfg->max_draft, V = cfg->vocab, dt = cfg->dtype;
    if (K > 0 && (!draft_logits || !draft_tokens)) return SV_EINVAL;
    Plan pl;
    if (!make_plan(B, K, V, dt, &pl)) return SV_EINVAL;
    const int64_t ts = cfg->target_row_stride ? cfg->target_row_stride : V;
    const int64_t ds = (K > 0 && cfg->draft_row_stride) ? cfg->draft_row_stride : V;
    if (ts < V || ds < V) return SV_EINVAL;
    if (!cfg->workspace || cfg->workspace_bytes < pl.bytes) return SV_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(cfg->workspace) % 256 != 0) return SV_EWORKSPACE;

    char* ws = static_cast<char*>(cfg->workspace);
    StepArgs a;
    a.target = target_logits;
    a.draft = draft_logits;
    a.t_stride = ts;
    a.d_stride = ds;
    a.B = B;
    a.K = K;
    a.V = V;
    a.ntiles = pl.ntiles;
    a.t_rows = K + 1;
    a.d_rows = K;
    a.stats = 0;
    a.force_full = 0;
    a.tokens = draft_tokens;
    a.uniforms = uniforms;
    a.rows = reinterpret_cast<RowInfo*>(ws + pl.off_rows);
    a.parts = reinterpret_cast<PartSlot*>(ws + pl.off_parts);
    a.chunks = reinterpret_cast<double2*>(ws + pl.off_chunks);
    a.out_tokens = out_tokens;
    a.out_acc = out_accept_len;
    a.diag = cfg->diag;
    a.pos = reinterpret_cast<PosDesc*>(ws + pl.off_pos);
    a.ulist = reinterpret_cast<int32_t*>(ws + pl.off_ulist);
    a.slist = reinterpret_cast<int32_t*>(ws + pl.off_slist);
    a.fn_unit = reinterpret_cast<FnUnit*>(ws + pl.off_fnu);
    a.tstat = reinterpret_cast<FullStat*>(ws + pl.off_tstat);
    a.hist = reinterpret_cast<uint64_t*>(ws + pl.off_hist);
    a.fn_keys = reinterpret_cast<uint64_t*>(ws + pl.off_fnkeys);
    a.fn_sync = reinterpret_cast<int32_t*>(ws + pl.off_fnsync);
    a.fn_row = reinterpret_cast<int32_t*>(ws + pl.off_fnrow);
    a.self = reinterpret_cast<const StepArgs*>(ws + pl.off_self);
    a.sdesc = reinterpret_cast<StatDesc*>(ws + pl.off_sdesc);
    a.srec = reinterpret_cast<double*>(ws + pl.off_srec);
    a.sout = nullptr;
    a.g_row = 0;
    a.tree = tree ? 1 : 0;
    a.parents = tree ? tree->parents : nullptr;
    a.out_path = tree ? tree->out_path : nullptr;
    a.wchain = reinterpret_cast<double*>(ws + pl.off_wchain);
    a.tlist = reinterpret_cast<int32_t*>(ws + pl.off_tlist);
    a.tcount = reinterpret_cast<int32_t*>(ws + pl.off_tcount);
    a.nscr = reinterpret_cast<int32_t*>(ws + pl.off_nscr);
    a.max_depth = tree ? tree->max_depth : K;
    a.max_kids = tree ? tree->max_kids : 1;
    const int d0 = tree ? K + 1 : step_d0(B, K, cfg->step_mode);
    if (d0 < 0) return SV_EINVAL;
    a.d0 = d0;
    a.ustride = pl.ustride;
    a.dli = reinterpret_cast<int32_t*>(ws + pl.off_dli);

    const size_t esz = (dt == SV_F32) ? 4 : 2;
    const bool aligned = reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                         ((size_t)ts * esz) % 16 == 0 &&
                         (K == 0 || (reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0 &&
                                     ((size_t)ds * esz) % 16 == 0));
    hipStream_t st = static_cast<hipStream_t>(cfg->stream);
    if (tree) {
        if (dt == SV_F32)
            return aligned ? launch_tree<SV_F32, true>(draft_len, sampler_params, a, st)
                           : launch_tree<SV_F32, false>(draft_len, sampler_params, a, st);
        return aligned ? launch_tree<SV_BF16, true>(draft_len, sampler_params, a, st)
                       : launch_tree<SV_BF16, false>(draft_len, sampler_params, a, st);
    }
    if (dt == SV_F32)
        return aligned ? launch_all<SV_F32, true>(draft_len, sampler_params, a, st, ev)
                       : launch_all<SV_F32, false>(draft_len, sampler_params, a, st, ev);
    return aligned ? launch_all<SV_BF16, true>(draft_len, sampler_params, a, st, ev)
                   : launch_all<SV_BF16, false>(draft_len, sampler_params, a, st, ev);
}

// ---- sv_verify_noalloc: the workspace in a static device array -------------
// One array per GPU, loaded with the code object and held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): its device address is looked up once
// per device with hipGetSymbolAddress and that pointer is what the kernels
// get.  Every call on one GPU shares the array; the plan kernel of each call
// clears the counters that must start at zero.
static constexpr size_t kNoAllocBytes = SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocBytes];

static int scratch_for_device(void** out) {
    static std::mutex mu;
    static void* ptr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return SV_EINVAL;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return SV_OK;
}

extern "C" int sv_verify(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const int32_t* draft_len,
                         const sv_sampler_params* sampler_params, const float* uniforms,
                         int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg) {
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, sampler_params,
                       uniforms, out_tokens, out_accept_len, cfg, nullptr);
}

extern "C" int sv_verify_noalloc(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const int32_t* draft_len,
                                 const sv_sampler_params* sampler_params, const float* uniforms,
                                 int32_t* out_tokens, int32_t* out_accept_len,
                                 const sv_config* cfg) {
    if (!cfg) return SV_EINVAL;
    Plan pl;
    if (!make_plan(cfg->batch, cfg->max_draft, cfg->vocab, cfg->dtype, &pl)) return SV_EINVAL;
    if (pl.bytes > kNoAllocBytes) return SV_ESCRATCH;
    void* ws = nullptr;
    const int rc = scratch_for_device(&ws);
    if (rc != SV_OK) return rc;
    sv_config c = *cfg;
    c.workspace = ws;
    c.workspace_bytes = kNoAllocBytes;
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, sampler_params,
                       uniforms, out_tokens, out_accept_len, &c, nullptr);
}

extern "C" size_t sv_noalloc_scratch_bytes(void) { return kNoAllocBytes; }

extern "C" int sv_verify_tree(const void* target_logits, const void* draft_logits,
                              const int32_t* node_tokens, const int32_t* node_parents,
                              const int32_t* n_cand, const sv_sampler_params* sampler_params,
                              const float* uniforms, int32_t* out_tokens, int32_t* out_accept_len,
                              int32_t* out_path, int32_t max_depth, int32_t max_children,
                              const sv_config* cfg) {
    if (!cfg) return SV_EINVAL;
    const int K = cfg->max_draft;
    if (K > 0 && !node_parents) return SV_EINVAL;
    if (max_depth < 0 || max_depth > K) return SV_EINVAL;
    if (K > 0 && (max_children < 1 || max_children > kMaxKids)) return SV_EINVAL;
    TreeIn t;
    t.parents = node_parents;
    t.out_path = out_path;
    t.max_depth = max_depth;
    t.max_kids = K > 0 ? max_children : 1;
    return verify_impl(target_logits, draft_logits, node_tokens, n_cand, sampler_params, uniforms,
                       out_tokens, out_accept_len, cfg, nullptr, &t);
}

extern "C" int sv_verify_profiled(const void* target_logits, const void* draft_logits,
                                  const int32_t* draft_tokens, const int32_t* draft_len,
                                  const sv_sampler_params* sampler_params, const float* uniforms,
                                  int32_t* out_tokens, int32_t* out_accept_len,
                                  const sv_config* cfg, void* const* events, int32_t n_events) {
    if (!cfg || !events || cfg->batch <= 0 || cfg->max_draft < 0 || cfg->max_draft > kMaxDraft)
        return SV_EINVAL;
    const int nl = launch_count(cfg->batch, cfg->max_draft, cfg->step_mode);
    if (nl == 0 || n_events < nl + 1) return SV_EINVAL;
    for (int i = 0; i <= nl; i++)
        if (!events[i]) return SV_EINVAL;
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, sampler_params,
                       uniforms, out_tokens, out_accept_len, cfg,
                       reinterpret_cast<hipEvent_t const*>(events));
}

extern "C" int sv_sample(const void* logits, const sv_sampler_params* sampler_params,
                         const float* uniforms, int32_t* out_tokens, int32_t* out_status,
                         const sv_config* cfg) {
    if (!cfg) return SV_EINVAL;
    sv_config c = *cfg;
    c.max_draft = 0;
    c.draft_row_stride = 0;
    if (!out_status) {
        Plan pl;
        if (!make_plan(c.batch, 0, c.vocab, c.dtype, &pl)) return SV_EINVAL;
        if (!c.workspace || c.workspace_bytes < pl.bytes ||
            reinterpret_cast<uintptr_t>(c.workspace) % 256 != 0)
            return SV_EWORKSPACE;
        out_status = reinterpret_cast<int32_t*>(static_cast<char*>(c.workspace) + pl.off_status);
    }
    return verify_impl(logits, nullptr, nullptr, nullptr, sampler_params, uniforms, out_tokens,
                       out_status, &c, nullptr);
}

extern "C" int sv_accept_stats(const void* target_logits, const void* draft_logits,
                               const sv_sampler_params* sampler_params, double* out,
                               const sv_config* cfg) {
    if (!cfg || !target_logits || !draft_logits || !sampler_params || !out) return SV_EINVAL;
    const int32_t B = cfg->batch, V = cfg->vocab, dt = cfg->dtype;
    Plan pl;
    if (!make_plan(B, 1, V, dt, &pl)) return SV_EINVAL;
    const int64_t ts = cfg->target_row_stride ? cfg->target_row_stride : V;
    const int64_t ds = cfg->draft_row_stride ? cfg->draft_row_stride : V;
    if (ts < V || ds < V) return SV_EINVAL;
    if (!cfg->workspace || cfg->workspace_bytes < pl.bytes) return SV_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(cfg->workspace) % 256 != 0) return SV_EWORKSPACE;
    char* ws = static_cast<char*>(cfg->workspace);
    StepArgs a;
    a.target = target_logits;
    a.draft = draft_logits;
    a.t_stride = ts;
    a.d_stride = ds;
    a.B = B;
    a.K = 1;  // one draft position: target and draft row b are rows b of their tensors
    a.V = V;
    a.ntiles = pl.ntiles;
    a.t_rows = 1;
    a.d_rows = 1;
    a.stats = 1;
    a.force_full = 0;
    a.tokens = nullptr;
    a.uniforms = nullptr;
    a.rows = reinterpret_cast<RowInfo*>(ws + pl.off_rows);
    a.parts = reinterpret_cast<PartSlot*>(ws + pl.off_parts);
    a.chunks = reinterpret_cast<double2*>(ws + pl.off_chunks);
    a.out_tokens = nullptr;
    a.out_acc = nullptr;
    a.diag = nullptr;
    a.pos = reinterpret_cast<PosDesc*>(ws + pl.off_pos);
    a.ulist = reinterpret_cast<int32_t*>(ws + pl.off_ulist);
    a.slist = reinterpret_cast<int32_t*>(ws + pl.off_slist);
    a.fn_unit = reinterpret_cast<FnUnit*>(ws + pl.off_fnu);
    a.tstat = reinterpret_cast<FullStat*>(ws + pl.off_tstat);
    a.hist = reinterpret_cast<uint64_t*>(ws + pl.off_hist);
    a.fn_keys = reinterpret_cast<uint64_t*>(ws + pl.off_fnkeys);
    a.fn_sync = reinterpret_cast<int32_t*>(ws + pl.off_fnsync);
    a.fn_row = reinterpret_cast<int32_t*>(ws + pl.off_fnrow);
    a.self = reinterpret_cast<const StepArgs*>(ws + pl.off_self);
    a.sdesc = reinterpret_cast<StatDesc*>(ws + pl.off_sdesc);
    a.srec = reinterpret_cast<double*>(ws + pl.off_srec);
    a.sout = out;
    a.g_row = 0;
    a.tree = 0;
    a.parents = nullptr;
    a.out_path = nullptr;
    a.wchain = reinterpret_cast<double*>(ws + pl.off_wchain);
    a.tlist = reinterpret_cast<int32_t*>(ws + pl.off_tlist);
    a.tcount = reinterpret_cast<int32_t*>(ws + pl.off_tcount);
    a.nscr = reinterpret_cast<int32_t*>(ws + pl.off_nscr);
    a.max_depth = 1;
    a.max_kids = 1;
    a.d0 = a.K + 1;
    a.ustride = pl.ustride;
    a.dli = reinterpret_cast<int32_t*>(ws + pl.off_dli);
    const size_t esz = (dt == SV_F32) ? 4 : 2;
    const bool aligned = reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0 &&
                         ((size_t)ts * esz) % 16 == 0 && ((size_t)ds * esz) % 16 == 0;
    hipStream_t st = static_cast<hipStream_t>(cfg->stream);
    if (dt == SV_F32)
        return aligned ? launch_stats<SV_F32, true>(sampler_params, a, st)
                       : launch_stats<SV_F32, false>(sampler_params, a, st);
    return aligned ? launch_stats<SV_BF16, true>(sampler_params, a, st)
                   : launch_stats<SV_BF16, false>(sampler_params, a, st);
}

extern "C" int32_t sv_launch_count(int32_t batch, int32_t max_draft, int32_t step_mode) {
    return (batch > 0 && max_draft >= 0 && max_draft <= kMaxDraft)
               ? launch_count(batch, max_draft, step_mode)
               : 0;
}

extern "C" const char* sv_launch_name(int32_t batch, int32_t max_draft, int32_t step_mode,
                                      int32_t i) {
    return (batch > 0 && max_draft >= 0 && max_draft <= kMaxDraft)
               ? launch_name(batch, max_draft, step_mode, i)
               : nullptr;
}

extern "C" const char* sv_strerror(int code) {
    switch (code) {
        case SV_OK:
            return "ok";
        case SV_EINVAL:
            return "invalid argument (null pointer, size, dtype or stride)";
        case SV_EWORKSPACE:
            return "workspace missing, misaligned or smaller than sv_workspace_bytes()";
        case SV_EHIP:
            return g_hip_msg[0] ? g_hip_msg : "HIP error";
        case SV_ESCRATCH:
            return "shape needs more scratch than sv_verify_noalloc holds "
                   "(sv_workspace_bytes() > SV_NOALLOC_SCRATCH_BYTES); use sv_verify with a "
                   "workspace";
        default:
            return "unknown error code";
    }
}
