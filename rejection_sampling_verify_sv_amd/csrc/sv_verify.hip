// sv_verify.hip — host side of the C ABI declared in include/sv.h.
//
// Launch sequence for one verify step (all on the caller's stream, no host
// synchronisation, no device reads on the host):
//   plan_kernel                     classify rows, initialise outputs
//   fn_table_kernel, fn_zero_kernel nucleus-cut constants and histograms
//   for k = 0 .. K:
//     rowpass_kernel<k>             stream the rows still live at position k
//     fn_hist / fn_select /
//     fn_collect / fn_resolve<k>    exact top_p cut of full-vocab nucleus rows
//     decide_kernel<k>              accept / reject / draw for those rows
//   sample_sums_kernel              full-vocab rows: per-chunk draw masses
//   sample_pick_kernel              full-vocab rows: the drawn token
// Positions after a row's first rejection are never read (the first
// rejection ends the row: tinycto.tv "Spekülatif Kod Çözme…", section
// "1. Temel Çalışma Mekanizması").
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include "sv.h"
#include "sv_decide.h"
#include "sv_device.h"
#include "sv_nucleus.h"
#include "sv_rowpass.h"
#include "sv_sample.h"

namespace {

using namespace sv;

constexpr int kTargetBlocks = 2048;  // row-pass blocks wanted per position
constexpr int kMaxSeg = 64;          // decide merges at most 64 x 64 keys

struct Plan {
    int tile, ntiles, nseg, tiles_per_seg, nch;
    size_t off_rows, off_parts, off_chunks, off_fnu, off_hi, off_lo, off_cnt, off_coll, off_ebk,
        bytes;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan* p) {
    if (B <= 0 || K < 1 || V < 2 || (dtype != SV_F32 && dtype != SV_BF16)) return false;
    p->tile = (dtype == SV_F32) ? TileShape<SV_F32>::kTile : TileShape<SV_BF16>::kTile;
    p->ntiles = (V + p->tile - 1) / p->tile;
    int want = (kTargetBlocks + 2 * B - 1) / (2 * B);
    if (want < 1) want = 1;
    int cap = p->ntiles < kMaxSeg ? p->ntiles : kMaxSeg;
    if (want > cap) want = cap;
    p->tiles_per_seg = (p->ntiles + want - 1) / want;
    p->nseg = (p->ntiles + p->tiles_per_seg - 1) / p->tiles_per_seg;
    p->nch = p->ntiles;
    size_t off = 0;
    p->off_rows = off;
    off = align_up(off + sizeof(RowInfo) * (size_t)B, 256);
    p->off_parts = off;
    off = align_up(off + sizeof(PartSlot) * (size_t)B * 2 * p->nseg, 256);
    p->off_chunks = off;
    off = align_up(off + sizeof(double2) * (size_t)B * p->nch, 256);
    const size_t units = (size_t)B * 2;
    p->off_fnu = off;
    off = align_up(off + sizeof(FnUnit) * units, 256);
    p->off_hi = off;
    off = align_up(off + sizeof(uint64_t) * units * kNB, 256);
    p->off_lo = off;
    off = align_up(off + sizeof(uint64_t) * units * kNB, 256);
    p->off_cnt = off;
    off = align_up(off + sizeof(uint32_t) * units * kNB, 256);
    p->off_coll = off;
    off = align_up(off + sizeof(uint64_t) * units * kCollectCap, 256);
    p->off_ebk = off;
    off = align_up(off + sizeof(double) * kNB, 256);
    p->bytes = off;
    return true;
}

thread_local char g_hip_msg[256];

int hip_fail(hipError_t e) {
    snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error: %s", hipGetErrorString(e));
    return SV_EHIP;
}

// Launch order of one step; sv_launch_count / sv_launch_name describe it.
constexpr int kPerPos = 6;
const char* const kPosNames[kPerPos] = {"rowpass", "fn_hist", "fn_select",
                                        "fn_collect", "fn_resolve", "decide"};
int launch_count(int K) { return 3 + kPerPos * (K + 1) + 2; }

const char* launch_name(int K, int i) {
    if (i < 0 || i >= launch_count(K)) return nullptr;
    if (i == 0) return "plan";
    if (i == 1) return "fn_table";
    if (i == 2) return "fn_zero";
    if (i < 3 + kPerPos * (K + 1)) return kPosNames[(i - 3) % kPerPos];
    return (i == 3 + kPerPos * (K + 1)) ? "sample_sums" : "sample_pick";
}

// ev (optional, launch_count+1 events): ev[i] is recorded just before launch
// i and ev[launch_count] after the last launch.
template <int DT, bool kAligned>
int launch_all(const void* target, const void* draft, const int32_t* draft_len,
               const sv_sampler_params* params, const Plan& pl, StepArgs a, FnWork fw, int B,
               hipStream_t st, hipEvent_t const* ev) {
    int n = 0;
    auto mark = [&]() {
        if (ev) (void)hipEventRecord(ev[n], st);
        n++;
    };
    const unsigned seg_blocks = (unsigned)(B * 2 * pl.nseg);
    mark();
    plan_kernel<<<(B + kThreads - 1) / kThreads, kThreads, 0, st>>>(a, B, draft_len, params);
    mark();
    fn_table_kernel<<<(kNB + kThreads - 1) / kThreads, kThreads, 0, st>>>(
        const_cast<double*>(fw.ebk));
    mark();
    fn_zero_kernel<<<(unsigned)(B * 2), kThreads, 0, st>>>(a, fw);
    for (int k = 0; k <= a.K; k++) {
        mark();
        rowpass_kernel<DT, kAligned><<<seg_blocks, kThreads, 0, st>>>(
            target, draft, a.t_stride, a.d_stride, a.K, a.V, k, pl.nseg, pl.tiles_per_seg, a.rows,
            const_cast<PartSlot*>(a.parts));
        mark();
        fn_hist_kernel<DT, kAligned><<<seg_blocks, kThreads, 0, st>>>(a, fw, k, pl.tiles_per_seg);
        mark();
        fn_select_kernel<<<(unsigned)(B * 2), kThreads, 0, st>>>(a, fw, k);
        mark();
        fn_collect_kernel<DT, kAligned><<<seg_blocks, kThreads, 0, st>>>(a, fw, k,
                                                                         pl.tiles_per_seg);
        mark();
        fn_resolve_kernel<<<(unsigned)(B * 2), kThreads, 0, st>>>(a, fw, k);
        mark();
        decide_kernel<DT><<<(unsigned)B, kThreads, 0, st>>>(a, k);
    }
    mark();
    sample_sums_kernel<DT, kAligned><<<(unsigned)(B * pl.nch), kThreads, 0, st>>>(a);
    mark();
    sample_pick_kernel<DT><<<(unsigned)B, kThreads, 0, st>>>(a);
    mark();
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : hip_fail(e);
}

}  // namespace

extern "C" size_t sv_workspace_bytes(int32_t batch, int32_t max_draft, int32_t vocab,
                                     int32_t dtype) {
    Plan p;
    return make_plan(batch, max_draft, vocab, dtype, &p) ? p.bytes : 0;
}

static int verify_impl(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_len,
                       const sv_sampler_params* sampler_params, const float* uniforms,
                       int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg,
                       hipEvent_t const* ev) {
    if (!cfg || !target_logits || !draft_logits || !draft_tokens || !sampler_params ||
        !uniforms || !out_tokens || !out_accept_len)
        return SV_EINVAL;
    const int32_t B = cfg->batch, K = cfg->max_draft, V = cfg->vocab, dt = cfg->dtype;
    Plan pl;
    if (!make_plan(B, K, V, dt, &pl)) return SV_EINVAL;
    const int64_t ts = cfg->target_row_stride ? cfg->target_row_stride : V;
    const int64_t ds = cfg->draft_row_stride ? cfg->draft_row_stride : V;
    if (ts < V || ds < V) return SV_EINVAL;
    if ((int64_t)B * 2 * pl.nseg > 0x7FFFFFFFll || (int64_t)B * pl.nch > 0x7FFFFFFFll)
        return SV_EINVAL;
    if (!cfg->workspace || cfg->workspace_bytes < pl.bytes) return SV_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(cfg->workspace) % 256 != 0) return SV_EWORKSPACE;

    char* ws = static_cast<char*>(cfg->workspace);
    StepArgs a;
    a.target = target_logits;
    a.draft = draft_logits;
    a.t_stride = ts;
    a.d_stride = ds;
    a.K = K;
    a.V = V;
    a.nseg = pl.nseg;
    a.nch = pl.nch;
    a.tokens = draft_tokens;
    a.uniforms = uniforms;
    a.rows = reinterpret_cast<RowInfo*>(ws + pl.off_rows);
    a.parts = reinterpret_cast<const PartSlot*>(ws + pl.off_parts);
    a.chunks = reinterpret_cast<double2*>(ws + pl.off_chunks);
    a.out_tokens = out_tokens;
    a.out_acc = out_accept_len;
    a.diag = cfg->diag;
    FnWork fw;
    fw.unit = reinterpret_cast<FnUnit*>(ws + pl.off_fnu);
    fw.hi = reinterpret_cast<uint64_t*>(ws + pl.off_hi);
    fw.lo = reinterpret_cast<uint64_t*>(ws + pl.off_lo);
    fw.cnt = reinterpret_cast<uint32_t*>(ws + pl.off_cnt);
    fw.coll = reinterpret_cast<uint64_t*>(ws + pl.off_coll);
    fw.ebk = reinterpret_cast<const double*>(ws + pl.off_ebk);
    a.fn_unit = fw.unit;
    a.ebk = fw.ebk;

    const size_t esz = (dt == SV_F32) ? 4 : 2;
    const bool aligned = reinterpret_cast<uintptr_t>(target_logits) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0 &&
                         ((size_t)ts * esz) % 16 == 0 && ((size_t)ds * esz) % 16 == 0;
    hipStream_t st = static_cast<hipStream_t>(cfg->stream);
    if (dt == SV_F32)
        return aligned ? launch_all<SV_F32, true>(target_logits, draft_logits, draft_len,
                                                  sampler_params, pl, a, fw, B, st, ev)
                       : launch_all<SV_F32, false>(target_logits, draft_logits, draft_len,
                                                   sampler_params, pl, a, fw, B, st, ev);
    return aligned ? launch_all<SV_BF16, true>(target_logits, draft_logits, draft_len,
                                               sampler_params, pl, a, fw, B, st, ev)
                   : launch_all<SV_BF16, false>(target_logits, draft_logits, draft_len,
                                                sampler_params, pl, a, fw, B, st, ev);
}

extern "C" int sv_verify(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const int32_t* draft_len,
                         const sv_sampler_params* sampler_params, const float* uniforms,
                         int32_t* out_tokens, int32_t* out_accept_len, const sv_config* cfg) {
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, sampler_params,
                       uniforms, out_tokens, out_accept_len, cfg, nullptr);
}

extern "C" int sv_verify_profiled(const void* target_logits, const void* draft_logits,
                                  const int32_t* draft_tokens, const int32_t* draft_len,
                                  const sv_sampler_params* sampler_params, const float* uniforms,
                                  int32_t* out_tokens, int32_t* out_accept_len,
                                  const sv_config* cfg, void* const* events, int32_t n_events) {
    if (!cfg || !events || n_events < launch_count(cfg->max_draft) + 1) return SV_EINVAL;
    for (int i = 0; i <= launch_count(cfg->max_draft); i++)
        if (!events[i]) return SV_EINVAL;
    return verify_impl(target_logits, draft_logits, draft_tokens, draft_len, sampler_params,
                       uniforms, out_tokens, out_accept_len, cfg,
                       reinterpret_cast<hipEvent_t const*>(events));
}

extern "C" int32_t sv_launch_count(int32_t max_draft) {
    return max_draft >= 1 ? launch_count(max_draft) : 0;
}

extern "C" const char* sv_launch_name(int32_t max_draft, int32_t i) {
    return max_draft >= 1 ? launch_name(max_draft, i) : nullptr;
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
        default:
            return "unknown error code";
    }
}
