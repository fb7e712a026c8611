// specverify C ABI: argument checks, workspace layout and kernel launches.
// The operation and the conventions are documented in include/specverify.h.
#include "specverify.h"
#include "specverify_profile.h"

#include <hip/hip_ext.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "sv_common.hpp"
#include "sv_stats.hpp"
#include "sv_topk.hpp"
#include "sv_select.hpp"
#include "sv_verify.hpp"
#include "sv_likelihood.hpp"
#include "sv_nucleus.hpp"

static_assert(SV_MAX_DRAFT == sv::kMaxDraft, "draft limit mismatch");
static_assert(SV_MAX_VOCAB == sv::kMaxSeg * sv::kSeg, "vocab limit mismatch");
static_assert(sv::kKeepCap == sv::kKeepCapList, "kept-list capacity mismatch");
// the per-row top-p kernel groups a row's 16-byte blocks by at most 64 (adjacent lanes)
static_assert((int64_t)sv::kNucGroups * 64 >= SV_MAX_VOCAB / 4 + 2, "top-p block groups too small for the largest row");
static_assert((int64_t)sv::NucRowSize<true>::kGroups * 64 >= SV_MAX_VOCAB / 4 + 2, "top-p block groups too small for the largest row");

namespace {

// 16-byte loads per thread per chunk in the streaming passes, and whether
// they bypass the caches (nontemporal); both chosen by measurement.
#ifndef SV_STREAM_LOADS
#define SV_STREAM_LOADS 4
#endif
#ifndef SV_CAND_LOADS
#define SV_CAND_LOADS 6
#endif
#ifndef SV_STREAM_NT
#define SV_STREAM_NT 1
#endif
constexpr int kLoads = SV_STREAM_LOADS;      // row statistics (sampling and greedy)
constexpr int kLoadsBig = 8;                 // row statistics over grids much larger than the chip
constexpr int kLoadsBigArgmax = 6;           // the greedy argmax pass over such grids (measured: 93.1 against 94.5 us
                                             // for the step on 2304 rows of 128256 bf16 logits; 4, 8 and 12 slower)
constexpr int64_t kBigGridTiles = 16384;     // 4-load tiles beyond which kLoadsBig is used (8x the resident slots)
constexpr int kCandLoads = SV_CAND_LOADS;   // top-k candidate pass
constexpr bool kNT = SV_STREAM_NT != 0;
constexpr int32_t kCandCap = 512;    // candidate slots per (row, chunk) in the top-k pass
// Largest top_k whose candidate pass takes its tile bound from one key per
// lane (the lane maximum).  Near the pass's own limit (256 lane maxima) that
// bound sinks to the smallest lane maxima and the candidates grow; two keys
// per lane (the lane's two largest block maxima) keep it tighter.  Measured
// on 314 rows of 151936 bf16 logits (us per call, one key / two keys):
// top_k 128: 46.6 / 46.4; 160: 48.6 / 49.1; 200: 57.9 / 50.6; 240: 68.8 / 52.5.
constexpr int32_t kTopkFastPlanMax = 160;
static_assert(kTopkFastPlanMax <= sv::kTopkFastMax, "the candidate pass needs top_k lane maxima");
// Largest top_k that takes the candidate pass with two keys per lane (about
// 400 candidates per tile at top_k 300; tiles past their 512 slots cut to
// their own top_k); above it the exact workgroup-per-row select.  top_k 300:
// 70 us per call, 400: 79 us, against 163 and 166 us for the exact select.
constexpr int32_t kTopkFast2PlanMax = 400;
static_assert(kTopkFast2PlanMax <= sv::kTopkFastMax2, "the candidate pass needs top_k keys");
static_assert(sv::kSpecSlots * sv::kWave <= kCandCap, "speculative select reads past a chunk's candidate slots");
constexpr int kVerifyFullThreads = 1024;  // verify over full rows: 16 waves keep the residual re-read in flight
constexpr int kSplitThreads = 512;        // workgroups of the split verify over full rows
// Workgroups per sequence of the full-row verify: enough to spread a batch's
// residual walks over about 512 workgroups (a batch of 256 sequences or more
// keeps one 1024-thread workgroup per sequence), with at least 4 segments of
// 512 ids each.
int32_t split_groups(int32_t batch, int32_t vocab)
{
    if (batch >= 256) return 1;
    const int32_t nseg = (vocab + sv::kSeg - 1) / sv::kSeg;
    int32_t g = 512 / batch;
    if (g > 16) g = 16;
    if (g > nseg / 4) g = nseg / 4;
    return g < 2 ? 1 : g;
}
constexpr int32_t kDraftSmallRowsMin = 512;  // draft rows from which full-row draft draws use smaller workgroups
constexpr size_t kAlign = 256;
// XCDs of an MI355X: workgroups are dealt to them in turn, workgroup g to XCD g mod 8
#ifndef SV_XCDS
#define SV_XCDS 8
#endif
constexpr int32_t kXcds = SV_XCDS;

enum PlanMode { PLAN_FULL = 0, PLAN_TOPK_FAST = 1, PLAN_TOPK_EXACT = 2, PLAN_GREEDY = 3 };
enum CallKind { CALL_SAMPLE = 0, CALL_GREEDY = 1, CALL_DRAFT = 2, CALL_LIKE = 3 };

struct Plan {
    PlanMode mode;
    int32_t rows_t, rows_d, rows;
    int32_t nchunk;
    int32_t loads;  // 16-byte loads per thread per tile of the streaming pass
    int32_t nchunk2;  // tiles per row pair of the likelihood's pair pass (full rows)
    int32_t groups;   // workgroups per sequence of the split verify over full rows (1: one workgroup)
    int32_t pair_loads;  // 16-byte loads per thread per row in that pass
    int32_t top_k;
    int32_t keys;  // keys per lane of the top-k candidate pass's tile bound (1 or 2)
    float top_p;
    bool topp;  // top_p < 1: the nucleus pass runs after the statistics
    bool desc;  // the consumers read row descriptors (top-k and/or top-p), not chunk partials
    size_t off_partials, off_counts, off_bounds, off_cands, off_descs, off_kept, off_pair, off_segsum, off_tickets,
        bytes;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int vec_of(sv_dtype_t dt) { return dt == SV_DTYPE_F32 ? 4 : 8; }
size_t esize_of(sv_dtype_t dt) { return dt == SV_DTYPE_F32 ? 4 : 2; }

// Calls fn with std::integral_constant<int, DT> for the element type
// (the shape check has already rejected any other value).
template <class F>
sv_status_t by_dtype(sv_dtype_t dt, F&& fn)
{
    switch (dt) {
        case SV_DTYPE_F32: return fn(std::integral_constant<int, sv::DT_F32>{});
        case SV_DTYPE_BF16: return fn(std::integral_constant<int, sv::DT_BF16>{});
        case SV_DTYPE_F16: return fn(std::integral_constant<int, sv::DT_F16>{});
    }
    return SV_ERR_INVALID_ARGUMENT;
}

// Chunks per row of the streaming passes: a row with start misalignment up
// to VEC-1 elements touches at most ceil((V + VEC - 1) / VEC) blocks.
int32_t chunks_for(int32_t vocab, int vec, int loads)
{
    const int64_t nblk = ((int64_t)vocab + 2 * vec - 2) / vec;
    const int64_t per = (int64_t)sv::kThreads * loads;
    return (int32_t)((nblk + per - 1) / per);
}

// Launch a streaming-pass kernel, one tile per workgroup.  With `prof`
// (the benchmark entry points), the launch itself records the caller's
// events right before and after the kernel on the call's stream.
template <class K, class... Args>
void launch_stream_nt(const sv_profile_events_t* prof, K kernel, uint32_t ntiles, uint32_t nt, hipStream_t s,
                      Args... args)
{
    if (prof != nullptr) {
        hipExtLaunchKernelGGL(kernel, dim3(ntiles), dim3(nt), 0, s, prof->start, prof->stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, dim3(ntiles), dim3(nt), 0, s, args...);
    }
}

template <class K, class... Args>
void launch_stream(const sv_profile_events_t* prof, K kernel, uint32_t ntiles, hipStream_t s, Args... args)
{
    launch_stream_nt(prof, kernel, ntiles, sv::kThreads, s, args...);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The caller's dtype field as an integer.  A C caller may store any int in
// it; reading a value outside the enumerators through the C++ enum type is
// undefined, so the bytes are copied out and checked first.
static_assert(sizeof(sv_dtype_t) == sizeof(int32_t), "sv_dtype_t is an int-sized enum");
int32_t dtype_field(const sv_shape_t* sh)
{
    int32_t v;
    memcpy(&v, &sh->dtype, sizeof v);
    return v;
}

sv_status_t check_shape(const sv_shape_t* sh, CallKind kind)
{
    const bool need_draft_rows = kind != CALL_GREEDY;
    if (sh == nullptr) return SV_ERR_INVALID_ARGUMENT;
    if (sh->batch < 1 || sh->vocab < 1 || sh->max_draft < 0 || sh->total_draft < 0)
        return SV_ERR_INVALID_ARGUMENT;
    const int32_t dt = dtype_field(sh);
    if (dt != SV_DTYPE_F32 && dt != SV_DTYPE_BF16 && dt != SV_DTYPE_F16) return SV_ERR_INVALID_ARGUMENT;
    if (sh->cu_draft == nullptr && (int64_t)sh->total_draft != (int64_t)sh->batch * sh->max_draft)
        return SV_ERR_INVALID_ARGUMENT;
    if (sh->cu_draft != nullptr && !aligned(sh->cu_draft, 4)) return SV_ERR_INVALID_ARGUMENT;
    if ((int64_t)sh->total_draft > (int64_t)sh->batch * sh->max_draft) return SV_ERR_INVALID_ARGUMENT;
    if (kind != CALL_DRAFT && sh->target_row_stride < sh->vocab) return SV_ERR_INVALID_ARGUMENT;
    if (need_draft_rows && sh->total_draft > 0 && sh->draft_row_stride < sh->vocab)
        return SV_ERR_INVALID_ARGUMENT;
    if (sh->vocab > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
    if (kind != CALL_LIKE && sh->max_draft > SV_MAX_DRAFT) return SV_ERR_UNSUPPORTED;
    const int64_t rows_t = (int64_t)sh->total_draft + sh->batch;
    if (rows_t > INT32_MAX / 2) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

// Rows of the streaming pass: rows [0, rows_t) are read through RowSet::tgt
// (the target rows, or the draft rows for draft-side sampling), the rest
// through RowSet::drf.
Plan make_plan(const sv_shape_t* sh, CallKind kind, int32_t top_k, float top_p = 1.0f)
{
    const bool greedy = kind == CALL_GREEDY;
    Plan p{};
    p.top_k = top_k;
    p.top_p = top_p;
    p.topp = !greedy && top_p < 1.0f;
    p.rows_t = (kind == CALL_DRAFT || kind == CALL_LIKE) ? sh->total_draft : sh->total_draft + sh->batch;
    p.rows_d = (kind == CALL_SAMPLE || kind == CALL_LIKE) ? sh->total_draft : 0;
    p.rows = p.rows_t + p.rows_d;
    const bool topk = !greedy && top_k > 0 && top_k < sh->vocab;
    if (greedy) {
        p.mode = PLAN_GREEDY;
    } else if (!topk) {
        p.mode = PLAN_FULL;
    } else {
        p.mode = top_k <= kTopkFast2PlanMax ? PLAN_TOPK_FAST : PLAN_TOPK_EXACT;
        p.keys = top_k <= kTopkFastPlanMax ? 1 : 2;
    }
    // Streaming tiles: measured on MI355X, 8 loads per thread beat 4 once the
    // grid holds many times more tiles than the chip keeps resident, and lose
    // below that (fewer, longer tiles leave the last wave of tiles thin).  The
    // top-k candidate pass measured best at 6 (20.5 us against 21.0-21.4 us at
    // 8, and 21.0-21.2 at 7, on 314 rows of 151936 bf16 logits).
    if (p.mode == PLAN_TOPK_FAST) {
        p.loads = kCandLoads;
    } else {
        const int64_t rows_stream = greedy ? p.rows_t : p.rows;
        const bool big = rows_stream * chunks_for(sh->vocab, vec_of(sh->dtype), kLoads) > kBigGridTiles;
        p.loads = big ? (greedy ? kLoadsBigArgmax : kLoadsBig) : kLoads;
    }
    p.nchunk = chunks_for(sh->vocab, vec_of(sh->dtype), p.loads);
    p.desc = (p.mode == PLAN_TOPK_FAST || p.mode == PLAN_TOPK_EXACT) || p.topp;
    size_t off = 0;
    const size_t slots = (size_t)p.rows * (size_t)p.nchunk;
    if (p.mode == PLAN_FULL) {
        if (!p.topp) {  // with top-p, one kernel per row writes row descriptors instead of chunk partials
            p.off_partials = off;
            off = align_up(off + slots * sizeof(sv::PartialFull));
        }
        p.groups = (kind == CALL_SAMPLE && !p.topp) ? split_groups(sh->batch, sh->vocab) : 1;
        if (p.groups > 1) {
            const size_t nseg = (size_t)(sh->vocab + sv::kSeg - 1) / sv::kSeg;
            p.off_segsum = off;
            off = align_up(off + (size_t)sh->batch * nseg * sizeof(double));
            p.off_tickets = off;
            off = align_up(off + (size_t)sh->batch * sv::kTicketStride * sizeof(int32_t));
        }
        if (kind == CALL_LIKE && !p.topp) {
            const bool big2 =
                (int64_t)p.rows_t * chunks_for(sh->vocab, vec_of(sh->dtype), sv::kPairLoads) > kBigGridTiles;
            p.pair_loads = big2 ? sv::kPairLoadsBig : sv::kPairLoads;
            p.nchunk2 = chunks_for(sh->vocab, vec_of(sh->dtype), p.pair_loads);
            p.off_pair = off;
            off = align_up(off + (size_t)p.rows_t * (size_t)p.nchunk2 * sizeof(double));
        }
        if (p.topp) {  // the nucleus pass writes descriptors and kept lists
            p.off_descs = off;
            off = align_up(off + (size_t)p.rows * sizeof(sv::RowDesc));
            p.off_kept = off;
            off = align_up(off + (size_t)p.rows * sv::kKeepCap * sizeof(sv::KeptEntry));
        }
    } else if (p.mode == PLAN_GREEDY) {
        p.off_partials = off;
        off = align_up(off + slots * sizeof(sv::PartialArg));
    } else {
        if (p.mode == PLAN_TOPK_FAST) {
            p.off_counts = off;
            off = align_up(off + slots * sizeof(int32_t));
            p.off_bounds = off;
            off = align_up(off + slots * sizeof(float));
            p.off_cands = off;
            off = align_up(off + slots * (size_t)kCandCap * sizeof(sv::KeptEntry));
        }
        p.off_descs = off;
        off = align_up(off + (size_t)p.rows * sizeof(sv::RowDesc));
        p.off_kept = off;
        off = align_up(off + (size_t)p.rows * sv::kKeepCap * sizeof(sv::KeptEntry));
    }
    p.bytes = off == 0 ? kAlign : off;
    return p;
}

template <class T>
T* ws_at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

sv_status_t launch_status()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// The streaming pass and, with top-k, the per-row select over the rows of rs:
// fills va.partials (full rows) or va.descs / va.kept (top-k).
template <int DT>
sv_status_t run_stats_topk(const sv_shape_t* sh, const Plan& p, const sv::RowSet& rs, float c, void* ws,
                           hipStream_t stream, sv::VerifyArgs& va, const sv_profile_events_t* prof)
{
    const int32_t top_k = p.top_k;
    const uint32_t grid_stream = (uint32_t)((int64_t)p.rows * p.nchunk);
    if (p.mode == PLAN_FULL) {
        sv::PartialFull* part = ws_at<sv::PartialFull>(ws, p.off_partials);
        int32_t* tickets = p.groups > 1 ? ws_at<int32_t>(ws, p.off_tickets) : nullptr;
        const int32_t nzero = p.groups > 1 ? sh->batch * sv::kTicketStride : 0;
        if (p.loads == kLoadsBig) {
            launch_stream(prof, sv::row_stats_kernel<DT, sv::MODE_FULL, kLoadsBig, kNT, true>, grid_stream, stream, rs,
                          sh->vocab, p.nchunk, (int32_t)grid_stream, c, (void*)part, tickets, nzero);
        } else {
            launch_stream(prof, sv::row_stats_kernel<DT, sv::MODE_FULL, kLoads, kNT>, grid_stream, stream, rs,
                          sh->vocab, p.nchunk, (int32_t)grid_stream, c, (void*)part, tickets, nzero);
        }
        va.partials = part;
        return launch_status();
    }
    sv::RowDesc* descs = ws_at<sv::RowDesc>(ws, p.off_descs);
    sv::KeptEntry* kept = ws_at<sv::KeptEntry>(ws, p.off_kept);
    int32_t* counts = nullptr;
    float* bounds = nullptr;
    sv::KeptEntry* cands = nullptr;
    if (p.mode == PLAN_TOPK_FAST) {
        counts = ws_at<int32_t>(ws, p.off_counts);
        bounds = ws_at<float>(ws, p.off_bounds);
        cands = ws_at<sv::KeptEntry>(ws, p.off_cands);
        // tiles grouped by XCD so that each row's candidates are in the L2 of
        // the XCD that runs the row's select (workgroup `row` of the next kernel)
        const uint32_t xrows = (uint32_t)((p.rows + kXcds - 1) / kXcds * kXcds);
        if (p.keys == 1) {
            launch_stream(prof, sv::topk_cand_kernel<DT, kCandLoads, kNT, 1>, xrows * (uint32_t)p.nchunk, stream, rs,
                          sh->vocab, p.nchunk, (int32_t)grid_stream, top_k, kCandCap, counts, bounds, cands,
                          (int32_t)kXcds);
        } else {
            launch_stream(prof, sv::topk_cand_kernel<DT, kCandLoads, kNT, 2>, xrows * (uint32_t)p.nchunk, stream, rs,
                          sh->vocab, p.nchunk, (int32_t)grid_stream, top_k, kCandCap, counts, bounds, cands,
                          (int32_t)kXcds);
        }
        if (launch_status() != SV_OK) return SV_ERR_HIP;
        // one workgroup per row; rows whose chunks overflowed take the exact path inside
        if (p.topp)
            hipLaunchKernelGGL((sv::topk_select_wave_kernel<DT, true>), dim3(p.rows), dim3(sv::kSelWaves * sv::kWave), 0,
                               stream, rs, sh->vocab, p.nchunk, top_k, kCandCap, c, p.top_p, counts, bounds, cands, descs,
                               kept);
        else
            hipLaunchKernelGGL((sv::topk_select_wave_kernel<DT, false>), dim3(p.rows), dim3(sv::kSelWaves * sv::kWave), 0,
                               stream, rs, sh->vocab, p.nchunk, top_k, kCandCap, c, 1.0f, counts, bounds, cands, descs,
                               kept);
    } else {
        hipLaunchKernelGGL((sv::topk_select_kernel<DT>), dim3(p.rows), dim3(sv::kThreads), 0, stream, rs, sh->vocab,
                           top_k, c, (int32_t)sv::kKeepCap, descs, kept);
    }
    va.descs = descs;
    va.kept = kept;
    return launch_status();
}

// The streaming pass, the top-k select when top-k is on, and the top-p
// nucleus pass when top_p < 1 (which turns full-row partials into row
// descriptors too).
template <int DT>
sv_status_t run_stats(const sv_shape_t* sh, const Plan& p, const sv::RowSet& rs, float c, void* ws,
                      hipStream_t stream, sv::VerifyArgs& va, const sv_profile_events_t* prof)
{
    if (p.mode == PLAN_FULL && p.topp) {
        // full rows with top-p: statistics and cut in one kernel per row (it
        // reads every row, so it is the timed streaming pass)
        const sv::NucArgs na{rs, sh->vocab, p.rows, c, p.top_p,
                             ws_at<sv::RowDesc>(ws, p.off_descs), ws_at<sv::KeptEntry>(ws, p.off_kept)};
        // (+1: a row that starts inside a block covers one more)
        if ((int64_t)sh->vocab <= (int64_t)(sv::kNucSmallBlocks - 1) * sv::Dt<DT>::kVec)
            launch_stream_nt(prof, sv::nucleus_row_kernel<DT, sv::kNucRowThreads, true>, (uint32_t)p.rows,
                             (uint32_t)sv::kNucRowThreads, stream, na);
        else
            launch_stream_nt(prof, sv::nucleus_row_kernel<DT, sv::kNucRowThreads, false>, (uint32_t)p.rows,
                             (uint32_t)sv::kNucRowThreads, stream, na);
        va.descs = na.descs;
        va.kept = na.kept;
        return launch_status();
    }
    if (run_stats_topk<DT>(sh, p, rs, c, ws, stream, va, prof) != SV_OK) return SV_ERR_HIP;
    // (the candidate path's select narrows its rows by top-p itself)
    if (!p.topp || p.mode == PLAN_TOPK_FAST) return SV_OK;
    // a top-k row's kept list (or a kept set that outgrew it) narrowed by top-p
    const sv::NucArgs na{rs, sh->vocab, p.rows, c, p.top_p,
                         ws_at<sv::RowDesc>(ws, p.off_descs), ws_at<sv::KeptEntry>(ws, p.off_kept)};
    hipLaunchKernelGGL((sv::nucleus_kernel<DT>), dim3(p.rows), dim3(sv::kThreads), 0, stream, na);
    va.descs = na.descs;
    va.kept = na.kept;
    return launch_status();
}

sv::VerifyArgs base_args(const sv_shape_t* sh, const Plan& p, const sv::RowSet& rs, float c, uint64_t seed,
                         uint32_t offset)
{
    sv::VerifyArgs va{};
    va.rs = rs;
    va.cu = sh->cu_draft;
    va.batch = sh->batch;
    va.kmax = sh->max_draft;
    va.total_draft = sh->total_draft;
    va.vocab = sh->vocab;
    va.c = c;
    va.seed = seed;
    va.offset = offset;
    va.nchunk = p.nchunk;
    va.chunk_blocks = sv::kThreads * p.loads;
    return va;
}

template <int DT>
sv_status_t run_sample(const sv_shape_t* sh, const Plan& p, const void* tgt, const void* drf,
                       const int32_t* ids, float c, uint64_t seed, uint32_t offset,
                       int32_t* out_tokens, int32_t* out_nacc, float* out_probs, float* out_z, void* ws,
                       hipStream_t stream, int32_t argmax_draw, const sv_profile_events_t* prof)
{
    const size_t es = esize_of(sh->dtype);
    const sv::RowSet rs{static_cast<const char*>(tgt), static_cast<const char*>(drf),
                        (int64_t)(sh->target_row_stride * (int64_t)es), (int64_t)(sh->draft_row_stride * (int64_t)es),
                        p.rows_t};
    sv::VerifyArgs va = base_args(sh, p, rs, c, seed, offset);
    va.ids = ids;
    va.out_tokens = out_tokens;
    va.out_nacc = out_nacc;
    va.out_probs = out_probs;
    va.out_zmass = out_z;
    va.argmax_draw = argmax_draw;
    if (run_stats<DT>(sh, p, rs, c, ws, stream, va, prof) != SV_OK) return SV_ERR_HIP;
    if (!p.desc && p.groups > 1 && argmax_draw == 0) {
        const sv::SplitArgs sa{va, ws_at<double>(ws, p.off_segsum), ws_at<int32_t>(ws, p.off_tickets)};
        hipLaunchKernelGGL((sv::verify_split_kernel<DT, kSplitThreads>), dim3(sh->batch, p.groups),
                           dim3(kSplitThreads), 0, stream, sa);
    } else if (!p.desc) {
        hipLaunchKernelGGL((sv::verify_kernel<DT, false, kVerifyFullThreads>), dim3(sh->batch), dim3(kVerifyFullThreads), 0,
                           stream, va);
    } else if (p.mode == PLAN_FULL) {  // top-p over full rows: a nucleus may still be a masked full row
        hipLaunchKernelGGL((sv::verify_kernel<DT, true, kVerifyFullThreads>), dim3(sh->batch), dim3(kVerifyFullThreads), 0,
                           stream, va);
    } else {
        hipLaunchKernelGGL((sv::verify_kernel<DT, true, sv::kThreads>), dim3(sh->batch), dim3(sv::kThreads), 0, stream,
                           va);
    }
    return launch_status();
}

template <int DT>
sv_status_t run_draft(const sv_shape_t* sh, const Plan& p, const void* drf, float c, uint64_t seed, uint32_t offset,
                      int32_t* out_ids, void* ws, hipStream_t stream, const sv_profile_events_t* prof)
{
    const size_t es = esize_of(sh->dtype);
    // the draft rows are the streamed rows
    const sv::RowSet rs{static_cast<const char*>(drf), nullptr, (int64_t)(sh->draft_row_stride * (int64_t)es), 0,
                        p.rows_t};
    sv::VerifyArgs va = base_args(sh, p, rs, c, seed, offset);
    va.out_tokens = out_ids;
    if (run_stats<DT>(sh, p, rs, c, ws, stream, va, prof) != SV_OK) return SV_ERR_HIP;
    const dim3 grid((uint32_t)sh->batch, (uint32_t)sh->max_draft);  // max_draft <= SV_MAX_DRAFT fits grid y
    if (!p.desc) {
        // one chunk per row is walked: with many rows, smaller workgroups,
        // two per CU (measured: 150 -> 130 us on 2048 rows of 128256; slower
        // on 256 rows of 50304, which do not fill the chip either way)
        if (sh->total_draft >= kDraftSmallRowsMin) {
            hipLaunchKernelGGL((sv::draft_draw_kernel<DT, false, sv::kDraftChunkThreads>), grid,
                               dim3(sv::kDraftChunkThreads), 0, stream, va);
        } else {
            hipLaunchKernelGGL((sv::draft_draw_kernel<DT, false, kVerifyFullThreads>), grid, dim3(kVerifyFullThreads),
                               0, stream, va);
        }
    } else if (p.mode == PLAN_FULL) {
        hipLaunchKernelGGL((sv::draft_draw_kernel<DT, true, kVerifyFullThreads>), grid, dim3(kVerifyFullThreads), 0,
                           stream, va);
    } else {
        hipLaunchKernelGGL((sv::draft_draw_kernel<DT, true, sv::kThreads>), grid, dim3(sv::kThreads), 0, stream, va);
    }
    return launch_status();
}

template <int DT>
sv_status_t run_likelihood(const sv_shape_t* sh, const Plan& p, const void* tgt, const void* drf,
                           const int32_t* tokens, float c, float* out_terms, float* out_beta,
                           double* out_nll, void* ws, hipStream_t stream, const sv_profile_events_t* prof)
{
    const size_t es = esize_of(sh->dtype);
    const sv::RowSet rs{static_cast<const char*>(tgt), static_cast<const char*>(drf),
                        (int64_t)(sh->target_row_stride * (int64_t)es), (int64_t)(sh->draft_row_stride * (int64_t)es),
                        p.rows_t};
    sv::LikArgs la{};
    la.rs = rs;
    la.cu = sh->cu_draft;
    la.batch = sh->batch;
    la.kmax = sh->max_draft;
    la.rows = sh->total_draft;
    la.vocab = sh->vocab;
    la.tokens = tokens;
    la.c = c;
    la.nchunk = p.nchunk;
    la.nchunk2 = p.nchunk2;
    la.out_terms = out_terms;
    la.out_beta = out_beta;
    la.out_nll = out_nll;
    if (sh->total_draft > 0) {
        sv::VerifyArgs va = base_args(sh, p, rs, c, 0, 0);
        if (run_stats<DT>(sh, p, rs, c, ws, stream, va, prof) != SV_OK) return SV_ERR_HIP;
        la.partials = va.partials;
        la.descs = va.descs;
        la.kept = va.kept;
        if (!p.desc && out_beta != nullptr) {
            double* pair = ws_at<double>(ws, p.off_pair);
            const sv::PairArgs pa{rs, sh->vocab, sh->total_draft, va.partials, p.nchunk, p.nchunk2, c, pair};
            const uint32_t grid = (uint32_t)((int64_t)sh->total_draft * p.nchunk2);
            if (p.pair_loads == sv::kPairLoadsBig) {
                hipLaunchKernelGGL((sv::pair_min_kernel<DT, sv::kPairLoadsBig>), dim3(grid), dim3(sv::kThreads), 0,
                                   stream, pa);
            } else {
                hipLaunchKernelGGL((sv::pair_min_kernel<DT, sv::kPairLoads>), dim3(grid), dim3(sv::kThreads), 0,
                                   stream, pa);
            }
            if (launch_status() != SV_OK) return SV_ERR_HIP;
            la.pair = pair;
        }
    }
    if (!p.desc) {
        hipLaunchKernelGGL((sv::likelihood_kernel<DT, false>), dim3(sh->batch), dim3(sv::kThreads), 0, stream, la);
    } else {
        hipLaunchKernelGGL((sv::likelihood_kernel<DT, true>), dim3(sh->batch), dim3(sv::kThreads), 0, stream, la);
    }
    return launch_status();
}

template <int DT>
sv_status_t run_greedy(const sv_shape_t* sh, const Plan& p, const void* tgt, const int32_t* ids,
                       int32_t* out_tokens, int32_t* out_nacc, void* ws, hipStream_t stream,
                       const sv_profile_events_t* prof)
{
    const size_t es = esize_of(sh->dtype);
    sv::RowSet rs{static_cast<const char*>(tgt), nullptr, (int64_t)(sh->target_row_stride * (int64_t)es), 0,
                  p.rows_t};
    sv::PartialArg* part = ws_at<sv::PartialArg>(ws, p.off_partials);
    const uint32_t grid_stream = (uint32_t)((int64_t)p.rows_t * p.nchunk);
    if (p.loads == kLoadsBigArgmax) {
        launch_stream(prof, sv::row_stats_kernel<DT, sv::MODE_ARGMAX, kLoadsBigArgmax, kNT>, grid_stream, stream, rs,
                      sh->vocab, p.nchunk, (int32_t)grid_stream, 0.0f, (void*)part, (int32_t*)nullptr, (int32_t)0);
    } else {
        launch_stream(prof, sv::row_stats_kernel<DT, sv::MODE_ARGMAX, kLoads, kNT>, grid_stream, stream, rs,
                      sh->vocab, p.nchunk, (int32_t)grid_stream, 0.0f, (void*)part, (int32_t*)nullptr, (int32_t)0);
    }
    if (launch_status() != SV_OK) return SV_ERR_HIP;
    sv::GreedyArgs ga{sh->cu_draft, sh->batch, sh->max_draft, sh->total_draft, sh->vocab, ids, part, p.nchunk,
                      out_tokens, out_nacc};
    hipLaunchKernelGGL(sv::greedy_kernel, dim3((sh->batch + sv::kWaves - 1) / sv::kWaves), dim3(sv::kThreads), 0,
                       stream, ga);
    return launch_status();
}

// c = fl32(log2(e) / T): the softmax's exp(l / T) is computed as exp2(l * c).
float scale_of(float temperature) { return (float)(1.4426950408889634 / (double)temperature); }

// Temperature, top-k and top-p arguments shared by the sampling calls.  A
// temperature so small that c overflows fp32 (T below about 4.2e-39) is
// rejected: every weight would be inf/NaN.
bool filters_ok(const sv_shape_t* sh, float temperature, int32_t top_k, float top_p)
{
    return temperature > 0.0f && isfinite(temperature) && isfinite(scale_of(temperature)) && top_k >= 0 &&
           top_k <= sh->vocab && top_p > 0.0f && top_p <= 1.0f;
}

// Shape, filters and plan of a sampling verify (no pointer is looked at).
sv_status_t sample_plan(const sv_shape_t* shape, float temperature, int32_t top_k, float top_p, Plan* p)
{
    sv_status_t st = check_shape(shape, CALL_SAMPLE);
    if (st != SV_OK) return st;
    if (!filters_ok(shape, temperature, top_k, top_p)) return SV_ERR_INVALID_ARGUMENT;
    *p = make_plan(shape, CALL_SAMPLE, top_k, top_p);
    if (((int64_t)p->rows + kXcds) * p->nchunk > INT32_MAX) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

// The data pointers of a sampling verify: present where the shape needs them, aligned.
sv_status_t sample_pointers(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_ids, const int32_t* out_tokens, const int32_t* out_num_accepted,
                            const float* out_probs, const float* out_residual_mass)
{
    const size_t es = esize_of(shape->dtype);
    if (target_logits == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARGUMENT;
    if (shape->total_draft > 0 && (draft_logits == nullptr || draft_ids == nullptr)) return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(target_logits, es) || (draft_logits != nullptr && !aligned(draft_logits, es)))
        return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) || (draft_ids && !aligned(draft_ids, 4)) ||
        (out_probs && !aligned(out_probs, 4)) || (out_residual_mass && !aligned(out_residual_mass, 4)))
        return SV_ERR_INVALID_ARGUMENT;
    return SV_OK;
}

sv_status_t launch_sample(const sv_shape_t* shape, const Plan& p, const void* target_logits, const void* draft_logits,
                          const int32_t* draft_ids, float temperature, uint64_t seed, uint32_t offset,
                          int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs, float* out_residual_mass,
                          void* workspace, hipStream_t stream, int32_t argmax_draw, const sv_profile_events_t* prof)
{
    const float c = scale_of(temperature);
    return by_dtype(shape->dtype, [&](auto dt) {
        return run_sample<decltype(dt)::value>(shape, p, target_logits, draft_logits, draft_ids, c, seed,
                                               offset, out_tokens, out_num_accepted, out_probs, out_residual_mass,
                                               workspace, stream, argmax_draw, prof);
    });
}

sv_status_t verify_sample_common(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_ids, float temperature, int32_t top_k, float top_p, uint64_t seed,
                                 uint32_t offset, int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                 float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                                 hipStream_t stream, int32_t argmax_draw, const sv_profile_events_t* prof)
{
    if (workspace_bytes == nullptr) return SV_ERR_INVALID_ARGUMENT;
    Plan p;
    sv_status_t st = sample_plan(shape, temperature, top_k, top_p, &p);
    if (st != SV_OK) return st;
    if (workspace == nullptr) {
        *workspace_bytes = p.bytes;
        return SV_OK;
    }
    st = sample_pointers(shape, target_logits, draft_logits, draft_ids, out_tokens, out_num_accepted, out_probs,
                         out_residual_mass);
    if (st != SV_OK) return st;
    if (!aligned(workspace, kAlign)) return SV_ERR_INVALID_ARGUMENT;
    if (*workspace_bytes < p.bytes) return SV_ERR_WORKSPACE_TOO_SMALL;
    return launch_sample(shape, p, target_logits, draft_logits, draft_ids, temperature, seed, offset, out_tokens,
                         out_num_accepted, out_probs, out_residual_mass, workspace, stream, argmax_draw, prof);
}

sv_status_t verify_greedy_common(const sv_shape_t* shape, const void* target_logits, const int32_t* draft_ids,
                               int32_t* out_tokens, int32_t* out_num_accepted, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream,
                                 const sv_profile_events_t* prof)
{
    if (workspace_bytes == nullptr) return SV_ERR_INVALID_ARGUMENT;
    sv_status_t st = check_shape(shape, CALL_GREEDY);
    if (st != SV_OK) return st;
    const Plan p = make_plan(shape, CALL_GREEDY, 0);
    if ((int64_t)p.rows_t * p.nchunk > INT32_MAX) return SV_ERR_UNSUPPORTED;
    if (workspace == nullptr) {
        *workspace_bytes = p.bytes;
        return SV_OK;
    }
    const size_t es = esize_of(shape->dtype);
    if (target_logits == nullptr || out_tokens == nullptr || out_num_accepted == nullptr) return SV_ERR_INVALID_ARGUMENT;
    if (shape->total_draft > 0 && draft_ids == nullptr) return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(target_logits, es) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
        (draft_ids && !aligned(draft_ids, 4)))
        return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, kAlign)) return SV_ERR_INVALID_ARGUMENT;
    if (*workspace_bytes < p.bytes) return SV_ERR_WORKSPACE_TOO_SMALL;
    return by_dtype(shape->dtype, [&](auto dt) {
        return run_greedy<decltype(dt)::value>(shape, p, target_logits, draft_ids, out_tokens, out_num_accepted,
                                               workspace, stream, prof);
    });
}

sv_status_t draft_sample_common(const sv_shape_t* shape, const void* draft_logits, float temperature, int32_t top_k,
                              float top_p, uint64_t seed, uint32_t offset, int32_t* out_ids, void* workspace,
                              size_t* workspace_bytes, hipStream_t stream,
                                const sv_profile_events_t* prof)
{
    if (workspace_bytes == nullptr) return SV_ERR_INVALID_ARGUMENT;
    sv_status_t st = check_shape(shape, CALL_DRAFT);
    if (st != SV_OK) return st;
    if (!filters_ok(shape, temperature, top_k, top_p)) return SV_ERR_INVALID_ARGUMENT;
    const Plan p = make_plan(shape, CALL_DRAFT, top_k, top_p);
    if (((int64_t)p.rows + kXcds) * p.nchunk > INT32_MAX) return SV_ERR_UNSUPPORTED;
    if (workspace == nullptr) {
        *workspace_bytes = p.bytes;
        return SV_OK;
    }
    if (shape->total_draft > 0 && (draft_logits == nullptr || out_ids == nullptr)) return SV_ERR_INVALID_ARGUMENT;
    if ((draft_logits != nullptr && !aligned(draft_logits, esize_of(shape->dtype))) ||
        (out_ids != nullptr && !aligned(out_ids, 4)))
        return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, kAlign)) return SV_ERR_INVALID_ARGUMENT;
    if (*workspace_bytes < p.bytes) return SV_ERR_WORKSPACE_TOO_SMALL;
    if (shape->total_draft == 0 || shape->max_draft == 0) return SV_OK;  // no draft rows: nothing to draw

    const float c = scale_of(temperature);
    return by_dtype(shape->dtype, [&](auto dt) {
        return run_draft<decltype(dt)::value>(shape, p, draft_logits, c, seed, offset, out_ids, workspace, stream,
                                              prof);
    });
}

sv_status_t token_likelihood_common(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                                  const int32_t* tokens, float temperature, int32_t top_k, float top_p,
                                  float* out_terms,
                                  float* out_beta, double* out_nll, void* workspace, size_t* workspace_bytes,
                                  hipStream_t stream, const sv_profile_events_t* prof)
{
    if (workspace_bytes == nullptr) return SV_ERR_INVALID_ARGUMENT;
    sv_status_t st = check_shape(shape, CALL_LIKE);
    if (st != SV_OK) return st;
    if (!filters_ok(shape, temperature, top_k, top_p)) return SV_ERR_INVALID_ARGUMENT;
    const Plan p = make_plan(shape, CALL_LIKE, top_k, top_p);
    if (((int64_t)p.rows + kXcds) * p.nchunk > INT32_MAX || (int64_t)p.rows_t * (p.nchunk2 > 0 ? p.nchunk2 : 1) > INT32_MAX)
        return SV_ERR_UNSUPPORTED;
    if (workspace == nullptr) {
        *workspace_bytes = p.bytes;
        return SV_OK;
    }
    if (out_terms == nullptr && out_beta == nullptr && out_nll == nullptr) return SV_ERR_INVALID_ARGUMENT;
    const size_t es = esize_of(shape->dtype);
    if (shape->total_draft > 0 && (target_logits == nullptr || draft_logits == nullptr || tokens == nullptr))
        return SV_ERR_INVALID_ARGUMENT;
    if ((target_logits && !aligned(target_logits, es)) || (draft_logits && !aligned(draft_logits, es)) ||
        (tokens && !aligned(tokens, 4)) || (out_terms && !aligned(out_terms, 4)) ||
        (out_beta && !aligned(out_beta, 4)) || (out_nll && !aligned(out_nll, 8)))
        return SV_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, kAlign)) return SV_ERR_INVALID_ARGUMENT;
    if (*workspace_bytes < p.bytes) return SV_ERR_WORKSPACE_TOO_SMALL;

    const float c = scale_of(temperature);
    return by_dtype(shape->dtype, [&](auto dt) {
        return run_likelihood<decltype(dt)::value>(shape, p, target_logits, draft_logits, tokens, c, out_terms,
                                                   out_beta, out_nll, workspace, stream, prof);
    });
}

// ---- scratch of the allocation-free entry point
//
// One device array per GPU, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (in host code the name is a host-side
// stand-in, not a device address): the device address is taken once per
// device with hipGetSymbolAddress, with that device current, and kept here.
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's address of `scratch` (nullptr on a HIP error).
void* scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

sv_status_t spec_verify_sample(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                               const int32_t* draft_ids, float temperature, int32_t top_k, float top_p, uint64_t seed,
                               uint32_t offset, int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                               float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                               hipStream_t stream)
{
    return verify_sample_common(shape, target_logits, draft_logits, draft_ids, temperature, top_k, top_p, seed, offset,
                                out_tokens, out_num_accepted, out_probs, out_residual_mass, workspace,
                                workspace_bytes, stream, 0, nullptr);
}

sv_status_t spec_verify_sample_noalloc(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                                       const int32_t* draft_ids, float temperature, int32_t top_k, float top_p,
                                       uint64_t seed, uint32_t offset, int32_t* out_tokens, int32_t* out_num_accepted,
                                       float* out_probs, float* out_residual_mass, hipStream_t stream)
{
    // every argument check, then the plan's size: nothing touches the device before they pass
    Plan p;
    sv_status_t st = sample_plan(shape, temperature, top_k, top_p, &p);
    if (st != SV_OK) return st;
    st = sample_pointers(shape, target_logits, draft_logits, draft_ids, out_tokens, out_num_accepted, out_probs,
                         out_residual_mass);
    if (st != SV_OK) return st;
    if (p.bytes > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_WORKSPACE_TOO_SMALL;
    void* ws = scratch_for_current_device();
    if (ws == nullptr) return SV_ERR_HIP;
    return launch_sample(shape, p, target_logits, draft_logits, draft_ids, temperature, seed, offset, out_tokens,
                         out_num_accepted, out_probs, out_residual_mass, ws, stream, 0, nullptr);
}

sv_status_t spec_verify_argmax(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                               const int32_t* draft_ids, float temperature, int32_t top_k, float top_p, uint64_t seed,
                               uint32_t offset, int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                               float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                               hipStream_t stream)
{
    return verify_sample_common(shape, target_logits, draft_logits, draft_ids, temperature, top_k, top_p, seed, offset,
                                out_tokens, out_num_accepted, out_probs, out_residual_mass, workspace,
                                workspace_bytes, stream, 1, nullptr);
}

sv_status_t spec_verify_greedy(const sv_shape_t* shape, const void* target_logits, const int32_t* draft_ids,
                               int32_t* out_tokens, int32_t* out_num_accepted, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream)
{
    return verify_greedy_common(shape, target_logits, draft_ids, out_tokens, out_num_accepted, workspace,
                                workspace_bytes, stream, nullptr);
}

sv_status_t spec_draft_sample(const sv_shape_t* shape, const void* draft_logits, float temperature, int32_t top_k,
                              float top_p, uint64_t seed, uint32_t offset, int32_t* out_ids, void* workspace,
                              size_t* workspace_bytes, hipStream_t stream)
{
    return draft_sample_common(shape, draft_logits, temperature, top_k, top_p, seed, offset, out_ids, workspace,
                               workspace_bytes, stream, nullptr);
}

sv_status_t spec_token_likelihood(const sv_shape_t* shape, const void* target_logits, const void* draft_logits,
                                  const int32_t* tokens, float temperature, int32_t top_k, float top_p,
                                  float* out_terms, float* out_beta, double* out_nll, void* workspace,
                                  size_t* workspace_bytes, hipStream_t stream)
{
    return token_likelihood_common(shape, target_logits, draft_logits, tokens, temperature, top_k, top_p, out_terms,
                                   out_beta, out_nll, workspace, workspace_bytes, stream, nullptr);
}

const char* spec_verify_status_string(sv_status_t status)
{
    switch (status) {
        case SV_OK: return "SV_OK";
        case SV_ERR_INVALID_ARGUMENT: return "SV_ERR_INVALID_ARGUMENT";
        case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
        case SV_ERR_WORKSPACE_TOO_SMALL: return "SV_ERR_WORKSPACE_TOO_SMALL";
        case SV_ERR_HIP: return "SV_ERR_HIP";
    }
    return "SV_ERR_UNKNOWN";
}

// ---- benchmark entry points (specverify_profile.h): the same calls with
// the caller's events recorded around the streaming pass

sv_status_t spec_verify_sample_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                        const void* target_logits, const void* draft_logits, const int32_t* draft_ids,
                                        float temperature, int32_t top_k, float top_p, uint64_t seed, uint32_t offset,
                                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                        float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                                        hipStream_t stream)
{
    return verify_sample_common(shape, target_logits, draft_logits, draft_ids, temperature, top_k, top_p, seed, offset,
                                out_tokens, out_num_accepted, out_probs, out_residual_mass, workspace,
                                workspace_bytes, stream, 0, events);
}

sv_status_t spec_verify_argmax_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                        const void* target_logits, const void* draft_logits, const int32_t* draft_ids,
                                        float temperature, int32_t top_k, float top_p, uint64_t seed, uint32_t offset,
                                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                        float* out_residual_mass, void* workspace, size_t* workspace_bytes,
                                        hipStream_t stream)
{
    return verify_sample_common(shape, target_logits, draft_logits, draft_ids, temperature, top_k, top_p, seed, offset,
                                out_tokens, out_num_accepted, out_probs, out_residual_mass, workspace,
                                workspace_bytes, stream, 1, events);
}

sv_status_t spec_verify_greedy_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                        const void* target_logits, const int32_t* draft_ids, int32_t* out_tokens,
                                        int32_t* out_num_accepted, void* workspace, size_t* workspace_bytes,
                                        hipStream_t stream)
{
    return verify_greedy_common(shape, target_logits, draft_ids, out_tokens, out_num_accepted, workspace,
                                workspace_bytes, stream, events);
}

sv_status_t spec_draft_sample_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                       const void* draft_logits, float temperature, int32_t top_k, float top_p,
                                       uint64_t seed, uint32_t offset, int32_t* out_ids, void* workspace,
                                       size_t* workspace_bytes, hipStream_t stream)
{
    return draft_sample_common(shape, draft_logits, temperature, top_k, top_p, seed, offset, out_ids, workspace,
                               workspace_bytes, stream, events);
}

sv_status_t spec_token_likelihood_profiled(const sv_profile_events_t* events, const sv_shape_t* shape,
                                           const void* target_logits, const void* draft_logits, const int32_t* tokens,
                                           float temperature, int32_t top_k, float top_p, float* out_terms,
                                           float* out_beta, double* out_nll, void* workspace, size_t* workspace_bytes,
                                           hipStream_t stream)
{
    return token_likelihood_common(shape, target_logits, draft_logits, tokens, temperature, top_k, top_p, out_terms,
                                   out_beta, out_nll, workspace, workspace_bytes, stream, events);
}

sv_status_t spec_profile_stream_read(const sv_profile_events_t* events, const void* data, size_t bytes, uint32_t* sink,
                                     hipStream_t stream)
{
    if (data == nullptr || sink == nullptr || !aligned(data, 16) || !aligned(sink, 4) || bytes == 0 || bytes % 16 != 0)
        return SV_ERR_INVALID_ARGUMENT;
    const int64_t nblk = (int64_t)(bytes / 16);
    const int64_t per = (int64_t)sv::kThreads * kCandLoads;
    const int64_t grid = (nblk + per - 1) / per;
    if (grid > INT32_MAX) return SV_ERR_UNSUPPORTED;
    launch_stream(events, sv::stream_read_kernel<kCandLoads>, (uint32_t)grid, stream,
                  static_cast<const sv::u32x4*>(data), nblk, (uint32_t)0x9E3779B9u, sink);
    return launch_status();
}

}  // extern "C"
