// Accept / first rejection / residual or extra-token draw, one workgroup per
// sequence.  Follows the acceptance rule, residual and proof of
// "CS3602_FINAL_SpeDec" (section 2: accept x ~ q with min(1, p(x)/q(x)), on
// rejection draw from norm(max(0, p - q)) whose normaliser is 1 - beta) and
// the loop shape of "Text Generation via Speculative Sampling, KV Caching,
// and OpenVINO" ("Prepare speculative sampling", steps 3 and 4: one uniform
// per guess, stop at the first rejection, one extra token from the last
// target position when every guess is accepted).
//
// Phases (one workgroup per sequence b: 1024 threads when the draws walk full
// rows, so that enough loads are in flight for the residual's two-row
// re-read; 256 when they walk top-k kept lists):
//  A  per-row statistics of the sequence's K_b+1 target and K_b draft rows,
//     merged from the streaming pass's chunk partials (m, S) or read from the
//     top-k select pass's row descriptors;
//  B  every guess at once: p_k(x_k), q_k(x_k) in fp64 from the gathered
//     logits, u_k = U(b, k, 0), accept iff u_k < min(1, p/q); n = the first
//     rejected position (LDS atomic min) or K_b;
//  C  one inverse-CDF draw in ascending id order: the residual
//     max(0, p_n - q_n) with U(b, n, 1), or p_{K_b} with U(b, K_b, 2).  Over a
//     full row it runs as 512-id segments (fp32 weights, fp64 sums, one
//     wave-scan per segment), a workgroup scan of the segment sums, and a
//     re-walk of the one segment that holds the crossing.  Over a top-k kept
//     list (at most 1024 ids, sorted by id) one wave does it in registers;
//  D  tokens, accepted count, residual mass.
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr int kMaxDraft = 128;       // largest K (rows per sequence 2K+1)
constexpr int kSegElems = 8;         // ids per lane per segment
constexpr int kSeg = kWave * kSegElems;   // 512 ids per segment
constexpr int kMaxSeg = (1 << 20) / kSeg;  // vocabularies up to 2^20
constexpr int kSegUnroll = 4;        // segments per wave with loads in flight together
constexpr int kKeepCap = 1024;       // kept-list capacity per row (same as the select passes')

struct VerifyArgs {
    RowSet rs;
    const int32_t* cu;  // device [B+1] or null
    int32_t batch;
    int32_t kmax;
    int32_t total_draft;
    int32_t vocab;
    const int32_t* ids;
    float c;  // log2(e) / T, fp32
    int32_t argmax_draw;  // 1: the new token is the argmax of the residual / of p_K instead of a draw
    uint64_t seed;
    uint32_t offset;
    // statistics source: chunk partials (no top-k) or row descriptors (top-k)
    const PartialFull* partials;
    int32_t nchunk;
    int32_t chunk_blocks;  // aligned 16-byte blocks per chunk of the streaming pass
    const RowDesc* descs;
    const KeptEntry* kept;
    // outputs
    int32_t* out_tokens;
    int32_t* out_nacc;
    float* out_probs;
    float* out_zmass;
};

struct RowLds {
    float tau;
    float mcc;
    float inv_s;   // fl32(1 / S)
    int32_t kept;  // list length, or -1 for a full row
    double s;
};

// The residual weight max(0, p - q) of one id from its two unnormalised
// terms and the rows' fl32(1 / S): both probabilities are rounded to fp32
// before the difference.  Fusing one product into the subtraction would leave
// its rounding error where the two probabilities are equal, and a residual
// that has no mass (p = q on the whole support) would then be drawn from that
// noise instead of being recognised as empty.
__device__ __forceinline__ float resid_weight(float et, float inv_t, float ed, float inv_d)
{
#pragma clang fp contract(off)
    const float pt = et * inv_t;
    const float pd = ed * inv_d;
    return fmaxf(pt - pd, 0.0f);
}

// Weights of the inverse-CDF draw, in probability units (fp32).
struct ResidualW {
    float tau_t, mcc_t, inv_t, tau_d, mcc_d, inv_d, c;
    __device__ __forceinline__ float operator()(float lt, float ld) const
    {
        const float et = lt >= tau_t ? __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t)) : 0.0f;
        const float ed = ld >= tau_d ? __builtin_amdgcn_exp2f(__builtin_fmaf(ld, c, -mcc_d)) : 0.0f;
        return resid_weight(et, inv_t, ed, inv_d);
    }
};
// The same weights for rows with no top-k threshold (tau = -inf): a -inf
// logit already gives exp2(-inf) = 0, so the threshold test is dropped.
struct ResidualWFull {
    float tau_t, mcc_t, inv_t, tau_d, mcc_d, inv_d, c;
    __device__ __forceinline__ float operator()(float lt, float ld) const
    {
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t));
        const float ed = __builtin_amdgcn_exp2f(__builtin_fmaf(ld, c, -mcc_d));
        return resid_weight(et, inv_t, ed, inv_d);
    }
};
struct BonusW {
    float tau_t, mcc_t, inv_t, c;
    __device__ __forceinline__ float operator()(float lt, float) const
    {
        return lt >= tau_t ? __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t)) * inv_t : 0.0f;
    }
};
// BonusW for rows with no top-k threshold (tau = -inf; see ResidualWFull).
struct BonusWFull {
    float tau_t, mcc_t, inv_t, c;
    __device__ __forceinline__ float operator()(float lt, float) const
    {
        return __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t)) * inv_t;
    }
};

// Weights of one lane's kSegElems ids of segment s (0 outside the row).
template <int DT, bool TWO, class W>
__device__ __forceinline__ void seg_weights(const char* ra, const char* rb, int32_t vocab, bool vec,
                                            int32_t s, const W& wfn, float* w)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int NV = kSegElems / VEC;  // 16-byte loads per lane per row
    const int32_t v0 = s * kSeg + lane_id() * kSegElems;
    if (vec && v0 + kSegElems <= vocab) {
        const u32x4* pa = reinterpret_cast<const u32x4*>(ra) + v0 / VEC;
        const u32x4* pb = reinterpret_cast<const u32x4*>(rb) + v0 / VEC;
        u32x4 wa[NV], wb[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            wa[q] = load16<false>(pa + q);
            if constexpr (TWO) wb[q] = load16<false>(pb + q);
        }
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            float fa[VEC], fb[VEC];
            unpack<DT>(wa[q], fa);
            if constexpr (TWO) unpack<DT>(wb[q], fb);
#pragma unroll
            for (int e = 0; e < VEC; ++e) w[q * VEC + e] = wfn(fa[e], TWO ? fb[e] : 0.0f);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kSegElems; ++e) {
            const int32_t v = v0 + e;
            w[e] = (v < vocab) ? wfn(load_one<DT>(ra, v), TWO ? load_one<DT>(rb, v) : 0.0f) : 0.0f;
        }
    }
}

// Pass 1 of the inverse CDF over a full row (or row pair): the sums of the
// weights of segments [s_begin, s_end), each handed to put(s, sum).  A lane
// sums its kSegElems weights in fp32, then a wave scan carries them in fp64;
// the order is fixed, so a segment's sum is the same whichever workgroup
// computes it.
template <int DT, bool TWO, int NT, class W, class Put>
__device__ __forceinline__ void cdf_segment_sums(const char* ra, const char* rb, int32_t vocab, bool vec,
                                                 const W& wfn, int32_t s_begin, int32_t s_end, Put&& put)
{
    const int lane = lane_id();
    for (int32_t s0 = s_begin + wave_id(); s0 < s_end; s0 += (NT / kWave) * kSegUnroll) {
        float w[kSegUnroll][kSegElems];
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu) {
            const int32_t s = s0 + uu * (NT / kWave);
            if (s < s_end) seg_weights<DT, TWO>(ra, rb, vocab, vec, s, wfn, w[uu]);
        }
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu) {
            const int32_t s = s0 + uu * (NT / kWave);
            if (s < s_end) {
                float fs = 0.0f;
#pragma unroll
                for (int e = 0; e < kSegElems; ++e) fs += w[uu][e];
                const double incl = wave_incl_scan_dpp((double)fs);
                if (lane == kWave - 1) put(s, incl);
            }
        }
    }
}

// The rest of the inverse CDF, with every segment sum in s_seg[0 .. nseg):
// a workgroup scan of them (in place), the first segment whose running mass
// exceeds u times the total, and a re-walk of that segment by wave 0.  All
// threads call it; all get the token and the total.
template <int DT, bool TWO, int NT, class W>
__device__ void cdf_finish(const char* ra, const char* rb, int32_t vocab, bool vec, const W& wfn, double u,
                           int32_t nseg, double* s_seg, double* s_wd, int32_t* s_i, double* s_dd, int32_t* token,
                           double* total)
{
    const int lane = lane_id();
    // workgroup inclusive scan of the segment sums, in place
    const int32_t per = (nseg + NT - 1) / NT;
    const int32_t lo = min(nseg, (int32_t)threadIdx.x * per), hi = min(nseg, lo + per);
    double run = 0.0;
    for (int32_t s = lo; s < hi; ++s) {
        run += s_seg[s];
        s_seg[s] = run;
    }
    const double tincl = wave_incl_scan_dpp(run);
    const double texcl = wave_prev_dpp(tincl);
    if (lane == kWave - 1) s_wd[wave_id()] = tincl;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave_id(); ++w) off += s_wd[w];
    off += texcl;
    for (int32_t s = lo; s < hi; ++s) s_seg[s] += off;
    if (threadIdx.x == 0) s_i[0] = nseg;
    __syncthreads();
    const double z = s_seg[nseg - 1];
    const double t = u * z;
    for (int32_t s = lo; s < hi; ++s) {
        if (s_seg[s] > t) {
            atomicMin(&s_i[0], s);
            break;
        }
    }
    __syncthreads();

    // pass 2: re-walk the segment holding the crossing (wave 0)
    if (wave_id() == 0) {
        int32_t s = s_i[0];
        if (s >= nseg) s = nseg - 1;
        int32_t tok = -1;
        for (; s >= 0 && tok < 0; --s) {
            float w[kSegElems];
            seg_weights<DT, TWO>(ra, rb, vocab, vec, s, wfn, w);
            float fs = 0.0f;
#pragma unroll
            for (int e = 0; e < kSegElems; ++e) fs += w[e];
            const double incl = wave_incl_scan_dpp((double)fs);
            const double excl = wave_prev_dpp(incl);
            const double start = (s > 0 ? s_seg[s - 1] : 0.0) + excl;
            // the running mass inside the lane in the same fp32 order as pass 1,
            // so that a lane ends exactly where the next one starts
            float run = 0.0f;
            int hit = -1, lastpos = -1;
#pragma unroll
            for (int e = 0; e < kSegElems; ++e) {
                run += w[e];
                if (hit < 0 && start + (double)run > t) hit = e;
                if (w[e] > 0.0f) lastpos = e;
            }
            const uint64_t bh = __ballot(hit >= 0);
            if (bh != 0) {
                const int src = __builtin_ctzll(bh);
                tok = s * kSeg + src * kSegElems + __builtin_amdgcn_readlane(hit, src);
            } else {
                // rounding put the target past this segment's walk: its last positive id
                const uint64_t bp = __ballot(lastpos >= 0);
                if (bp != 0) {
                    const int src = 63 - __builtin_clzll(bp);
                    tok = s * kSeg + src * kSegElems + __builtin_amdgcn_readlane(lastpos, src);
                }
            }
        }
        if (lane == 0) {
            s_i[1] = tok;
            s_dd[0] = z;
        }
    }
    __syncthreads();
    *token = s_i[1];
    *total = s_dd[0];
    __syncthreads();
}

// Inverse CDF over a full row (or row pair) by one workgroup.  All threads
// call it; all get the token and the total.
template <int DT, bool TWO, int NT, class W>
__device__ void inverse_cdf_full(const char* ra, const char* rb, int32_t vocab, const W& wfn, double u,
                                 double* s_seg, double* s_wd, int32_t* s_i, double* s_dd,
                                 int32_t* token, double* total)
{
    const int32_t nseg = (vocab + kSeg - 1) / kSeg;
    const bool vec = ((uintptr_t)ra & 15u) == 0 && (!TWO || ((uintptr_t)rb & 15u) == 0);
    cdf_segment_sums<DT, TWO, NT>(ra, rb, vocab, vec, wfn, 0, nseg, [&](int32_t s, double v) { s_seg[s] = v; });
    __syncthreads();
    cdf_finish<DT, TWO, NT>(ra, rb, vocab, vec, wfn, u, nseg, s_seg, s_wd, s_i, s_dd, token, total);
}

// Inverse CDF over a kept list (ascending ids), one wave.  entry(i) yields the
// list's i-th (id, logit); draft(i, id) the draft logit at that id (RESID only).
template <bool RESID, class Entry, class Draft>
__device__ void inverse_cdf_list_of(Entry&& entry, int32_t n, Draft&& draft, const ResidualW& rw, double u,
                                    int32_t* token, double* total)
{
    constexpr int PER = kKeepCap / kWave;  // entries per lane
    const int lane = lane_id();
    const int32_t per = (n + kWave - 1) / kWave;
    const int32_t lo = min(n, lane * per), hi = min(n, lo + per);
    float w[PER];
    int32_t ix[PER];
    double ls = 0.0;
    // slots q >= per are empty in every lane: both loops stop there (per is
    // uniform), which leaves every sum and every pick as it was
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q >= per) break;
        const int32_t i = lo + q;
        w[q] = 0.0f;
        ix[q] = -1;
        if (i < hi) {
            const KeptEntry e = entry(i);
            ix[q] = e.idx;
            const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(e.val, rw.c, -rw.mcc_t));
            if constexpr (RESID) {
                const float ld = draft(i, e.idx);
                const float ed = ld >= rw.tau_d ? __builtin_amdgcn_exp2f(__builtin_fmaf(ld, rw.c, -rw.mcc_d)) : 0.0f;
                w[q] = resid_weight(et, rw.inv_t, ed, rw.inv_d);
            } else {
                w[q] = et * rw.inv_t;
            }
            ls += (double)w[q];
        }
    }
    const double incl = wave_incl_scan_dpp(ls);
    const double excl = wave_prev_dpp(incl);
    const double z = readlane_f64(incl, kWave - 1);
    const double t = u * z;
    double cum = excl;
    int hit = -1, lastpos = -1;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q >= per) break;
        cum += (double)w[q];
        if (hit < 0 && ix[q] >= 0 && cum > t) hit = ix[q];
        if (w[q] > 0.0f) lastpos = ix[q];
    }
    int32_t tok = -1;
    const uint64_t bh = __ballot(hit >= 0);
    if (bh != 0) {
        tok = __builtin_amdgcn_readlane(hit, __builtin_ctzll(bh));
    } else {
        const uint64_t bp = __ballot(lastpos >= 0);
        if (bp != 0) tok = __builtin_amdgcn_readlane(lastpos, 63 - __builtin_clzll(bp));
    }
    *token = tok;
    *total = z;
}

// The same over a kept list in global memory, the draft logits gathered from
// the draft row.
template <int DT, bool RESID>
__device__ void inverse_cdf_list(const KeptEntry* list, int32_t n, const char* drow, const ResidualW& rw,
                                 double u, int32_t* token, double* total)
{
    inverse_cdf_list_of<RESID>([&](int32_t i) { return list[i]; }, n,
                               [&](int32_t, int32_t v) { return load_one<DT>(drow, v); }, rw, u, token, total);
}

// LDS of the one-draw phase.
template <int NT>
struct DrawLds {
    double seg[kMaxSeg];
    double wd[NT / kWave];
    double dd[2];
    int32_t i[4];
    float bv[NT / kWave];
    int32_t bi[NT / kWave];
};

// Argmax of the weights over a kept list (one wave; entry / draft as in
// inverse_cdf_list_of): the lowest id among the largest positive weights, or
// -1 when no weight is positive; total = their fp64 sum.
template <bool RESID, class Entry, class Draft>
__device__ void argmax_list_of(Entry&& entry, int32_t n, Draft&& draft, const ResidualW& rw, int32_t* token,
                               double* total)
{
    constexpr int PER = kKeepCap / kWave;  // entries per lane
    const int32_t per = (n + kWave - 1) / kWave;
    const int32_t lo = min(n, lane_id() * per), hi = min(n, lo + per);
    float best = 0.0f;
    int32_t bid = INT32_MAX;
    double ls = 0.0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q >= per) break;  // uniform: empty in every lane from here on
        const int32_t i = lo + q;
        if (i >= hi) continue;
        const KeptEntry e = entry(i);
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(e.val, rw.c, -rw.mcc_t));
        float w = et * rw.inv_t;
        if constexpr (RESID) {
            const float ld = draft(i, e.idx);
            const float ed = ld >= rw.tau_d ? __builtin_amdgcn_exp2f(__builtin_fmaf(ld, rw.c, -rw.mcc_d)) : 0.0f;
            w = resid_weight(et, rw.inv_t, ed, rw.inv_d);
        }
        ls += (double)w;
        if (w > 0.0f) argmax_merge(best, bid, w, e.idx);
    }
    wave_argmax(best, bid);
    *token = bid == INT32_MAX ? -1 : __builtin_amdgcn_readlane(bid, 0);
    *total = wave_sum_dpp(ls);
}

// Argmax of the weights over a full row (or row pair), all threads: the
// lowest id among the largest positive weights, or -1; total = their sum.
template <int DT, bool TWO, int NT, class W>
__device__ void argmax_full(const char* ra, const char* rb, int32_t vocab, const W& wfn, DrawLds<NT>& L,
                            int32_t* token, double* total)
{
    constexpr int NW = NT / kWave;
    const int32_t nseg = (vocab + kSeg - 1) / kSeg;
    const bool vec = ((uintptr_t)ra & 15u) == 0 && (!TWO || ((uintptr_t)rb & 15u) == 0);
    float best = 0.0f;
    int32_t bid = INT32_MAX;
    double ls = 0.0;
    for (int32_t s0 = wave_id(); s0 < nseg; s0 += NW * kSegUnroll) {
        float w[kSegUnroll][kSegElems];
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu) {
            const int32_t s = s0 + uu * NW;
            if (s < nseg) seg_weights<DT, TWO>(ra, rb, vocab, vec, s, wfn, w[uu]);
        }
        // a lane meets its ids in ascending order, so a strict > keeps the
        // lowest id among equal weights (and best starting at 0 drops zeros);
        // a lane's kSegElems weights are summed in fp32, then carried in fp64
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu) {
            const int32_t s = s0 + uu * NW;
            if (s < nseg) {
                const int32_t v0 = s * kSeg + lane_id() * kSegElems;
                float fs = 0.0f;
#pragma unroll
                for (int e = 0; e < kSegElems; ++e) {
                    fs += w[uu][e];
                    if (w[uu][e] > best) {
                        best = w[uu][e];
                        bid = v0 + e;
                    }
                }
                ls += (double)fs;
            }
        }
    }
    wave_argmax(best, bid);
    ls = wave_sum_dpp(ls);
    if (lane_id() == 0) {
        L.bv[wave_id()] = best;
        L.bi[wave_id()] = bid;
        L.wd[wave_id()] = ls;
    }
    __syncthreads();
    float v = L.bv[0];
    int32_t ix = L.bi[0];
    double z = L.wd[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        argmax_merge(v, ix, L.bv[w], L.bi[w]);
        z += L.wd[w];
    }
    __syncthreads();
    *token = ix == INT32_MAX ? -1 : ix;
    *total = z;
}

// Inverse CDF of p over a full row that starts at the chunk holding the
// crossing instead of walking the row: the streaming pass's chunk sums,
// rescaled to the row maximum and normalised like the weights
// (W_c = S_c 2^(mcc_c - mcc) fl32(1/S), fp64, ascending chunks), locate the
// first chunk whose running mass exceeds u times their total; only its ids
// are read (up to BPT consecutive blocks per thread), their fp32 weights scanned in fp64
// from the mass before the chunk.  If rounding leaves the crossing past the
// chunk, the walk moves on to the next one; past the last chunk the full
// walk decides.  All threads call it; all get the token.  Each thread takes
// up to BPT consecutive blocks of the chunk (enough for the longest chunk,
// kMaxChunkBlocks, at NT threads).
constexpr int kMaxChunkBlocks = 8 * kThreads;  // 8 loads per thread per streaming tile
// Draft-side draws over full rows walk one chunk each.  With many rows they
// run 512-thread workgroups (four blocks per thread), two per CU, instead of
// one 1024-thread workgroup per CU.
constexpr int kDraftChunkThreads = 512;

// The full-row walk as the rare fallback of the chunk walk below: out of line,
// with the weights taken by value and the token and total returned, so that
// no local of the caller needs an address (one would be kept in scratch memory
// on every path).
struct TokenTotal {
    int32_t token;
    double total;
};
template <int DT, int NT, class W>
__device__ __attribute__((noinline)) TokenTotal cdf_full_fallback(const char* row, int32_t vocab, W wfn, double u,
                                                                   DrawLds<NT>& L)
{
    TokenTotal r;
    inverse_cdf_full<DT, false, NT>(row, nullptr, vocab, wfn, u, L.seg, L.wd, L.i, L.dd, &r.token, &r.total);
    return r;
}

template <int DT, int NT, class W>
__device__ void inverse_cdf_chunks(const char* row, const PartialFull* pp, int32_t nchunk, int32_t chunk_blocks,
                                   int32_t vocab, const W& wfn, double u, DrawLds<NT>& L, int32_t* token,
                                   double* total)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    constexpr int NW = NT / kWave;
    constexpr int BPT = (kMaxChunkBlocks + NT - 1) / NT;
    auto chunk_mass = [&](int32_t ch) {
        double w = 0.0;
        if (ch < nchunk) {
            const PartialFull q = pp[ch];
            if (q.s > 0.0) w = q.s * exp2((double)q.mcc - (double)wfn.mcc_t) * (double)wfn.inv_t;
        }
        return w;
    };
    // the first chunk whose running mass exceeds u * total (wave 0), and the mass before it
    if (wave_id() == 0) {
        double tot = 0.0;
        for (int32_t c0 = 0; c0 < nchunk; c0 += kWave) tot += chunk_mass(c0 + lane_id());
        tot = wave_sum_dpp(tot);
        const double t = u * tot;
        double carry = 0.0;
        int32_t found = -1;
        double before = 0.0;
        for (int32_t c0 = 0; c0 < nchunk && found < 0; c0 += kWave) {
            const int32_t ch = c0 + lane_id();
            const double w = chunk_mass(ch);
            const double incl = carry + wave_incl_scan_dpp(w);
            const uint64_t m = __ballot(ch < nchunk && incl > t);
            if (m != 0) {
                const int src = __builtin_ctzll(m);
                found = c0 + src;
                before = readlane_f64(incl - w, src);
            }
            carry = readlane_f64(incl, kWave - 1);
        }
        if (lane_id() == 0) {
            L.i[0] = found;
            L.dd[0] = before;
            L.dd[1] = tot;
        }
    }
    __syncthreads();
    int32_t ch = L.i[0];
    double before = L.dd[0];
    const double tot = L.dd[1];
    const double t = u * tot;
    __syncthreads();
    const uintptr_t addr = (uintptr_t)row;
    const int32_t mis = (int32_t)((addr & 15u) / ES);
    const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
    const int32_t bpt = (chunk_blocks + NT - 1) / NT;  // blocks per thread
    if (bpt > BPT) {  // chunks longer than BPT blocks per thread: walk the row
        const TokenTotal r = cdf_full_fallback<DT, NT>(row, vocab, wfn, u, L);
        *token = r.token;
        *total = r.total;
        return;
    }
    int32_t tok = -1;
    for (; ch >= 0 && ch < nchunk; ++ch) {
        // this thread's blocks of the chunk, ascending with the thread index.
        // With at most two blocks per thread the weights are held; with more,
        // the raw words are held and the weights formed twice (sum, then walk),
        // which keeps the register count down.
        constexpr bool HOLD_W = BPT <= 2;
        const int32_t j0 = ch * chunk_blocks + (int32_t)threadIdx.x * bpt;
        u32x4 raw[BPT];
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int32_t j = j0 + q;
            const bool in = q < bpt && j < nblk && j < (ch + 1) * chunk_blocks;
            raw[q] = in ? load16<false>(base + j) : u32x4{0u, 0u, 0u, 0u};
        }
        auto weights = [&](int q, float* w) {
            const int32_t j = j0 + q;
            const bool in = q < bpt && j < nblk && j < (ch + 1) * chunk_blocks;
            float f[VEC];
            unpack<DT>(raw[q], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int32_t r = j * VEC - mis + e;
                w[e] = (in && r >= 0 && r < vocab) ? wfn(f[e], 0.0f) : 0.0f;
            }
        };
        // a block's weights are summed in fp32, the blocks carried in fp64
        float held[HOLD_W ? BPT * VEC : 1];
        double ls = 0.0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            float w[VEC];
            weights(q, w);
            float bs = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                bs += w[e];
                if constexpr (HOLD_W) held[q * VEC + e] = w[e];
            }
            ls += (double)bs;
        }
        if constexpr (!HOLD_W) {
            // (an empty asm that claims to update the raw words keeps the
            // compiler from holding the weights across the scan; no instruction)
#pragma unroll
            for (int q = 0; q < BPT; ++q) asm volatile("" : "+v"(raw[q]));
        }
        // exclusive scan of the thread sums in thread order (fp64)
        const double incl = wave_incl_scan_dpp(ls);
        if (lane_id() == kWave - 1) L.wd[wave_id()] = incl;
        if (threadIdx.x == 0) L.i[1] = INT32_MAX;
        __syncthreads();
        double off = before;
        double chunk_sum = 0.0;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            if (wv < wave_id()) off += L.wd[wv];
            chunk_sum += L.wd[wv];
        }
        double cum = off + wave_prev_dpp(incl);
        int32_t hit = INT32_MAX;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            float w[VEC];
            if constexpr (HOLD_W) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) w[e] = held[q * VEC + e];
            } else {
                weights(q, w);
            }
            // the running mass in the same fp32 order as the block sums above
            float run = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                run += w[e];
                const int32_t r = (j0 + q) * VEC - mis + e;
                if (hit == INT32_MAX && w[e] > 0.0f && cum + (double)run > t) hit = r;
            }
            cum += (double)run;
        }
        if (hit != INT32_MAX) atomicMin(&L.i[1], hit);
        __syncthreads();
        tok = L.i[1];
        __syncthreads();
        if (tok != INT32_MAX) break;
        before += chunk_sum;
        tok = -1;
    }
    if (tok < 0 || tok == INT32_MAX) {
        const TokenTotal r = cdf_full_fallback<DT, NT>(row, vocab, wfn, u, L);
        *token = r.token;
        *total = r.total;
        return;
    }
    *token = tok;
    *total = tot;
}

// The argmax of p over a full row: the lowest index of the row maximum, found
// in the first chunk whose partial maximum equals it (logits compare exactly,
// and p is increasing in the logit).  All threads call it.
template <int DT, int NT>
__device__ int32_t argmax_chunks(const char* row, const PartialFull* pp, int32_t nchunk, int32_t chunk_blocks,
                                 int32_t vocab, DrawLds<NT>& L)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    if (wave_id() == 0) {
        float m = neg_inf();
        for (int32_t c0 = lane_id(); c0 < nchunk; c0 += kWave) m = fmaxf(m, pp[c0].m);
        m = wave_max_dpp(m);
        int32_t first = INT32_MAX;
        for (int32_t c0 = lane_id(); c0 < nchunk; c0 += kWave)
            if (pp[c0].m == m) first = min(first, c0);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, kWave));
        if (lane_id() == 0) {
            L.i[0] = first;
            L.bv[0] = m;
            L.i[1] = INT32_MAX;
        }
    }
    __syncthreads();
    const int32_t ch = L.i[0];
    const float m = L.bv[0];
    if (ch != INT32_MAX) {
        const uintptr_t addr = (uintptr_t)row;
        const int32_t mis = (int32_t)((addr & 15u) / ES);
        const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
        const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
        for (int32_t j = ch * chunk_blocks + (int32_t)threadIdx.x; j < min(nblk, (ch + 1) * chunk_blocks); j += NT) {
            float f[VEC];
            unpack<DT>(load16<false>(base + j), f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int32_t r = j * VEC - mis + e;
                if (r >= 0 && r < vocab && f[e] == m) {
                    atomicMin(&L.i[1], r);
                    break;
                }
            }
        }
    }
    __syncthreads();
    const int32_t tok = L.i[1];
    __syncthreads();
    return tok == INT32_MAX ? -1 : tok;
}

// The new token of a sequence (all threads call it; all get the result):
// at the first rejection n < kb the residual max(0, p_n - q_n), else p_kb --
// drawn by the inverse CDF with u (U(b, n, 1), or U(b, kb, 2)), or, with
// a.argmax_draw, its argmax.  rt / rd: statistics of target row n and draft
// row n; kept_row_n: target row n's index in the kept lists.
template <int DT, bool FROM_DESC, int NT>
__device__ __forceinline__ void draw_token(const VerifyArgs& a, int32_t n, int32_t kb, double u, const RowLds& rt,
                                           const RowLds& rd, const char* trow, const char* drow, int64_t kept_row_n,
                                           DrawLds<NT>& L, int32_t* token_out, double* z_out)
{
    const bool list = FROM_DESC && rt.kept >= 0;
    const KeptEntry* kl = a.kept + kept_row_n * kKeepCap;
    auto entry = [&](int32_t i) { return kl[i]; };
    auto dlogit = [&](int32_t, int32_t v) { return load_one<DT>(drow, v); };
    auto none = [](int32_t, int32_t) { return 0.0f; };
    const ResidualW pw{rt.tau, rt.mcc, rt.inv_s, 0.f, 0.f, 0.f, a.c};
    const BonusW bw{rt.tau, rt.mcc, rt.inv_s, a.c};
    // the token of p_n (or p_kb) alone
    auto pick_p = [&](int32_t* tok) {
        double zz;
        if (list) {
            if (wave_id() == 0) {
                int32_t t1;
                if (a.argmax_draw) argmax_list_of<false>(entry, rt.kept, none, pw, &t1, &zz);
                else inverse_cdf_list_of<false>(entry, rt.kept, none, pw, u, &t1, &zz);
                if (lane_id() == 0) L.i[3] = t1;  // not i[2]: it may still be read for the residual's token
            }
            __syncthreads();
            *tok = L.i[3];
        } else if (!FROM_DESC) {
            const PartialFull* pp = a.partials + kept_row_n * a.nchunk;
            const BonusWFull bwf{rt.tau, rt.mcc, rt.inv_s, a.c};
            if (a.argmax_draw) *tok = argmax_chunks<DT, NT>(trow, pp, a.nchunk, a.chunk_blocks, a.vocab, L);
            else inverse_cdf_chunks<DT, NT>(trow, pp, a.nchunk, a.chunk_blocks, a.vocab, bwf, u, L, tok, &zz);
        } else if (a.argmax_draw) {
            argmax_full<DT, false, NT>(trow, nullptr, a.vocab, bw, L, tok, &zz);
        } else {
            inverse_cdf_full<DT, false, NT>(trow, nullptr, a.vocab, bw, u, L.seg, L.wd, L.i, L.dd, tok, &zz);
        }
    };
    int32_t token = -1;
    double z = 0.0;
    if (n < kb) {
        const ResidualW wfn{rt.tau, rt.mcc, rt.inv_s, rd.tau, rd.mcc, rd.inv_s, a.c};
        if (list) {
            if (wave_id() == 0) {
                int32_t t1;
                double z1;
                if (a.argmax_draw) argmax_list_of<true>(entry, rt.kept, dlogit, wfn, &t1, &z1);
                else inverse_cdf_list_of<true>(entry, rt.kept, dlogit, wfn, u, &t1, &z1);
                if (lane_id() == 0) {
                    L.i[2] = t1;
                    L.dd[1] = z1;
                }
            }
            __syncthreads();
            token = L.i[2];
            z = L.dd[1];
        } else if (a.argmax_draw) {
            if constexpr (!FROM_DESC) {
                const ResidualWFull wf{rt.tau, rt.mcc, rt.inv_s, rd.tau, rd.mcc, rd.inv_s, a.c};
                argmax_full<DT, true, NT>(trow, drow, a.vocab, wf, L, &token, &z);
            } else {
                argmax_full<DT, true, NT>(trow, drow, a.vocab, wfn, L, &token, &z);
            }
        } else if constexpr (!FROM_DESC) {
            const ResidualWFull wf{rt.tau, rt.mcc, rt.inv_s, rd.tau, rd.mcc, rd.inv_s, a.c};
            inverse_cdf_full<DT, true, NT>(trow, drow, a.vocab, wf, u, L.seg, L.wd, L.i, L.dd, &token, &z);
        } else {
            inverse_cdf_full<DT, true, NT>(trow, drow, a.vocab, wfn, u, L.seg, L.wd, L.i, L.dd, &token, &z);
        }
        // no positive residual mass (rounding only): p_n with the same uniform, or its argmax
        if (token < 0) pick_p(&token);
    } else {
        pick_p(&token);
    }
    *token_out = token;
    *z_out = z;
}

// LDS of one sequence's verify.
template <int NT>
struct VerifyLds {
    RowLds row[2 * kMaxDraft + 1];
    DrawLds<NT> draw;
    double udraw[kMaxDraft + 1];
    int32_t n, bad, ticket;
};

// The sequence's draft offset k0 and length kb from cu (or the uniform K);
// false when its cu entries are out of range.
__device__ __forceinline__ bool seq_range(const VerifyArgs& a, int32_t b, int32_t* k0, int32_t* kb)
{
    if (a.cu != nullptr) {
        *k0 = a.cu[b];
        const int32_t k1 = a.cu[b + 1];
        *kb = k1 - *k0;
        return !(*k0 < 0 || *kb < 0 || *kb > a.kmax || k1 > a.total_draft);
    }
    *k0 = b * a.kmax;
    *kb = a.kmax;
    return true;
}

// Sequence row r -> global row (target rows k0+b .. k0+b+kb first, then the
// draft rows k0 .. k0+kb-1 after all rows_t target rows).
__device__ __forceinline__ int32_t seq_row(const VerifyArgs& a, int32_t b, int32_t k0, int32_t kb, int32_t r)
{
    return r <= kb ? k0 + b + r : a.rs.rows_t + k0 + (r - kb - 1);
}

// Phases A and B of sequence b's verify, by all NT threads of the workgroup:
// row statistics into S.row, every uniform into S.udraw, and the accept test
// at every guess.  Returns n, the first rejected position (or kb), or -1
// when a guess id is out of range.  p(x), q(x) go to out_probs when
// write_probs.
// Merge one row's chunk partials (m, fl32(m c), S at the chunk max) into the
// row's fl32(m c) and S, by one wave; every lane gets the result.  Rows of at
// most one chunk per lane load their partials once (one memory round instead
// of one for the maximum and one for the sums); the per-lane terms and the
// reduction order are the same either way.
__device__ __forceinline__ PartialFull lane_partial(const PartialFull* pp, int32_t nchunk)
{
    const int l = lane_id();
    return l < nchunk ? pp[l] : PartialFull{neg_inf(), neg_inf(), 0.0};
}
__device__ __forceinline__ void reduce_lane_partials(const PartialFull& q, float c, float* mcc_out, double* s_out)
{
    const float mcc = wave_max_dpp(q.m) * c;
    *mcc_out = mcc;
    *s_out = wave_sum_dpp(q.s > 0.0 ? q.s * exp2((double)q.mcc - (double)mcc) : 0.0);
}
__device__ __forceinline__ void merge_row_partials(const PartialFull* pp, int32_t nchunk, float c, float* mcc_out,
                                                   double* s_out)
{
    const int l = lane_id();
    if (nchunk <= kWave) {
        reduce_lane_partials(lane_partial(pp, nchunk), c, mcc_out, s_out);
        return;
    }
    float m = neg_inf();
    for (int32_t ch = l; ch < nchunk; ch += kWave) m = fmaxf(m, pp[ch].m);
    m = wave_max_dpp(m);
    const float mcc = m * c;
    double s = 0.0;
    for (int32_t ch = l; ch < nchunk; ch += kWave) {
        const PartialFull q = pp[ch];
        if (q.s > 0.0) s += q.s * exp2((double)q.mcc - (double)mcc);
    }
    *mcc_out = mcc;
    *s_out = wave_sum_dpp(s);
}

// The accept test of guess k (id x, logits lt / ld at it, uniform u): accepted
// when u < min(1, p / q) with p(x) and q(x) in fp64.  The same test in fp32
// decides first: with both exponents within 64 of the row maxima, fp32 p and
// q are within 3e-6 of the fp64 ones (the exponent's rounding, 2^-24 of at
// most 64, times ln 2, plus three roundings) and their ratio within 6e-6, so
// a u farther than 2^-12 of the ratio (relative) gets the fp64 test's answer;
// only the rest (about 5e-4 of the draws) take the fp64 test.  p and q are
// reported from whichever precision decided.  A rejection lowers n to k, a
// bad id sets bad.
__device__ __forceinline__ void accept_one(const VerifyArgs& a, int32_t k, int32_t x, float lt, float ld,
                                           const RowLds& rt, const RowLds& rd, double u, int32_t drow0,
                                           bool write_probs, int32_t& n, int32_t& bad)
{
    if (x < 0 || x >= a.vocab) {
        atomicOr(&bad, 1);
        return;
    }
    const bool pin = lt >= rt.tau, qin = ld >= rd.tau;  // kept by the filters
    const float at = __builtin_fmaf(lt, a.c, -rt.mcc), ad = __builtin_fmaf(ld, a.c, -rd.mcc);
    const float p32 = pin ? __builtin_amdgcn_exp2f(at) * rt.inv_s : 0.0f;
    const float q32 = qin ? __builtin_amdgcn_exp2f(ad) * rd.inv_s : 0.0f;
    constexpr float kMargin = 1.0f / 4096.0f;
    const float uf = (float)u;  // exact: u has 24 bits
    int dec = -1;               // 1 accept, 0 reject, -1 undecided
    if (!pin) {
        dec = 0;  // p = 0: the ratio is 0 whatever q is, and u >= 0 never passes
    } else if (qin && fabsf(at) <= 64.0f && fabsf(ad) <= 64.0f) {
        const float r32 = p32 / q32;
        if (r32 >= 1.0f + kMargin || uf < r32 * (1.0f - kMargin)) dec = 1;  // u < 1 <= p / q, or u clearly below
        else if (uf > r32 * (1.0f + kMargin)) dec = 0;
    }
    float pw = p32, qw = q32;
    if (dec < 0) {
        // (q = 0 lands here too: the ratio is then 1 exactly when p > 0 in fp64)
        const double cd = (double)a.c;
        const double p = pin ? exp2((double)lt * cd - (double)rt.mcc) / rt.s : 0.0;
        const double q = qin ? exp2((double)ld * cd - (double)rd.mcc) / rd.s : 0.0;
        const double ratio = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
        dec = u < ratio ? 1 : 0;
        pw = (float)p;
        qw = (float)q;
    }
    if (write_probs && a.out_probs != nullptr) {
        a.out_probs[2 * (int64_t)(drow0 + k)] = pw;
        a.out_probs[2 * (int64_t)(drow0 + k) + 1] = qw;
    }
    if (dec == 0) atomicMin(&n, k);
}

template <int DT, bool FROM_DESC, int NT>
__device__ __forceinline__ int32_t verify_accept(const VerifyArgs& a, int32_t b, int32_t k0, int32_t kb,
                                                 VerifyLds<NT>& S, bool write_probs)
{
    static_assert(NT >= kMaxDraft, "one guess per thread");
    const int32_t trow0 = k0 + b;  // first target row of the sequence
    const int32_t drow0 = k0;      // first draft row
    const int32_t nrows = 2 * kb + 1;
    // with row descriptors (one small load round), thread k's guess is
    // loaded with them, which saves the accept test a dependent round; over
    // full rows it is loaded with the accept test (measured faster there)
    const int32_t xk = FROM_DESC && (int32_t)threadIdx.x < kb ? a.ids[drow0 + threadIdx.x] : 0;

    if (threadIdx.x == 0) {
        S.n = kb;
        S.bad = 0;
    }
    // every uniform the step can use, computed while the first loads are in
    // flight: thread k holds U(b, k, 0); S.udraw[k] = U(b, k, 1),
    // S.udraw[kb] = U(b, kb, 2)
    const int32_t tk = threadIdx.x;
    const double u_acc = uniform24(a.seed, (uint32_t)b, (uint32_t)tk, 0u, a.offset);
    for (int32_t t = tk; t <= kb; t += NT)
        S.udraw[t] = uniform24(a.seed, (uint32_t)b, (uint32_t)t, t < kb ? 1u : 2u, a.offset);

    // ---- A: row statistics
    if constexpr (FROM_DESC) {
        for (int32_t r = threadIdx.x; r < nrows; r += NT) {
            const RowDesc d = a.descs[seq_row(a, b, k0, kb, r)];
            S.row[r] = RowLds{d.tau, d.mcc, (float)(1.0 / d.s), d.kept, d.s};
        }
    } else {
        constexpr int NW = NT / kWave;
        if (a.nchunk <= kWave) {
            // a wave's rows (up to RPW of them) have their partials in flight together
            constexpr int RPW = 4;
            for (int32_t r0 = wave_id(); r0 < nrows; r0 += NW * RPW) {
                PartialFull q[RPW];
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int32_t r = r0 + i * NW;
                    q[i] = r < nrows ? lane_partial(a.partials + (int64_t)seq_row(a, b, k0, kb, r) * a.nchunk, a.nchunk)
                                     : PartialFull{neg_inf(), neg_inf(), 0.0};
                }
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int32_t r = r0 + i * NW;
                    if (r < nrows) {
                        float mcc;
                        double s;
                        reduce_lane_partials(q[i], a.c, &mcc, &s);
                        if (lane_id() == 0) S.row[r] = RowLds{neg_inf(), mcc, (float)(1.0 / s), -1, s};
                    }
                }
            }
        } else {
            for (int32_t r = wave_id(); r < nrows; r += NW) {
                float mcc;
                double s;
                merge_row_partials(a.partials + (int64_t)seq_row(a, b, k0, kb, r) * a.nchunk, a.nchunk, a.c, &mcc,
                                   &s);
                if (lane_id() == 0) S.row[r] = RowLds{neg_inf(), mcc, (float)(1.0 / s), -1, s};
            }
        }
    }
    __syncthreads();

    // ---- B: accept test at every draft position
    const char* tbase = a.rs.tgt;
    const char* dbase = a.rs.drf;
    const int32_t k = threadIdx.x;
    if constexpr (FROM_DESC) {
        if (kb == 0) return S.n;
        // thread k's two logits at its guess; lanes past kb and a bad id load
        // a clamped element that is not used, so that the loads are unconditional
        const int32_t kc = min(k, kb - 1);
        const int32_t xc = min(max(xk, 0), a.vocab - 1);
        const float lt = load_one<DT>(tbase + (int64_t)(trow0 + kc) * a.rs.t_stride_bytes, xc);
        const float ld = load_one<DT>(dbase + (int64_t)(drow0 + kc) * a.rs.d_stride_bytes, xc);
        if (k < kb) accept_one(a, k, xk, lt, ld, S.row[k], S.row[kb + 1 + k], u_acc, drow0, write_probs, S.n, S.bad);
    } else if (k < kb) {
        const int32_t x = a.ids[drow0 + k];
        float lt = 0.0f, ld = 0.0f;
        if (x >= 0 && x < a.vocab) {
            lt = load_one<DT>(tbase + (int64_t)(trow0 + k) * a.rs.t_stride_bytes, x);
            ld = load_one<DT>(dbase + (int64_t)(drow0 + k) * a.rs.d_stride_bytes, x);
        }
        accept_one(a, k, x, lt, ld, S.row[k], S.row[kb + 1 + k], u_acc, drow0, write_probs, S.n, S.bad);
    }
    __syncthreads();
    return S.bad != 0 ? -1 : S.n;
}

// Phase D: tokens x_0 .. x_{n-1}, the new token, then -1; n; the residual mass.
template <int NT>
__device__ __forceinline__ void verify_outputs(const VerifyArgs& a, int32_t b, int32_t k0, int32_t kb, int32_t n,
                                               int32_t token, double z)
{
    const int32_t trow0 = k0 + b;
    for (int32_t j = threadIdx.x; j <= kb; j += NT) {
        a.out_tokens[trow0 + j] = j < n ? a.ids[k0 + j] : (j == n ? token : -1);
    }
    if (threadIdx.x == 0) {
        a.out_nacc[b] = n;
        if (a.out_zmass != nullptr) a.out_zmass[b] = (float)z;
    }
}

// Verify of sequence b by all NT threads of the workgroup.
template <int DT, bool FROM_DESC, int NT>
__device__ __forceinline__ void verify_seq(const VerifyArgs& a, int32_t b, int32_t k0, int32_t kb, VerifyLds<NT>& S)
{
    const int32_t n = verify_accept<DT, FROM_DESC, NT>(a, b, k0, kb, S, true);
    if (n < 0) {
        if (threadIdx.x == 0) a.out_nacc[b] = -1;
        return;
    }
    // ---- C: residual or extra-token draw
    int32_t token;
    double z;
    {
        const RowLds rt = S.row[n];
        const RowLds rd = S.row[n < kb ? kb + 1 + n : n];
        const char* trow = a.rs.tgt + (int64_t)(k0 + b + n) * a.rs.t_stride_bytes;
        const char* drow = n < kb ? a.rs.drf + (int64_t)(k0 + n) * a.rs.d_stride_bytes : nullptr;
        draw_token<DT, FROM_DESC, NT>(a, n, kb, S.udraw[n], rt, rd, trow, drow, (int64_t)seq_row(a, b, k0, kb, n),
                                      S.draw, &token, &z);
    }
    verify_outputs<NT>(a, b, k0, kb, n, token, z);
}

// One workgroup per sequence, after the streaming pass (and the top-k select
// or top-p pass) has finished.
template <int DT, bool FROM_DESC, int NT>
__global__ __launch_bounds__(NT) void verify_kernel(VerifyArgs a)
{
    __shared__ VerifyLds<NT> S;
    const int32_t b = blockIdx.x;
    int32_t k0, kb;
    if (!seq_range(a, b, &k0, &kb)) {
        if (threadIdx.x == 0) a.out_nacc[b] = -1;
        return;
    }
    verify_seq<DT, FROM_DESC, NT>(a, b, k0, kb, S);
}

// Verify over full rows with the residual draw spread over the G = gridDim.y
// workgroups of a sequence.  Each one repeats phases A and B (small), then
// computes the segment sums of its G-th of the two rows' residual weights
// max(0, p_n - q_n) and publishes them (agent-scope stores); the workgroup
// that takes the sequence's last ticket scans all of them and re-walks the
// one segment that holds the crossing.  The draw is the one-workgroup
// draw's, segment for segment.  Sequences that accept every guess draw the
// extra token from the streaming pass's chunk sums in workgroup 0 alone.
struct SplitArgs {
    VerifyArgs va;
    double* segsum;    // [B][nseg] residual segment sums
    int32_t* tickets;  // [B * kTicketStride], zero at launch (the streaming pass clears them)
};

template <int DT, int NT>
__global__ __launch_bounds__(NT) void verify_split_kernel(SplitArgs sa)
{
    __shared__ VerifyLds<NT> S;
    const VerifyArgs& a = sa.va;
    const int32_t b = blockIdx.x;
    const int32_t g = blockIdx.y;
    const int32_t G = gridDim.y;
    int32_t k0, kb;
    if (!seq_range(a, b, &k0, &kb)) {
        if (g == 0 && threadIdx.x == 0) a.out_nacc[b] = -1;
        return;
    }
    const int32_t n = verify_accept<DT, false, NT>(a, b, k0, kb, S, g == 0);
    if (n < 0) {
        if (g == 0 && threadIdx.x == 0) a.out_nacc[b] = -1;
        return;
    }
    const RowLds rt = S.row[n];
    const char* trow = a.rs.tgt + (int64_t)(k0 + b + n) * a.rs.t_stride_bytes;
    const PartialFull* pp = a.partials + (int64_t)seq_row(a, b, k0, kb, n) * a.nchunk;
    const BonusWFull bwf{rt.tau, rt.mcc, rt.inv_s, a.c};
    int32_t token = -1;
    double z = 0.0;
    if (n == kb) {  // every guess accepted: the extra token from p_kb
        if (g != 0) return;
        inverse_cdf_chunks<DT, NT>(trow, pp, a.nchunk, a.chunk_blocks, a.vocab, bwf, S.udraw[n], S.draw, &token, &z);
        verify_outputs<NT>(a, b, k0, kb, n, token, 0.0);
        return;
    }
    const RowLds rd = S.row[kb + 1 + n];
    const char* drow = a.rs.drf + (int64_t)(k0 + n) * a.rs.d_stride_bytes;
    const ResidualWFull wf{rt.tau, rt.mcc, rt.inv_s, rd.tau, rd.mcc, rd.inv_s, a.c};
    const int32_t nseg = (a.vocab + kSeg - 1) / kSeg;
    const bool vec = ((uintptr_t)trow & 15u) == 0 && ((uintptr_t)drow & 15u) == 0;
    double* ss = sa.segsum + (int64_t)b * nseg;
    const int32_t s_lo = (int32_t)((int64_t)nseg * g / G), s_hi = (int32_t)((int64_t)nseg * (g + 1) / G);
    cdf_segment_sums<DT, true, NT>(trow, drow, a.vocab, vec, wf, s_lo, s_hi,
                                   [&](int32_t s, double v) { st_agent_f64(ss + s, v); });
    // publish, then take the sequence's ticket
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) S.ticket = ticket_agent(sa.tickets + (int64_t)b * kTicketStride);
    __syncthreads();
    if (S.ticket != G - 1) return;
    // the last workgroup: every segment sum, then the scan and the re-walk
    for (int32_t s = threadIdx.x; s < nseg; s += NT) S.draw.seg[s] = ld_agent_f64(ss + s);
    __syncthreads();
    cdf_finish<DT, true, NT>(trow, drow, a.vocab, vec, wf, S.udraw[n], nseg, S.draw.seg, S.draw.wd, S.draw.i,
                             S.draw.dd, &token, &z);
    // no positive residual mass (rounding only): p_n with the same uniform
    if (token < 0) {
        double zz;
        inverse_cdf_chunks<DT, NT>(trow, pp, a.nchunk, a.chunk_blocks, a.vocab, bwf, S.udraw[n], S.draw, &token, &zz);
    }
    verify_outputs<NT>(a, b, k0, kb, n, token, z);
}

// ---------------------------------------------------------------------------
// Draft-side sampling, the step before verify: x(b, k) ~ q_k, the
// inverse-CDF draw (ascending ids) with U(b, k, 3) ("Text Generation via
// Speculative Sampling, KV Caching, and OpenVINO", "Prepare speculative
// sampling", step 1, sampling in place of its argmax).  One workgroup per
// (sequence b, position k): blockIdx.x = b, blockIdx.y = k.  The rows of
// a.rs are the draft rows (rows_t = total_draft), their statistics come from
// the same streaming passes as the verify's, and the draw is the verify's
// extra-token draw: over the kept list after a top-k select, over the full
// row (16 waves keep its re-read in flight) otherwise.
// ---------------------------------------------------------------------------
template <int DT, bool FROM_DESC, int NT>
__global__ __launch_bounds__(NT, NT == kDraftChunkThreads ? 4 : 1) void draft_draw_kernel(VerifyArgs a)
{
    __shared__ DrawLds<NT> s_draw;
    __shared__ RowLds s_r;
    __shared__ int32_t s_tok;
    const int32_t b = blockIdx.x;
    const int32_t k = blockIdx.y;
    int32_t k0, kb;
    if (a.cu != nullptr) {
        k0 = a.cu[b];
        const int32_t k1 = a.cu[b + 1];
        kb = k1 - k0;
        if (k0 < 0 || kb < 0 || kb > a.kmax || k1 > a.total_draft) return;  // slots left untouched
    } else {
        k0 = b * a.kmax;
        kb = a.kmax;
    }
    if (k >= kb) return;
    const int32_t row = k0 + k;
    const double u = uniform24(a.seed, (uint32_t)b, (uint32_t)k, 3u, a.offset);

    if constexpr (FROM_DESC) {
        if (threadIdx.x == 0) {
            const RowDesc d = a.descs[row];
            s_r = RowLds{d.tau, d.mcc, (float)(1.0 / d.s), d.kept, d.s};
        }
    } else {
        if (wave_id() == 0) {
            float mcc;
            double s;
            merge_row_partials(a.partials + (int64_t)row * a.nchunk, a.nchunk, a.c, &mcc, &s);
            if (lane_id() == 0) s_r = RowLds{neg_inf(), mcc, (float)(1.0 / s), -1, s};
        }
    }
    __syncthreads();
    const RowLds rt = s_r;
    int32_t token;
    double z;
    if (FROM_DESC && rt.kept >= 0) {
        if (wave_id() == 0) {
            const KeptEntry* kl = a.kept + (int64_t)row * kKeepCap;
            const ResidualW lw{rt.tau, rt.mcc, rt.inv_s, 0.f, 0.f, 0.f, a.c};
            int32_t tok;
            inverse_cdf_list_of<false>([&](int32_t i) { return kl[i]; }, rt.kept,
                                       [](int32_t, int32_t) { return 0.0f; }, lw, u, &tok, &z);
            if (lane_id() == 0) s_tok = tok;
        }
        __syncthreads();
        token = s_tok;
    } else if (!FROM_DESC) {
        const BonusWFull bw{rt.tau, rt.mcc, rt.inv_s, a.c};
        inverse_cdf_chunks<DT, NT>(row_ptr(a.rs, row), a.partials + (int64_t)row * a.nchunk, a.nchunk,
                                   a.chunk_blocks, a.vocab, bw, u, s_draw, &token, &z);
    } else {
        const BonusW bw{rt.tau, rt.mcc, rt.inv_s, a.c};
        inverse_cdf_full<DT, false, NT>(row_ptr(a.rs, row), nullptr, a.vocab, bw, u, s_draw.seg, s_draw.wd, s_draw.i,
                                         s_draw.dd, &token, &z);
    }
    if (threadIdx.x == 0) a.out_tokens[row] = token;
}

// ---------------------------------------------------------------------------
// Greedy argmax-compare: one wave per sequence merges the argmax partials of
// its K_b + 1 target rows and compares them with the guesses.
// ---------------------------------------------------------------------------
struct GreedyArgs {
    const int32_t* cu;
    int32_t batch;
    int32_t kmax;
    int32_t total_draft;
    int32_t vocab;
    const int32_t* ids;
    const PartialArg* partials;
    int32_t nchunk;
    int32_t* out_tokens;
    int32_t* out_nacc;
};

__global__ __launch_bounds__(kThreads) void greedy_kernel(GreedyArgs a)
{
    const int32_t b = blockIdx.x * kWaves + wave_id();
    if (b >= a.batch) return;
    int32_t k0, kb;
    if (a.cu != nullptr) {
        k0 = a.cu[b];
        const int32_t k1 = a.cu[b + 1];
        kb = k1 - k0;
        if (k0 < 0 || kb < 0 || kb > a.kmax || k1 > a.total_draft) {
            if (lane_id() == 0) a.out_nacc[b] = -1;
            return;
        }
    } else {
        k0 = b * a.kmax;
        kb = a.kmax;
    }
    const int32_t trow0 = k0 + b;
    // every guess id is checked first, also those past the first mismatch, as
    // the sampling verify does: a sequence with any id outside [0, V) reports -1
    bool bad_id = false;
    for (int32_t k = lane_id(); k < kb; k += kWave) {
        const int32_t x = a.ids[k0 + k];
        bad_id |= x < 0 || x >= a.vocab;
    }
    if (__ballot(bad_id) != 0) {
        if (lane_id() == 0) a.out_nacc[b] = -1;
        return;
    }
    int32_t n = kb, an = -1;
    for (int32_t k = 0; k <= kb; ++k) {
        const PartialArg* pp = a.partials + (int64_t)(trow0 + k) * a.nchunk;
        float v = neg_inf();
        int32_t ix = INT32_MAX;
        for (int32_t ch = lane_id(); ch < a.nchunk; ch += kWave) argmax_merge(v, ix, pp[ch].m, pp[ch].idx);
        wave_argmax(v, ix);
        ix = __shfl(ix, 0, kWave);
        if (k == kb) {
            an = ix;
            break;
        }
        const int32_t x = a.ids[k0 + k];
        if (x != ix) {
            n = k;
            an = ix;
            break;
        }
    }
    for (int32_t j = lane_id(); j <= kb; j += kWave) {
        a.out_tokens[trow0 + j] = j < n ? a.ids[k0 + j] : (j == n ? an : -1);
    }
    if (lane_id() == 0) a.out_nacc[b] = n;
}

}  // namespace sv
