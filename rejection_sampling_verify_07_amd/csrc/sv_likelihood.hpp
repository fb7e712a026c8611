// Per-token speculative likelihood, the quantity behind the perplexity check
// of "CS3602_FINAL_SpeDec" (section 2's proof; problem analysis, item 1): for
// an observed token y at a position with target distribution p and draft
// distribution q, one speculative step emits y with probability
//   accept part  P(guess accepted, x = y) = q(y) min(1, p(y)/q(y)) = min(p, q)(y)
//   reject part  P(guess rejected, x = y) = (1 - beta) p'(y)      = p(y) - min(p, q)(y)
// whose sum is p(y); beta = sum_v min(p(v), q(v)) is the position's
// acceptance mass.  The parts need only the row statistics and the two
// logits at y; beta needs a second look at every id of both rows.
//
// Position (b, k), k < K_b, is row cu[b] + k of both tensors.  The streaming
// passes see the target rows as rows [0, R) and the draft rows as [R, 2R).
//
// Kernels:
//  pair_min_kernel    full rows, beta requested: one tile of both rows per
//                     workgroup, sum of min(p, q) over the tile (fp32 terms,
//                     fp64 sums), one fp64 partial per (position, tile).
//  likelihood_kernel  one workgroup per sequence, one wave per position:
//                     row statistics, p(y), q(y) in fp64, the two parts,
//                     beta (from the pair partials, or over the top-k kept
//                     list), and the sequence's -sum log P(y).
#pragma once

#include "sv_common.hpp"
#include "sv_stats.hpp"
#include "sv_verify.hpp"

namespace sv {

constexpr int kPairLoads = 4;  // 16-byte loads per thread per row in the pair pass
constexpr int kPairLoadsBig = 8;  // the same over grids many times larger than the chip (measured: 334 against
                                  // 342-346 us for the step on 2048 positions of 128256 bf16 logits; slower on
                                  // small grids, 34.3 against 32.7 us on 256 positions of 50304)

// min(p(v), q(v)) in probability units (fp32), each side masked by its
// top-k threshold.
struct MinW {
    float tau_t, mcc_t, inv_t, tau_d, mcc_d, inv_d, c;
    __device__ __forceinline__ float operator()(float lt, float ld) const
    {
        const float et = lt >= tau_t ? __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t)) * inv_t : 0.0f;
        const float ed = ld >= tau_d ? __builtin_amdgcn_exp2f(__builtin_fmaf(ld, c, -mcc_d)) * inv_d : 0.0f;
        return fminf(et, ed);
    }
};

// MinW for rows with no top-k threshold: a -inf logit (a mask, or an
// out-of-row slot filled with -inf) already weighs exp2(-inf) = 0.
struct MinWFull {
    float mcc_t, inv_t, mcc_d, inv_d, c;
    __device__ __forceinline__ float operator()(float lt, float ld) const
    {
        const float et = __builtin_amdgcn_exp2f(__builtin_fmaf(lt, c, -mcc_t)) * inv_t;
        const float ed = __builtin_amdgcn_exp2f(__builtin_fmaf(ld, c, -mcc_d)) * inv_d;
        return fminf(et, ed);
    }
};

struct PairArgs {
    RowSet rs;          // target rows [0, R), draft rows [R, 2R)
    int32_t vocab;
    int32_t rows;       // R
    const PartialFull* partials;  // the streaming pass's, [2R][nchunk]
    int32_t nchunk;
    int32_t nchunk2;    // tiles per row pair of this pass
    float c;
    double* out;        // [R][nchunk2]
};

template <int DT, int LOADS>
__global__ __launch_bounds__(kThreads) void pair_min_kernel(PairArgs a)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    __shared__ float s_st[4];  // mcc_t, inv_t, mcc_d, inv_d
    __shared__ double s_w[kWaves];

    const int32_t tile = (int32_t)blockIdx.x;
    const int32_t r = (int32_t)((uint32_t)tile / (uint32_t)a.nchunk2);
    const int32_t ch = tile - r * a.nchunk2;
    const uintptr_t at = (uintptr_t)row_ptr(a.rs, r);
    const uintptr_t ad = (uintptr_t)row_ptr(a.rs, a.rows + r);
    const int32_t mis_t = (int32_t)((at & 15u) / ES);
    const int32_t mis_d = (int32_t)((ad & 15u) / ES);
    const int32_t nblk = (mis_t + a.vocab + VEC - 1) / VEC;
    const int32_t b0 = ch * (kThreads * LOADS) + (int32_t)threadIdx.x;
    const bool same = mis_t == mis_d;  // uniform: both rows share the block grid

    // both rows' blocks in flight before the statistics are merged
    u32x4 rt[LOADS], rd[LOADS];
    if (same) {
        const u32x4* bt = reinterpret_cast<const u32x4*>(at - (at & 15u));
        const u32x4* bd = reinterpret_cast<const u32x4*>(ad - (ad & 15u));
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int32_t j = b0 + i * kThreads;
            rt[i] = j < nblk ? load16<true>(bt + j) : u32x4{0u, 0u, 0u, 0u};
            rd[i] = j < nblk ? load16<true>(bd + j) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (wave_id() < 2) {
        const int32_t row = wave_id() == 0 ? r : a.rows + r;
        float mcc;
        double s;
        merge_row_partials(a.partials + (int64_t)row * a.nchunk, a.nchunk, a.c, &mcc, &s);
        if (lane_id() == 0) {
            s_st[2 * wave_id()] = mcc;
            s_st[2 * wave_id() + 1] = (float)(1.0 / s);
        }
    }
    __syncthreads();
    const MinW wfn{neg_inf(), s_st[0], s_st[1], neg_inf(), s_st[2], s_st[3], a.c};

    float acc = 0.0f;
    if (same) {
        // tiles that reach outside the row fill their out-of-row slots with
        // -inf (weight 0), so the element loop needs no threshold or bounds test
        Tile tl;
        tl.index = tile;
        tl.row = r;
        tl.cb0 = ch * (kThreads * LOADS);
        tl.mis = mis_t;
        tl.nblk = nblk;
        sanitize_edge<DT, LOADS>(tl, a.vocab, rt);
        sanitize_edge<DT, LOADS>(tl, a.vocab, rd);
        const MinWFull wf{s_st[0], s_st[1], s_st[2], s_st[3], a.c};
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            float ft[VEC], fd[VEC];
            unpack<DT>(rt[i], ft);
            unpack<DT>(rd[i], fd);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc += wf(ft[e], fd[e]);
        }
    } else {
        // rows on different 16-byte phases: element loads on the target's block grid
        const char* pt = reinterpret_cast<const char*>(at);
        const char* pd = reinterpret_cast<const char*>(ad);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int32_t v0 = (b0 + i * kThreads) * VEC - mis_t;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int32_t v = v0 + e;
                if ((uint32_t)v < (uint32_t)a.vocab) acc += wfn(load_one<DT>(pt, v), load_one<DT>(pd, v));
            }
        }
    }
    const double ws = wave_sum_dpp((double)acc);
    if (lane_id() == 0) s_w[wave_id()] = ws;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += s_w[w];
        a.out[tile] = t;
    }
}

struct LikArgs {
    RowSet rs;          // target rows [0, R), draft rows [R, 2R)
    const int32_t* cu;  // device [B+1] or null
    int32_t batch;
    int32_t kmax;
    int32_t rows;       // R = total positions
    int32_t vocab;
    const int32_t* tokens;
    float c;
    const PartialFull* partials;  // full rows
    int32_t nchunk;
    const RowDesc* descs;         // top-k
    const KeptEntry* kept;
    const double* pair;           // full rows with beta: [R][nchunk2]
    int32_t nchunk2;
    float* out_terms;   // [R][2] or null
    float* out_beta;    // [R] or null
    double* out_nll;    // [B] or null
};

// Sum of min(p, q) over a full row pair by one wave, ids in 512-id segments
// (the top-k path's fallback for rows whose kept set outgrew its list).
template <int DT>
__device__ double wave_pair_min_full(const char* ta, const char* da, int32_t vocab, const MinW& wfn)
{
    const int32_t nseg = (vocab + kSeg - 1) / kSeg;
    const bool vec = (((uintptr_t)ta | (uintptr_t)da) & 15u) == 0;
    double acc = 0.0;
    for (int32_t s0 = 0; s0 < nseg; s0 += kSegUnroll) {
        float w[kSegUnroll][kSegElems];
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu)
            if (s0 + uu < nseg) seg_weights<DT, true>(ta, da, vocab, vec, s0 + uu, wfn, w[uu]);
#pragma unroll
        for (int uu = 0; uu < kSegUnroll; ++uu)
            if (s0 + uu < nseg) {
#pragma unroll
                for (int e = 0; e < kSegElems; ++e) acc += (double)w[uu][e];
            }
    }
    return wave_sum_dpp(acc);
}

template <int DT, bool FROM_DESC>
__global__ __launch_bounds__(kThreads) void likelihood_kernel(LikArgs a)
{
    __shared__ double s_nll[kWaves];
    const int32_t b = blockIdx.x;
    int32_t k0, kb;
    if (a.cu != nullptr) {
        k0 = a.cu[b];
        const int32_t k1 = a.cu[b + 1];
        kb = k1 - k0;
        if (k0 < 0 || kb < 0 || kb > a.kmax || k1 > a.rows) {
            if (threadIdx.x == 0 && a.out_nll != nullptr) a.out_nll[b] = __builtin_nan("");
            return;
        }
    } else {
        k0 = b * a.kmax;
        kb = a.kmax;
    }
    const int lane = lane_id();
    const double cd = (double)a.c;
    double nll = 0.0;  // lane 0's running -sum log P(y) over this wave's positions
    for (int32_t k = wave_id(); k < kb; k += kWaves) {
        const int32_t r = k0 + k;
        const char* trow = row_ptr(a.rs, r);
        const char* drow = row_ptr(a.rs, a.rows + r);
        // row statistics: threshold, fl32(m c), S, kept-list length (-1: full row)
        float tau_t, mcc_t, tau_d, mcc_d;
        double s_t, s_d;
        int32_t kept_t = -1;
        if constexpr (FROM_DESC) {
            const RowDesc dt = a.descs[r];
            const RowDesc dd = a.descs[a.rows + r];
            tau_t = dt.tau;
            mcc_t = dt.mcc;
            s_t = dt.s;
            kept_t = dt.kept;
            tau_d = dd.tau;
            mcc_d = dd.mcc;
            s_d = dd.s;
        } else {
            tau_t = tau_d = neg_inf();
            merge_row_partials(a.partials + (int64_t)r * a.nchunk, a.nchunk, a.c, &mcc_t, &s_t);
            merge_row_partials(a.partials + (int64_t)(a.rows + r) * a.nchunk, a.nchunk, a.c, &mcc_d, &s_d);
        }
        const MinW wfn{tau_t, mcc_t, (float)(1.0 / s_t), tau_d, mcc_d, (float)(1.0 / s_d), a.c};
        const bool bad_rows = !(s_t > 0.0) || !(s_d > 0.0);  // a row with no finite kept logit

        // beta = sum_v min(p(v), q(v))
        double beta = 0.0;
        if (a.out_beta != nullptr) {
            if constexpr (FROM_DESC) {
                if (kept_t >= 0) {
                    // min(p, q) vanishes outside the target's kept set: walk its list
                    const KeptEntry* kl = a.kept + (int64_t)r * kKeepCap;
                    double acc = 0.0;
                    for (int32_t i = lane; i < kept_t; i += kWave) {
                        const KeptEntry e = kl[i];
                        acc += (double)wfn(e.val, load_one<DT>(drow, e.idx));
                    }
                    beta = wave_sum_dpp(acc);
                } else {
                    beta = wave_pair_min_full<DT>(trow, drow, a.vocab, wfn);
                }
            } else {
                double acc = 0.0;
                const double* pp = a.pair + (int64_t)r * a.nchunk2;
                for (int32_t j = lane; j < a.nchunk2; j += kWave) acc += pp[j];
                beta = wave_sum_dpp(acc);
            }
        }

        if (bad_rows) beta = __builtin_nan("");

        if (lane == 0) {
            const int32_t y = a.tokens[r];
            double acc_part, rej_part;
            if (y < 0 || y >= a.vocab || bad_rows) {
                acc_part = rej_part = __builtin_nan("");
            } else {
                const float lt = load_one<DT>(trow, y);
                const float ld = load_one<DT>(drow, y);
                const double p = lt >= tau_t ? exp2((double)lt * cd - (double)mcc_t) / s_t : 0.0;
                const double q = ld >= tau_d ? exp2((double)ld * cd - (double)mcc_d) / s_d : 0.0;
                acc_part = fmin(p, q);
                rej_part = p - acc_part;
            }
            if (a.out_terms != nullptr) {
                a.out_terms[2 * (int64_t)r] = (float)acc_part;
                a.out_terms[2 * (int64_t)r + 1] = (float)rej_part;
            }
            if (a.out_beta != nullptr) a.out_beta[r] = (float)beta;
            nll -= log(acc_part + rej_part);
        }
    }
    if (lane == 0) s_nll[wave_id()] = nll;
    __syncthreads();
    if (threadIdx.x == 0 && a.out_nll != nullptr) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += s_nll[w];
        a.out_nll[b] = t;
    }
}

}  // namespace sv
