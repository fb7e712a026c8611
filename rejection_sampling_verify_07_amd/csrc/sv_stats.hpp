// Streaming pass over every logit row: the only O(rows x V) work of the
// verify step, and the one that sets its speed (it is bound by HBM reads).
//
// Softmax over the vocabulary of each target and draft row ("Text
// Generation via Speculative Sampling, KV Caching, and OpenVINO", sections
// "Prepare autoregressive sampling" and "Prepare speculative sampling") is
// reduced here to per-chunk statistics; the accept pass merges them.
//
// Tiles of 256 * LOADS aligned 16-byte blocks per (row, chunk), walked by a
// persistent pipelined grid (sv_stream.hpp).  Every thread keeps its LOADS
// raw words in registers and walks them twice:
//   MODE_FULL   chunk max m_c, then S_c = sum exp2(fl32(l * c - fl32(m_c * c)))
//               (fp32 terms, fp64 accumulation across blocks and lanes);
//   MODE_ARGMAX chunk max and the lowest row index that holds it.
// Rows need not be 16-byte aligned: the blocks that straddle a row edge are
// masked element by element.
#pragma once

#include "sv_common.hpp"
#include "sv_stream.hpp"

namespace sv {

enum { MODE_FULL = 0, MODE_ARGMAX = 1 };

template <int DT, int MODE, int LOADS, bool NT, bool PIPE>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(RowSet rs, int32_t vocab, int32_t nchunk,
                                                             int32_t ntiles, float c, void* __restrict__ partials)
{
    constexpr int VEC = Dt<DT>::kVec;
    __shared__ float s_m[kWaves];
    __shared__ int32_t s_i[kWaves];
    __shared__ double s_s[kWaves];

    walk_tiles<DT, LOADS, NT, PIPE>(rs, vocab, nchunk, ntiles, [&](const Tile& t, const u32x4* raw) {
        if constexpr (MODE == MODE_ARGMAX) {
            float best = neg_inf();
            // lowest valid row index this thread covers (ties at -inf resolve to it)
            int32_t bidx = (tile_b0(t) < t.nblk) ? max(tile_b0(t) * VEC - t.mis, 0) : INT32_MAX;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                float f[VEC];
                tile_block<DT>(t, raw, i, vocab, neg_inf(), f);
                const int32_t r0 = (tile_b0(t) + i * kThreads) * VEC - t.mis;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (f[e] > best) {
                        best = f[e];
                        bidx = r0 + e;
                    }
                }
            }
            wave_argmax(best, bidx);
            if (lane_id() == 0) {
                s_m[wave_id()] = best;
                s_i[wave_id()] = bidx;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                float v = s_m[0];
                int32_t ix = s_i[0];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) argmax_merge(v, ix, s_m[w], s_i[w]);
                PartialArg* out = reinterpret_cast<PartialArg*>(partials) + t.index;
                out->m = v;
                out->idx = ix;
            }
            __syncthreads();  // s_m / s_i are rewritten by the next tile
        } else {
            float mx = neg_inf();
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                float f[VEC];
                tile_block<DT>(t, raw, i, vocab, neg_inf(), f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) mx = fmaxf(mx, f[e]);
            }
            mx = wave_max(mx);
            if (lane_id() == 0) s_m[wave_id()] = mx;
            __syncthreads();
            float m = s_m[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_m[w]);

            const float mcc = m * c;
            double acc = 0.0;
            if (m != neg_inf()) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    float f[VEC];
                    tile_block<DT>(t, raw, i, vocab, neg_inf(), f);
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
                    acc += (double)s;
                }
            }
            acc = wave_sum(acc);
            if (lane_id() == 0) s_s[wave_id()] = acc;
            __syncthreads();
            if (threadIdx.x == 0) {
                double s = s_s[0];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) s += s_s[w];
                PartialFull* out = reinterpret_cast<PartialFull*>(partials) + t.index;
                out->m = m;
                out->mcc = mcc;
                out->s = s;
            }
        }
    });
}

}  // namespace sv
