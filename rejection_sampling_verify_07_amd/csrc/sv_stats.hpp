// Streaming pass over every logit row: the only O(rows x V) work of the
// verify step, and the one that sets its speed (it is bound by HBM reads).
//
// Softmax over the vocabulary of each target and draft row ("Text
// Generation via Speculative Sampling, KV Caching, and OpenVINO", sections
// "Prepare autoregressive sampling" and "Prepare speculative sampling") is
// reduced here to per-chunk statistics; the accept pass merges them.
//
// Tiles of 256 * LOADS aligned 16-byte blocks per (row, chunk), one tile per
// workgroup (sv_stream.hpp).  Every thread keeps its LOADS raw words in
// registers and walks them twice:
//   MODE_FULL   chunk max m_c, then S_c = sum exp2(fl32(l * c - fl32(m_c * c)))
//               (fp32 terms, fp64 accumulation across blocks and lanes);
//   MODE_ARGMAX chunk max, then the lowest row index that holds it.
// Rows need not be 16-byte aligned: the out-of-row slots of the blocks that
// straddle a row edge are overwritten with -inf before either walk.
#pragma once

#include "sv_common.hpp"
#include "sv_stream.hpp"

namespace sv {

enum { MODE_FULL = 0, MODE_ARGMAX = 1 };

// Edge tiles (a block reaching outside the row) overwrite the out-of-row
// slots of their raw words with -inf first: -inf never raises a maximum and
// exp2(-inf) = 0, so the element loops below need no masks.
template <int DT, int LOADS>
__device__ __forceinline__ void sanitize_edge(const Tile& t, int32_t vocab, u32x4* rw)
{
    constexpr int VEC = Dt<DT>::kVec;
    const bool interior = t.cb0 * VEC >= t.mis && (t.cb0 + kThreads * LOADS) * VEC <= t.mis + vocab;
    if (interior) return;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int32_t r0 = (tile_b0(t) + i * kThreads) * VEC - t.mis;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t w = rw[i][q];
            if constexpr (Dt<DT>::kSize == 2) {
                if ((uint32_t)(r0 + 2 * q) >= (uint32_t)vocab) w = (w & 0xffff0000u) | Dt<DT>::kNegInf;
                if ((uint32_t)(r0 + 2 * q + 1) >= (uint32_t)vocab) w = (w & 0x0000ffffu) | (Dt<DT>::kNegInf << 16);
            } else {
                if ((uint32_t)(r0 + q) >= (uint32_t)vocab) w = 0xff800000u;
            }
            rw[i][q] = w;
        }
    }
}

template <int DT, int LOADS>
__device__ __forceinline__ float lane_max(const u32x4* raw)
{
    float tm = neg_inf();
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        float f[Dt<DT>::kVec];
        unpack<DT>(raw[i], f);
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e) tm = fmaxf(tm, f[e]);
    }
    return tm;
}

// MODE_FULL with every element masked in place of the -inf fill of edge
// tiles.  Same results; on MI355X this form sustains more HBM bandwidth than
// the masked-free one over grids far larger than the chip (1.1 GB of logits
// at 8 loads per thread: about 157 us against 170-175 us), and less over
// grids of a few resident waves of tiles, so the plan picks per grid size.
template <int DT, int LOADS>
__device__ __forceinline__ void full_masked(const Tile& t, const u32x4* raw, int32_t vocab, float c,
                                            void* __restrict__ partials, float* s_m, double* s_s)
{
    constexpr int VEC = Dt<DT>::kVec;
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

// zero[0 .. nzero): cleared (grid-stride) for a kernel that runs after this
// one (the per-sequence tickets of the split verify).
template <int DT, int MODE, int LOADS, bool NT, bool MASKED = false>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(RowSet rs, int32_t vocab, int32_t nchunk,
                                                             int32_t ntiles, float c, void* __restrict__ partials,
                                                             int32_t* __restrict__ zero, int32_t nzero)
{
    for (int32_t i = (int32_t)(blockIdx.x * kThreads + threadIdx.x); i < nzero; i += (int32_t)(gridDim.x * kThreads))
        zero[i] = 0;
    constexpr int VEC = Dt<DT>::kVec;
    __shared__ float s_m[kWaves];
    __shared__ int32_t s_i[kWaves];
    __shared__ double s_s[kWaves];

    walk_tiles<DT, LOADS, NT>(rs, vocab, nchunk, ntiles, [&](const Tile& t, u32x4* raw) {
        if constexpr (MODE == MODE_FULL && MASKED) {
            full_masked<DT, LOADS>(t, raw, vocab, c, partials, s_m, s_s);
            return;
        }
        sanitize_edge<DT, LOADS>(t, vocab, raw);
        const float tm = lane_max<DT, LOADS>(raw);
        // With 8 loads per thread, widen again after the barrier rather than
        // keep every widened value live across it (an empty asm that claims
        // to update the raw words; it emits no instruction), which keeps the
        // pass within 64 VGPRs.  With 4 the widened values fit and are kept.
        if constexpr (LOADS > 4) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) asm volatile("" : "+v"(raw[i]));
        }
        const float wm = wave_max(tm);
        if (lane_id() == 0) s_m[wave_id()] = wm;
        __syncthreads();
        float m = s_m[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_m[w]);

        if constexpr (MODE == MODE_ARGMAX) {
            // the lowest row index holding m: only lanes whose own maximum is m
            // look for it (-inf also matches the fill, so indexes are range-checked)
            int32_t idx = INT32_MAX;
            if (tm == m) {
#pragma unroll
                for (int i = LOADS - 1; i >= 0; --i) {  // backwards: the last hit is the lowest index
                    float f[VEC];
                    unpack<DT>(raw[i], f);
                    const int32_t r0 = (tile_b0(t) + i * kThreads) * VEC - t.mis;
#pragma unroll
                    for (int e = VEC - 1; e >= 0; --e) {
                        const int32_t r = r0 + e;
                        idx = (f[e] == m && (uint32_t)r < (uint32_t)vocab) ? r : idx;
                    }
                }
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) idx = min(idx, __shfl_xor(idx, o, kWave));
            if (lane_id() == 0) s_i[wave_id()] = idx;
            __syncthreads();
            if (threadIdx.x == 0) {
                int32_t ix = s_i[0];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) ix = min(ix, s_i[w]);
                PartialArg* out = reinterpret_cast<PartialArg*>(partials) + t.index;
                out->m = m;
                out->idx = ix;
            }
        } else {
            const float mcc = m * c;
            double acc = 0.0;
            if (m != neg_inf()) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    float f[VEC];
                    unpack<DT>(raw[i], f);
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
