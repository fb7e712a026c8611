// Top-k kept sets for the sampling path (top-K filtering of the sampling
// helpers on "CS3602_FINAL_SpeDec", project structure / utils.py).
//
// The kept set of a row is every id whose raw logit is >= tau, the top_k-th
// largest logit counted with multiplicity (ties at tau are all kept).
//
// Pass 1 (topk_cand_kernel, streaming, one workgroup per (row, chunk)):
//   Each wave finds, with a 16-step ballot radix select, the j-th largest
//   (j = ceil(top_k / 4)) of its 64 lane maxima; the smallest of the four
//   wave results is a lower bound of the chunk's top_k-th largest logit
//   (at least 4 * j >= top_k distinct elements reach it), hence of the row's
//   tau.  Every chunk element >= that bound is written out as a candidate.
//   The candidate set of a row therefore contains its whole kept set.
// Pass 2 (topk_select_kernel, one workgroup per row):
//   exact radix select of the top_k-th largest key among the candidates,
//   the kept list sorted by id, its max and its sum of exp2 terms.  When a
//   chunk overflowed its candidate slots (or top_k is too large for pass 1)
//   the same exact select runs over the full row instead; a kept set larger
//   than the list capacity is described as "full row masked by tau".
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr int kSelCap = 4096;  // candidates a row can hold in LDS
constexpr int kTopkFastMax = 4 * kWave;  // largest top_k pass 1 supports

template <int DT, int LOADS, bool NT>
__global__ __launch_bounds__(kThreads) void topk_cand_kernel(RowSet rs, int32_t vocab, int32_t nchunk,
                                                             int32_t top_k, int32_t cap,
                                                             int32_t* __restrict__ counts,
                                                             KeptEntry* __restrict__ cands)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    __shared__ uint32_t s_h[kWaves];
    __shared__ int32_t s_cnt;

    const int32_t row = (int32_t)(blockIdx.x / (uint32_t)nchunk);
    const int32_t chunk = (int32_t)blockIdx.x - row * nchunk;
    const uintptr_t addr = (uintptr_t)row_ptr(rs, row);
    const int32_t mis = (int32_t)((addr & 15u) / ES);
    const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
    const int32_t b0 = chunk * (kThreads * LOADS) + (int32_t)threadIdx.x;

    u32x4 raw[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int32_t j = b0 + i * kThreads;
        raw[i] = (j < nblk) ? load16<NT>(base + j) : u32x4{0u, 0u, 0u, 0u};
    }
    auto block = [&](int i, float* f) {
        const int32_t j = b0 + i * kThreads;
        unpack<DT>(raw[i], f);
        const int32_t r0 = j * VEC - mis;
        if (j >= nblk || r0 < 0 || r0 + VEC > vocab) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int32_t r = r0 + e;
                if (j >= nblk || r < 0 || r >= vocab) f[e] = neg_inf();
            }
        }
    };

    float tm = neg_inf();
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        float f[VEC];
        block(i, f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) tm = fmaxf(tm, f[e]);
    }

    // j-th largest of the 64 lane maxima on the top 16 key bits
    const int jw = (top_k + kWaves - 1) / kWaves;
    const uint32_t key16 = order_key(tm) >> 16;
    uint32_t h = 0;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cand = h | (1u << bit);
        const uint64_t bal = __ballot(key16 >= cand);
        if (__popcll(bal) >= jw) h = cand;
    }
    if (lane_id() == 0) s_h[wave_id()] = h;
    if (threadIdx.x == 0) s_cnt = 0;
    __syncthreads();
    uint32_t hmin = s_h[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) hmin = min(hmin, s_h[w]);
    // smallest float whose key has these top bits; the -inf bucket maps to -inf
    const float bound = (hmin <= (order_key(neg_inf()) >> 16)) ? neg_inf() : key_to_float(hmin << 16);

    KeptEntry* out = cands + (int64_t)blockIdx.x * cap;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        float f[VEC];
        block(i, f);
        const int32_t j = b0 + i * kThreads;
        const int32_t r0 = j * VEC - mis;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool pred = f[e] >= bound;
            if (__ballot(pred) != 0) {
                const int32_t r = r0 + e;
                const bool take = pred && j < nblk && r >= 0 && r < vocab;
                const uint64_t m2 = __ballot(take);
                if (m2 != 0) {
                    int slot0 = 0;
                    if (lane_id() == 0) slot0 = atomicAdd(&s_cnt, (int)__popcll(m2));
                    slot0 = __shfl(slot0, 0, kWave);
                    if (take) {
                        const int slot = slot0 + lanes_below(m2);
                        if (slot < cap) out[slot] = KeptEntry{r, f[e]};
                    }
                }
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) counts[blockIdx.x] = s_cnt;
}

// ---------------------------------------------------------------------------
// Pass 2 helpers
// ---------------------------------------------------------------------------

// Visit every element of a full row (ascending blocks, 16-byte loads); fn(r, v)
// gets the row index r and the value, and is called only for r in [0, vocab).
// Iteration `it` covers blocks it*256 + tid, so a workgroup-wide scan per
// iteration yields ascending-id order.
template <int DT, class F>
__device__ __forceinline__ void for_row_blocks(const char* rowp, int32_t vocab, F&& fn)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    const uintptr_t addr = (uintptr_t)rowp;
    const int32_t mis = (int32_t)((addr & 15u) / ES);
    const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
    const int32_t iters = (nblk + kThreads - 1) / kThreads;
    for (int32_t it = 0; it < iters; ++it) {
        const int32_t j = it * kThreads + (int32_t)threadIdx.x;
        float f[VEC];
        bool ok[VEC];
        if (j < nblk) {
            unpack<DT>(load16<false>(base + j), f);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int32_t r = j * VEC - mis + e;
            ok[e] = j < nblk && r >= 0 && r < vocab;
        }
        fn(it, j * VEC - mis, f, ok);
    }
}

// Block-wide exclusive prefix sum of an int (fixed order); total via *total.
__device__ __forceinline__ int block_excl_scan_int(int v, int* s_w, int* total)
{
    const int incl = wave_incl_scan_int(v);
    if (lane_id() == kWave - 1) s_w[wave_id()] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave_id()) off += s_w[w];
        tot += s_w[w];
    }
    __syncthreads();
    *total = tot;
    return off + incl - v;
}

// Radix select over a set of keys: the rank-k largest (1-based, with
// multiplicity).  `visit(fn)` must call fn(key) once per key of the set, the
// same set on every call, from any threads of the block.  Digits of 8 bits
// from the top; `low_shift` stops early when the low key bits are implied
// (bf16: keys are determined by their top 16 bits).  Returns the key and
// the number of keys equal to it; *greater gets the number above it.
template <class Visit>
__device__ uint32_t block_radix_select(Visit&& visit, int32_t k, int low_shift, uint32_t* s_hist,
                                       int32_t* s_misc, int32_t* greater, int32_t* equal)
{
    uint32_t prefix = 0, pmask = 0;
    int32_t kk = k;
    int32_t eq = 0;
    for (int shift = 24; shift >= low_shift; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kThreads) s_hist[i] = 0;
        __syncthreads();
        visit([&](uint32_t key) {
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (wave_id() == 0) {
            // lane L holds digits 255-4L .. 252-4L (descending)
            const int l = lane_id();
            int c4[4];
            int lsum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c4[q] = (int)s_hist[255 - 4 * l - q];
                lsum += c4[q];
            }
            const int incl = wave_incl_scan_int(lsum);
            const int excl = incl - lsum;
            // first (descending) digit whose cumulative count reaches kk
            int found = -1, above = 0, cnt = 0;
            if (excl < kk && incl >= kk) {
                int c = excl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (found < 0 && c + c4[q] >= kk) {
                        found = 255 - 4 * l - q;
                        above = c;
                        cnt = c4[q];
                    }
                    c += c4[q];
                }
            }
            const uint64_t bal = __ballot(found >= 0);
            if (bal != 0) {
                const int src = __builtin_ctzll(bal);
                found = __shfl(found, src, kWave);
                above = __shfl(above, src, kWave);
                cnt = __shfl(cnt, src, kWave);
            } else {
                found = 0;  // fewer than kk keys match: report the lowest digit
                above = incl;
                cnt = 0;
                above = __shfl(above, kWave - 1, kWave);
            }
            if (l == 0) {
                s_misc[0] = found;
                s_misc[1] = kk - above;
                s_misc[2] = cnt;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_misc[0] << shift;
        pmask |= 0xffu << shift;
        kk = s_misc[1];
        eq = s_misc[2];
        __syncthreads();
    }
    if (low_shift > 0) {
        // bf16: the low key bits follow from the sign (0 for positive, ones for negative)
        prefix |= (prefix & 0x80000000u) ? 0u : ((1u << low_shift) - 1u);
    }
    *greater = k - kk;
    *equal = eq;
    return prefix;
}

// Block-wide max / sum (fixed order); every thread gets the result.
__device__ __forceinline__ float block_max_float(float v, float* s_f)
{
    v = wave_max(v);
    __syncthreads();
    if (lane_id() == 0) s_f[wave_id()] = v;
    __syncthreads();
    float m = s_f[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_f[w]);
    return m;
}

__device__ __forceinline__ double block_sum_double(double v, double* s_d)
{
    v = wave_sum(v);
    __syncthreads();
    if (lane_id() == 0) s_d[wave_id()] = v;
    __syncthreads();
    double t = s_d[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += s_d[w];
    return t;
}

template <int DT>
__device__ float block_row_max(const char* rowp, int32_t vocab, float* s_f)
{
    float lm = neg_inf();
    for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e)
            if (ok[e]) lm = fmaxf(lm, f[e]);
    });
    return block_max_float(lm, s_f);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    RowSet rs, int32_t vocab, int32_t nchunk, int32_t top_k, int32_t cap, float c,
    const int32_t* __restrict__ counts, const KeptEntry* __restrict__ cands, int32_t use_cands,
    int32_t keep_cap, RowDesc* __restrict__ descs, KeptEntry* __restrict__ kept)
{
    constexpr int LOW = (DT == DT_BF16) ? 16 : 0;
    __shared__ uint32_t s_key[kSelCap];
    __shared__ int32_t s_idx[kSelCap];
    __shared__ uint32_t s_hist[256];
    __shared__ int32_t s_misc[8];
    __shared__ int32_t s_w[kWaves];
    __shared__ double s_d[kWaves];
    __shared__ float s_f[kWaves];

    const int32_t row = blockIdx.x;
    const char* rowp = row_ptr(rs, row);
    KeptEntry* klist = kept + (int64_t)row * keep_cap;

    // ---- gather the candidates of this row (if pass 1 ran and nothing overflowed)
    int32_t total = 0;
    bool fast = use_cands != 0;
    if (fast) {
        if (threadIdx.x == 0) {
            int32_t t = 0, bad = 0;
            for (int32_t ch = 0; ch < nchunk; ++ch) {
                const int32_t n = counts[(int64_t)row * nchunk + ch];
                if (n > cap) bad = 1;
                t += min(n, cap);
            }
            s_misc[0] = t;
            s_misc[1] = bad || t > kSelCap || t < top_k;
        }
        __syncthreads();
        total = s_misc[0];
        fast = s_misc[1] == 0;
        __syncthreads();
    }
    if (fast) {
        int32_t off = 0;
        for (int32_t ch = 0; ch < nchunk; ++ch) {
            const int64_t g = (int64_t)row * nchunk + ch;
            const int32_t n = counts[g];
            const KeptEntry* src = cands + g * cap;
            for (int32_t t = threadIdx.x; t < n; t += kThreads) {
                const KeptEntry e = src[t];
                s_key[off + t] = order_key(e.val);
                s_idx[off + t] = e.idx;
            }
            off += n;
        }
        __syncthreads();
    }

    // ---- exact top_k-th largest key
    int32_t greater = 0, equal = 0;
    uint32_t tau_key;
    if (fast) {
        tau_key = block_radix_select(
            [&](auto&& fn) {
                for (int32_t i = threadIdx.x; i < total; i += kThreads) fn(s_key[i]);
            },
            top_k, LOW, s_hist, s_misc, &greater, &equal);
    } else {
        tau_key = block_radix_select(
            [&](auto&& fn) {
                for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
                    for (int e = 0; e < Dt<DT>::kVec; ++e)
                        if (ok[e]) fn(order_key(f[e]));
                });
            },
            top_k, LOW, s_hist, s_misc, &greater, &equal);
    }
    const float tau = key_to_float(tau_key);
    const int32_t nkept = greater + equal;

    // ---- kept list (ascending id) or masked full row
    float m;
    double s_sum = 0.0;
    int32_t kept_n;
    if (nkept <= keep_cap) {
        if (fast) {
            // compact the candidates >= tau, then sort them by id (bitonic)
            if (threadIdx.x == 0) s_misc[4] = 0;
            __syncthreads();
            __shared__ int32_t s_kidx[1024];
            __shared__ float s_kval[1024];
            for (int32_t i = threadIdx.x; i < total; i += kThreads) {
                if (s_key[i] >= tau_key) {
                    const int32_t slot = atomicAdd(&s_misc[4], 1);
                    if (slot < 1024) {
                        s_kidx[slot] = s_idx[i];
                        s_kval[slot] = key_to_float(s_key[i]);
                    }
                }
            }
            __syncthreads();
            int32_t npad = 1;
            while (npad < nkept) npad <<= 1;
            for (int32_t i = nkept + threadIdx.x; i < npad; i += kThreads) {
                s_kidx[i] = INT32_MAX;
                s_kval[i] = neg_inf();
            }
            __syncthreads();
            for (int32_t size = 2; size <= npad; size <<= 1) {
                for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int32_t i = threadIdx.x; i < npad; i += kThreads) {
                        const int32_t p = i ^ stride;
                        if (p > i) {
                            const bool up = (i & size) == 0;
                            const int32_t a = s_kidx[i], bb = s_kidx[p];
                            if ((a > bb) == up) {
                                s_kidx[i] = bb;
                                s_kidx[p] = a;
                                const float t = s_kval[i];
                                s_kval[i] = s_kval[p];
                                s_kval[p] = t;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            for (int32_t i = threadIdx.x; i < nkept; i += kThreads) klist[i] = KeptEntry{s_kidx[i], s_kval[i]};
            // max and sum over the list (fixed order)
            float lm = neg_inf();
            for (int32_t i = threadIdx.x; i < nkept; i += kThreads) lm = fmaxf(lm, s_kval[i]);
            m = block_max_float(lm, s_f);
            const float mcc = m * c;
            double ls = 0.0;
            for (int32_t i = threadIdx.x; i < nkept; i += kThreads)
                ls += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(s_kval[i], c, -mcc));
            s_sum = block_sum_double(ls, s_d);
        } else {
            // ordered compaction straight from the row, after its max
            m = block_row_max<DT>(rowp, vocab, s_f);
            const float mcc = m * c;
            int32_t base = 0;
            double ls = 0.0;
            for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t r0, const float* f, const bool* ok) {
                int cnt = 0;
#pragma unroll
                for (int e = 0; e < Dt<DT>::kVec; ++e) cnt += (ok[e] && order_key(f[e]) >= tau_key);
                int tot;
                int pos = base + block_excl_scan_int(cnt, s_w, &tot);
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < Dt<DT>::kVec; ++e) {
                    if (ok[e] && order_key(f[e]) >= tau_key) {
                        klist[pos++] = KeptEntry{r0 + e, f[e]};
                        s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
                    }
                }
                ls += (double)s;
                base += tot;
            });
            s_sum = block_sum_double(ls, s_d);
        }
        kept_n = nkept;
    } else {
        // too many kept ids for a list: describe the row as "full row masked by tau"
        m = block_row_max<DT>(rowp, vocab, s_f);
        const float mcc = m * c;
        double ls = 0.0;
        for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e)
                if (ok[e] && f[e] >= tau) s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
            ls += (double)s;
        });
        s_sum = block_sum_double(ls, s_d);
        kept_n = -1;
    }
    if (threadIdx.x == 0) {
        RowDesc d;
        d.tau = tau;
        d.m = m;
        d.mcc = m * c;
        d.kept = kept_n;
        d.s = s_sum;
        d.flags = fast ? 0 : 1;
        d.pad = 0;
        descs[row] = d;
    }
}

}  // namespace sv
