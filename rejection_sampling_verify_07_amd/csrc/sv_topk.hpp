// Top-k kept sets for the sampling path (top-K filtering of the sampling
// helpers on "CS3602_FINAL_SpeDec", project structure / utils.py).
//
// The kept set of a row is every id whose raw logit is >= tau, the top_k-th
// largest logit counted with multiplicity (ties at tau are all kept).
//
// Pass 1 (topk_cand_kernel, streaming, one workgroup per (row, chunk)):
//   a 16-step ballot radix select finds the top_k-th largest of the
//   workgroup's 256 lane maxima; top_k distinct elements reach it, so it is
//   a lower bound of the chunk's top_k-th largest logit, hence of the row's
//   tau.  Every chunk element >= that bound is written out as a candidate.
//   The candidate set of a row therefore contains its whole kept set.
// Pass 2 (topk_select_kernel, one workgroup per row):
//   exact radix select of the top_k-th largest key among the candidates,
//   the kept list sorted by id, its max and its sum of exp2 terms.  When a
//   chunk overflowed its candidate slots (or top_k is too large for pass 1)
//   the same exact select runs over the full row instead; a kept set larger
//   than the list capacity is described as "full row masked by tau".
#pragma once

#include <type_traits>

#include "sv_common.hpp"
#include "sv_stream.hpp"

namespace sv {

constexpr int kSelCap = 4096;  // candidates a row can hold in LDS
constexpr int kTopkFastMax = kThreads;   // largest top_k pass 1 supports (one lane maximum each)
constexpr int kTopkFastMax2 = 2 * kThreads;  // with two keys per lane
constexpr int kMaxChunks = 512;          // chunks per row the select pass can index
constexpr int kKeepCapList = 1024;       // kept-list capacity per row (ids kept by top-k)

// ---------------------------------------------------------------------------
// Pass 2 helpers
// ---------------------------------------------------------------------------

// Visit every element of a full row in ascending 16-byte blocks, with a
// workgroup of NT threads.  Each thread keeps U loads in flight;
// fn(step, r0, f, ok) is then called once per block, in the same step for
// all threads, where step s covers blocks s*NT .. s*NT+NT-1 (so a workgroup
// scan per step yields ascending id order); r0 is the row index of the
// block's first element and ok[e] tells which of its elements lie inside the
// row.
constexpr int kRowUnroll = 8;

template <int DT, int NT = kThreads, int U = kRowUnroll, class F>
__device__ __forceinline__ void for_row_blocks(const char* rowp, int32_t vocab, F&& fn)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    const uintptr_t addr = (uintptr_t)rowp;
    const int32_t mis = (int32_t)((addr & 15u) / ES);
    const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
    const int32_t iters = (nblk + NT * U - 1) / (NT * U);
    for (int32_t it = 0; it < iters; ++it) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j = (it * U + u) * NT + (int32_t)threadIdx.x;
            raw[u] = (j < nblk) ? load16<false>(base + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t step = it * U + u;
            const int32_t j = step * NT + (int32_t)threadIdx.x;
            float f[VEC];
            bool ok[VEC];
            unpack<DT>(raw[u], f);
            // one unsigned compare per element: r < 0 wraps past vocab, and a
            // block past the row (j >= nblk) starts at or beyond vocab
#pragma unroll
            for (int e = 0; e < VEC; ++e) ok[e] = (uint32_t)(j * VEC - mis + e) < (uint32_t)vocab;
            fn(step, j * VEC - mis, f, ok);
        }
    }
}

// Block-wide exclusive prefix sum of an int (fixed order); total via *total.
// s_w holds NT / 64 ints.
template <int NT = kThreads>
__device__ __forceinline__ int block_excl_scan_int(int v, int* s_w, int* total)
{
    const int incl = wave_incl_scan_int(v);
    if (lane_id() == kWave - 1) s_w[wave_id()] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
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
__device__ __forceinline__ uint32_t block_radix_select(Visit&& visit, int32_t k, int low_shift, uint32_t* s_hist,
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

// LDS staging of one chunk's candidates before they go to global memory:
// each wave owns kWaveLds slots, so no atomics are needed.
constexpr int kWaveLds = 512;
constexpr int kChunkLds = kWaves * kWaveLds;

// Eight waves per SIMD (at most 64 VGPRs): this pass is latency bound, and
// resident waves are what hides the HBM latency.  Only the raw words stay
// live across the barrier; values are widened where they are used.
//
// bf16: a 32-bit word holds two elements.  Its high element is compared
// through the raw word read as fp32: the top 16 bits are the element and the
// low 16 bits (its neighbour) move it by less than one bf16 step (toward
// -inf for negatives, +inf for positives); every threshold used here is the
// smallest fp32 of some bf16 order class, so `word >= t` and `element >= t`
// agree.  The low element needs a shift.  The lane maxima that set the bound
// are taken over all elements.  fp16 elements are widened (exactly) instead.
//
// KEYS = 2 (larger top_k): the bound comes from 512 keys, each lane's largest
// and second-largest 16-byte block maximum (distinct elements of the tile, so
// top_k of them reaching a value means top_k elements do).
template <int DT, int LOADS, bool NT, int KEYS>
__global__ __launch_bounds__(kThreads) void topk_cand_kernel(
    RowSet rs, int32_t vocab, int32_t nchunk, int32_t ntiles, int32_t top_k, int32_t cap,
    int32_t* __restrict__ counts, float* __restrict__ bounds, KeptEntry* __restrict__ cands, int32_t xcd)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int LOW = (DT == DT_BF16) ? 16 : 0;
    constexpr bool BF = DT == DT_BF16;
    constexpr bool H16 = DT == DT_F16;
    __shared__ __align__(16) float s_val[kChunkLds];
    __shared__ int32_t s_ix[kChunkLds];
    __shared__ uint32_t s_lk[kThreads * KEYS];
    __shared__ int32_t s_wc[kWaves];
    __shared__ uint32_t s_hist[256];
    __shared__ int32_t s_misc[8];

    walk_tiles<DT, LOADS, NT>(rs, vocab, nchunk, ntiles, [&](const Tile& t, u32x4* raw) {
        // Edge tiles (a block reaching outside the row) first overwrite the
        // out-of-row slots of their raw words with a NaN pattern: NaN is never
        // selected and the maximum ignores it, so one body serves every tile.
        const bool interior = t.cb0 * VEC >= t.mis && (t.cb0 + kThreads * LOADS) * VEC <= t.mis + vocab;
        u32x4* rw = raw;
        if (!interior) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int32_t r0 = (tile_b0(t) + i * kThreads) * VEC - t.mis;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t w = rw[i][q];
                    if constexpr (Dt<DT>::kSize == 2) {
                        if ((uint32_t)(r0 + 2 * q) >= (uint32_t)vocab) w = (w & 0xffff0000u) | Dt<DT>::kNaN;
                        if ((uint32_t)(r0 + 2 * q + 1) >= (uint32_t)vocab) w = (w & 0x0000ffffu) | (Dt<DT>::kNaN << 16);
                    } else {
                        if ((uint32_t)(r0 + q) >= (uint32_t)vocab) w = 0x7fc00000u;
                    }
                    rw[i][q] = w;
                }
            }
        }
        int wcount = 0;  // wave-uniform count of this wave's candidates
        const int wbase = wave_id() * kWaveLds;
        float bound;  // the tile's lower bound of the row's tau
        {
            // the maximum of each 16-byte block, and the lane's maximum
            float bm[LOADS];
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                float b = neg_inf();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = raw[i][q];
                    if constexpr (BF) {
                        // both elements exactly: the raw word would be a
                        // signalling NaN for a -inf high element
                        b = max3_quiet(b, __uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
                    } else if constexpr (H16) {
                        b = max3_quiet(b, lo16<DT>(w), hi16<DT>(w));
                    } else if (q & 1) {
                        b = max3_quiet(b, __uint_as_float(raw[i][q - 1]), __uint_as_float(w));
                    }
                }
                bm[i] = b;
            }
            float tm = bm[0];
#pragma unroll
            for (int i = 1; i < LOADS; i += 2)
                tm = (i + 1 < LOADS) ? max3_quiet(tm, bm[i], bm[i + 1]) : max3_quiet(tm, bm[i], bm[i]);

            // Recompute the widened values in the compaction pass instead of
            // keeping all of them live across the barrier (an empty asm that
            // claims to update the raw words stops the compiler from reusing
            // them; it emits no instruction).
#pragma unroll
            for (int i = 0; i < LOADS; ++i) asm volatile("" : "+v"(rw[i]));

            // the top_k-th largest of the workgroup's 256 * KEYS keys (lane maxima,
            // and with KEYS = 2 the lanes' second-largest block maxima too; on the
            // top 16 key bits): wave 0 runs a ballot radix select over all of
            // them, 4 * KEYS per lane, and hands the result to the others
            // through LDS, so the other waves' SIMDs are free for other tiles
            constexpr int KPL = 4 * KEYS;  // keys per lane
            s_lk[threadIdx.x] = order_key(tm) >> 16;
            if constexpr (KEYS == 2) {
                // the second largest of the lane's block maxima (never NaN: -inf or finite)
                float t1 = bm[0], t2 = neg_inf();
#pragma unroll
                for (int i = 1; i < LOADS; ++i) {
                    t2 = __builtin_amdgcn_fmed3f(t1, t2, bm[i]);
                    t1 = fmaxf(t1, bm[i]);
                }
                s_lk[kThreads + threadIdx.x] = order_key(t2) >> 16;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(threadIdx.x) < kWave) {
                uint32_t kk[KPL];
#pragma unroll
                for (int q = 0; q < KPL; ++q) kk[q] = s_lk[lane_id() + q * kWave];
                // bits above the highest one where the largest and smallest key
                // differ are common to all keys: start the select below them
                uint32_t kmax = kk[0], kmin = kk[0];
#pragma unroll
                for (int q = 1; q < KPL; ++q) {
                    kmax = max(kmax, kk[q]);
                    kmin = min(kmin, kk[q]);
                }
                wave_umax_umin_dpp(kmax, kmin);
                const uint32_t diff = kmax ^ kmin;
                const int top = diff ? 31 - __builtin_clz(diff) : -1;  // highest differing bit
                uint32_t hs = top >= 0 ? kmax & ~((2u << top) - 1u) : kmax;  // the common prefix
                for (int bit = top; bit >= 0; --bit) {
                    const uint32_t cand = hs | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int q = 0; q < KPL; ++q) cnt += (int)__popcll(__ballot(kk[q] >= cand));
                    if (cnt >= top_k) hs = cand;
                }
                if (lane_id() == 0) s_misc[0] = (int32_t)hs;
            }
            __syncthreads();
            const uint32_t h = (uint32_t)s_misc[0];
            // smallest float whose key has these top bits; the -inf bucket maps to -inf
            bound = (h <= (order_key(neg_inf()) >> 16)) ? neg_inf() : key_to_float(h << 16);

            // Candidates into this wave's LDS region.  Only blocks whose maximum
            // reaches the bound can hold one (about 14 of the wave's 64 * LOADS
            // blocks on logits of a language model), so those blocks are first
            // staged in the same region (at most kStage of them), read back one
            // per lane, and only they take the per-element ballots.  The compare
            // of each element is the one of the full walk below, so both give
            // the same candidates.  The exact value and the row index are formed
            // only on the rare taken branch.  Slots past the region are clamped
            // (the tile is then reported as overflowed and its staging is not
            // used).
            auto element_cmp = [&](uint32_t w, int e) -> float {
                return BF    ? __uint_as_float((e & 1) ? w : (w << 16))
                       : H16 ? ((e & 1) ? hi16<DT>(w) : lo16<DT>(w))
                             : __uint_as_float(w);
            };
            auto element_bits = [&](uint32_t w, int e, float cmp) -> uint32_t {
                return BF ? ((e & 1) ? (w & 0xffff0000u) : (w << 16)) : H16 ? __float_as_uint(cmp) : w;
            };
            constexpr int kStage = kWaveLds / 4;  // 16-byte blocks in the wave's part of s_val
            u32x4* stage = reinterpret_cast<u32x4*>(s_val + wbase);
            int32_t* stage_blk = s_ix + wbase;
            int32_t nb = 0;  // wave-uniform count of blocks that reach the bound
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const bool hb = bm[i] >= bound;
                const uint64_t m = __ballot(hb);
                if (hb) {
                    const int32_t pos = nb + lanes_below(m);
                    if (pos < kStage) {
                        stage[pos] = raw[i];
                        stage_blk[pos] = i * kThreads + (int32_t)threadIdx.x;  // block - t.cb0
                    }
                }
                nb += (int32_t)__popcll(m);
            }
            __builtin_amdgcn_wave_barrier();
            if (nb <= 2 * kWave) {
                // read every staged block back before the candidates overwrite
                // them (a wave's LDS operations complete in issue order)
                u32x4 sb[2];
                int32_t so[2];
                bool sv[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int32_t sidx = r * kWave + lane_id();
                    sv[r] = sidx < nb;
                    const int32_t sc = min(sidx, kStage - 1);
                    sb[r] = stage[sc];
                    so[r] = stage_blk[sc];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    if (r * kWave >= nb) break;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int q = Dt<DT>::kSize == 2 ? e / 2 : e;
                        const uint32_t w = sb[r][q];
                        const float cmp = element_cmp(w, e);
                        const bool pred = sv[r] && cmp >= bound;
                        const uint64_t m = __ballot(pred);
                        if (m != 0) {
                            if (pred) {
                                const int pos = min(wcount + lanes_below(m), kWaveLds - 1);
                                s_val[wbase + pos] = __uint_as_float(element_bits(w, e, cmp));
                                s_ix[wbase + pos] = (t.cb0 + so[r]) * VEC - t.mis + e;
                            }
                            wcount += (int)__popcll(m);
                        }
                    }
                }
            } else {
                // many blocks reach the bound (ties, flat rows): every element
                // of the tile, in (load, element, lane) order
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int q = Dt<DT>::kSize == 2 ? e / 2 : e;
                        const uint32_t w = raw[i][q];
                        const float cmp = element_cmp(w, e);
                        const bool pred = cmp >= bound;
                        const uint64_t m = __ballot(pred);
                        if (m != 0) {
                            if (pred) {
                                const int pos = min(wcount + lanes_below(m), kWaveLds - 1);
                                s_val[wbase + pos] = __uint_as_float(element_bits(w, e, cmp));
                                s_ix[wbase + pos] = (tile_b0(t) + i * kThreads) * VEC - t.mis + e;
                            }
                            wcount += (int)__popcll(m);
                        }
                    }
                }
            }
        }
        if (lane_id() == 0) s_wc[wave_id()] = wcount;
        __syncthreads();
        int32_t total = 0, wover = 0, woff = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave_id()) woff += s_wc[w];
            total += s_wc[w];
            wover |= s_wc[w] > kWaveLds;
        }
        KeptEntry* out = cands + (int64_t)t.index * cap;
        int32_t written = total;
        if (!wover && total <= cap) {
            for (int32_t q = lane_id(); q < wcount; q += kWave)
                out[woff + q] = KeptEntry{s_ix[wbase + q], s_val[wbase + q]};
        } else if (!wover) {
            // too many for the slots: keep only the tile's own top_k (ties kept)
            int32_t greater, equal;
            const uint32_t tkey = block_radix_select(
                [&](auto&& fn) {
                    for (int w = 0; w < kWaves; ++w)
                        for (int32_t q = threadIdx.x; q < s_wc[w]; q += kThreads) fn(order_key(s_val[w * kWaveLds + q]));
                },
                top_k, LOW, s_hist, s_misc + 2, &greater, &equal);
            written = greater + equal;
            // The tile's own top_k-th largest value is a lower bound of the
            // row's tau too, and a much tighter one than the lane maxima give
            // when top_k is close to 256: reported as the tile's bound, it
            // keeps the select's survivors (candidates >= the largest bound)
            // within its list.
            if (tkey > (order_key(neg_inf()) & (~0u << LOW))) bound = fmaxf(bound, key_to_float(tkey));
            if (written <= cap) {
                if (threadIdx.x == 0) s_misc[1] = 0;
                __syncthreads();
                for (int w = 0; w < kWaves; ++w) {
                    for (int32_t q = threadIdx.x; q < s_wc[w]; q += kThreads) {
                        const float v = s_val[w * kWaveLds + q];
                        if (order_key(v) >= tkey) {
                            const int32_t slot = atomicAdd(&s_misc[1], 1);
                            out[slot] = KeptEntry{s_ix[w * kWaveLds + q], v};
                        }
                    }
                }
            }
        } else {
            written = cap + 1;  // a wave overflowed its staging slots
        }
        if (threadIdx.x == 0) {
            counts[t.index] = written;  // > cap marks an overflow
            bounds[t.index] = bound;
        }
    }, xcd);
}

// Block-wide max / sum over NT threads (fixed order); every thread gets the
// result.  s_f / s_d hold NT / 64 values.
template <int NT = kThreads>
__device__ __forceinline__ float block_max_float(float v, float* s_f)
{
    v = wave_max(v);
    __syncthreads();
    if (lane_id() == 0) s_f[wave_id()] = v;
    __syncthreads();
    float m = s_f[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) m = fmaxf(m, s_f[w]);
    return m;
}

template <int NT = kThreads>
__device__ __forceinline__ double block_sum_double(double v, double* s_d)
{
    v = wave_sum(v);
    __syncthreads();
    if (lane_id() == 0) s_d[wave_id()] = v;
    __syncthreads();
    double t = s_d[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) t += s_d[w];
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

// The exact select over a full row, one workgroup per row: the path of
// top_k too large for the candidate pass.
template <int DT>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    RowSet rs, int32_t vocab, int32_t top_k, float c, int32_t keep_cap, RowDesc* __restrict__ descs,
    KeptEntry* __restrict__ kept)
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
    __shared__ int32_t s_kidx[kKeepCapList];
    __shared__ float s_kval[kKeepCapList];
    // ---- exact top_k-th largest key
    int32_t greater = 0, equal = 0;
    uint32_t tau_key = 0;
    // Full rows first take two walks: (1) a histogram of the top 12 key bits
    // (s_key as 4096 counters: few keys share a counter), which gives the
    // bucket holding the top_k-th key, the count above it and its size;
    // (2) the bucket's own entries staged in LDS, where the select finishes,
    // and, when the list can hold them, the ids above the bucket straight
    // into it.  Only a bucket too large for LDS leaves the select to the
    // radix passes over the row below.
    bool staged = false;  // s_kidx / s_kval already hold the kept entries
    bool have_tau = false;
    {
        for (int i = threadIdx.x; i < kSelCap; i += kThreads) s_key[i] = 0;
        __syncthreads();
        for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e)
                if (ok[e]) atomicAdd(&s_key[order_key(f[e]) >> 20], 1u);
        });
        __syncthreads();
        // thread t owns buckets 4095 - 16t down to 4080 - 16t
        constexpr int kPer = kSelCap / kThreads;
        const int32_t top = kSelCap - 1 - kPer * (int32_t)threadIdx.x;
        int32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) mine += (int32_t)s_key[top - j];
        int32_t tot;
        const int32_t excl = block_excl_scan_int(mine, s_w, &tot);
        if (threadIdx.x == 0) s_misc[5] = -1;
        __syncthreads();
        if (excl < top_k && excl + mine >= top_k) {
            int32_t cum = excl;
            for (int j = 0; j < kPer; ++j) {
                const int32_t n = (int32_t)s_key[top - j];
                if (cum + n >= top_k) {
                    s_misc[5] = top - j;  // the bucket
                    s_misc[6] = cum;      // ids above it
                    s_misc[7] = n;        // ids in it
                    break;
                }
                cum += n;
            }
        }
        __syncthreads();
        const int32_t bucket = s_misc[5], above = s_misc[6], inb = s_misc[7];
        __syncthreads();
        if (bucket >= 0 && inb <= kSelCap) {
            const bool list = above + inb <= kKeepCapList && above + inb <= keep_cap;
            if (threadIdx.x == 0) {
                s_misc[4] = 0;  // kept ids so far
                s_misc[3] = 0;  // staged entries of the bucket
            }
            __syncthreads();
            for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t r0, const float* f, const bool* ok) {
#pragma unroll
                for (int e = 0; e < Dt<DT>::kVec; ++e) {
                    if (!ok[e]) continue;
                    const uint32_t key = order_key(f[e]);
                    const int32_t b = (int32_t)(key >> 20);
                    if (b > bucket) {
                        if (!list) continue;
                        const int32_t slot = atomicAdd(&s_misc[4], 1);
                        if (slot < kKeepCapList) {
                            s_kidx[slot] = r0 + e;
                            s_kval[slot] = f[e];
                        }
                    } else if (b == bucket) {
                        const int32_t slot = atomicAdd(&s_misc[3], 1);
                        if (slot < kSelCap) {
                            s_key[slot] = key;
                            s_idx[slot] = r0 + e;
                        }
                    }
                }
            });
            __syncthreads();
            const int32_t nb = min(s_misc[3], kSelCap);
            int32_t gb, eb;
            tau_key = block_radix_select(
                [&](auto&& fn) {
                    for (int32_t i = threadIdx.x; i < nb; i += kThreads) fn(s_key[i]);
                },
                top_k - above, LOW, s_hist, s_misc, &gb, &eb);
            greater = above + gb;
            equal = eb;
            // the bucket's entries >= tau join the list
            for (int32_t i = threadIdx.x; list && i < nb; i += kThreads) {
                if (s_key[i] >= tau_key) {
                    const int32_t slot = atomicAdd(&s_misc[4], 1);
                    if (slot < kKeepCapList) {
                        s_kidx[slot] = s_idx[i];
                        s_kval[slot] = key_to_float(s_key[i]);
                    }
                }
            }
            __syncthreads();
            staged = list;
            have_tau = true;
        }
    }
    if (!have_tau) {
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
    if (nkept <= keep_cap && nkept <= kKeepCapList) {
        // the kept entries into LDS in any order (an LDS slot counter), then
        // sorted by id (bitonic); the row's maximum is one of them
        if (!staged && threadIdx.x == 0) s_misc[4] = 0;
        __syncthreads();
        if (!staged) {
            // one walk of the row: at most a list's worth of ids pass
            for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t r0, const float* f, const bool* ok) {
#pragma unroll
                for (int e = 0; e < Dt<DT>::kVec; ++e) {
                    if (ok[e] && order_key(f[e]) >= tau_key) {
                        const int32_t slot = atomicAdd(&s_misc[4], 1);
                        if (slot < kKeepCapList) {
                            s_kidx[slot] = r0 + e;
                            s_kval[slot] = f[e];
                        }
                    }
                }
            });
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
        d.flags = 1;
        d.pad = 0;
        descs[row] = d;
    }
}

}  // namespace sv
