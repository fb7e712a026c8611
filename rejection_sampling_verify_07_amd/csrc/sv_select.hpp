// Per-row top-k selection by one wave (64 threads, no workgroup barriers).
//
// Input: the candidates the streaming pass wrote for each (row, chunk) (every
// chunk element >= a lower bound of the row's tau, so the candidate set holds
// the whole kept set), or nothing (then the row itself is scanned).
// Output: the row descriptor (tau = the top_k-th largest logit with
// multiplicity, the max, fl32(max * c), the sum of exp2 terms over the kept
// set) and the kept list sorted by id, or kept = -1 ("full row masked by
// tau") when the kept set is larger than the list capacity.
//
// Fast path (no chunk overflowed, top_k <= candidates <= kKeepCapList):
// candidates go to registers (16 per lane), a ballot radix select over the
// top key bits finds tau without LDS atomics, the kept entries are
// compacted with ballots and sorted by id (a register bitonic network when
// at most 64 are kept, an LDS network otherwise).
// Exact path: the same radix select with one pass over the whole row per
// 8-bit digit, then an ordered compaction of the row.
#pragma once

#include "sv_common.hpp"
#include "sv_topk.hpp"

namespace sv {

constexpr int kSelPer = kKeepCapList / kWave;  // candidates per lane on the fast path

// Keys the radix select works on: bf16 logits are fully ordered by the top
// 16 bits of their fp32 order key; fp32 needs all 32.
template <int DT>
struct SelKey {
    static constexpr int kBits = (DT == DT_BF16) ? 16 : 32;
    __device__ __forceinline__ static uint32_t of(float v)
    {
        return (DT == DT_BF16) ? (order_key(v) >> 16) : order_key(v);
    }
    // the logit value of a key (bf16: the low 16 key bits follow from the sign)
    __device__ __forceinline__ static float value(uint32_t k)
    {
        if constexpr (DT == DT_BF16) {
            return key_to_float((k << 16) | ((k & 0x8000u) ? 0u : 0xffffu));
        } else {
            return key_to_float(k);
        }
    }
};

// Sort (id, value) pairs held one per lane (lanes >= n hold INT32_MAX) by id.
__device__ __forceinline__ void wave_bitonic_by_id(int32_t& ix, float& v)
{
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int32_t pix = __shfl_xor(ix, stride, kWave);
            const float pv = __shfl_xor(v, stride, kWave);
            const bool up = (lane & size) == 0;
            const bool lower = (lane & stride) == 0;
            const bool take = (lower == up) ? (pix < ix) : (pix > ix);
            if (take) {
                ix = pix;
                v = pv;
            }
        }
    }
}

// LDS scratch of one wave.
struct WaveSelLds {
    int32_t kidx[kKeepCapList];
    float kval[kKeepCapList];
    uint32_t hist[256];
};

template <int DT>
__device__ void wave_select_fast(int32_t row, int32_t nchunk, int32_t top_k, int32_t cap, float c,
                                 const int32_t* __restrict__ counts, const KeptEntry* __restrict__ cands,
                                 RowDesc* __restrict__ descs, KeptEntry* __restrict__ kept, WaveSelLds& L,
                                 const int32_t* choff, int32_t total)
{
    using K = SelKey<DT>;
    const int lane = lane_id();
    const int32_t nj = (total + kWave - 1) / kWave;  // wave-uniform

    // candidates into registers, all loads issued first
    KeptEntry e[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
        const int32_t i = lane + j * kWave;
        e[j] = KeptEntry{INT32_MAX, neg_inf()};
        if (j < nj && i < total) {
            int32_t lo = 0, hi = nchunk;
            while (hi - lo > 1) {
                const int32_t mid = (lo + hi) >> 1;
                if (choff[mid] <= i) lo = mid; else hi = mid;
            }
            e[j] = cands[((int64_t)row * nchunk + lo) * cap + (i - choff[lo])];
        }
    }
    uint32_t key[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) key[j] = (e[j].idx != INT32_MAX) ? K::of(e[j].val) : 0u;

    // ballot radix select: the largest h with #{key >= h} >= top_k
    uint32_t h = 0;
    for (int bit = K::kBits - 1; bit >= 0; --bit) {
        const uint32_t cand = h | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kSelPer; ++j)
            if (j < nj) cnt += (int)__popcll(__ballot(key[j] >= cand));
        if (cnt >= top_k) h = cand;
    }

    // kept entries (key >= h), compacted in candidate order
    int32_t nk = 0;
    float lm = neg_inf();
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
        if (j < nj) {
            const bool pred = key[j] >= h && e[j].idx != INT32_MAX;
            const uint64_t m = __ballot(pred);
            if (pred) {
                const int32_t pos = nk + lanes_below(m);
                L.kidx[pos] = e[j].idx;
                L.kval[pos] = e[j].val;
                lm = fmaxf(lm, e[j].val);
            }
            nk += (int32_t)__popcll(m);
        }
    }
    lm = __shfl(wave_max(lm), 0, kWave);
    const float mcc = lm * c;
    __builtin_amdgcn_wave_barrier();

    KeptEntry* klist = kept + (int64_t)row * kKeepCapList;
    double ls = 0.0;
    if (nk <= kWave) {
        int32_t ix = lane < nk ? L.kidx[lane] : INT32_MAX;
        float v = lane < nk ? L.kval[lane] : neg_inf();
        wave_bitonic_by_id(ix, v);
        if (lane < nk) {
            klist[lane] = KeptEntry{ix, v};
            ls = (double)__builtin_amdgcn_exp2f(__builtin_fmaf(v, c, -mcc));
        }
    } else {
        int32_t npad = kWave;
        while (npad < nk) npad <<= 1;
        for (int32_t i = nk + lane; i < npad; i += kWave) {
            L.kidx[i] = INT32_MAX;
            L.kval[i] = neg_inf();
        }
        __builtin_amdgcn_wave_barrier();
        for (int32_t size = 2; size <= npad; size <<= 1) {
            for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (int32_t i = lane; i < npad; i += kWave) {
                    const int32_t p = i ^ stride;
                    if (p > i) {
                        const bool up = (i & size) == 0;
                        const int32_t a = L.kidx[i], bb = L.kidx[p];
                        if ((a > bb) == up) {
                            L.kidx[i] = bb;
                            L.kidx[p] = a;
                            const float tv = L.kval[i];
                            L.kval[i] = L.kval[p];
                            L.kval[p] = tv;
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
        for (int32_t i = lane; i < nk; i += kWave) {
            klist[i] = KeptEntry{L.kidx[i], L.kval[i]};
            ls += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(L.kval[i], c, -mcc));
        }
    }
    ls = wave_sum(ls);
    if (lane == 0) {
        RowDesc d;
        d.tau = K::value(h);
        d.m = lm;
        d.mcc = mcc;
        d.kept = nk;
        d.s = ls;
        d.flags = 0;
        d.pad = 0;
        descs[row] = d;
    }
}

// Visit a full row by one wave, 16-byte loads, kRowUnroll per lane in flight;
// fn(r0, f, ok) per block (r0: row index of the block's first element).
template <int DT, class F>
__device__ __forceinline__ void wave_row_blocks(const char* rowp, int32_t vocab, F&& fn)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    const uintptr_t addr = (uintptr_t)rowp;
    const int32_t mis = (int32_t)((addr & 15u) / ES);
    const u32x4* base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    const int32_t nblk = (mis + vocab + VEC - 1) / VEC;
    for (int32_t b0 = 0; b0 < nblk; b0 += kWave * kRowUnroll) {
        u32x4 raw[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int32_t j = b0 + u * kWave + lane_id();
            raw[u] = (j < nblk) ? load16<false>(base + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const int32_t j = b0 + u * kWave + lane_id();
            float f[VEC];
            bool ok[VEC];
            unpack<DT>(raw[u], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int32_t r = j * VEC - mis + e;
                ok[e] = j < nblk && r >= 0 && r < vocab;
            }
            fn(j * VEC - mis, f, ok);
        }
    }
}

// Exact path: radix select over the whole row, 8-bit digits from the top
// (one pass per digit), then the kept list by an ordered compaction (ascending
// ids) or, past the list capacity, the masked full-row description.
template <int DT>
__device__ void wave_select_exact(int32_t row, const char* rowp, int32_t vocab, int32_t top_k, float c,
                                  RowDesc* __restrict__ descs, KeptEntry* __restrict__ kept, WaveSelLds& L)
{
    const int lane = lane_id();
    constexpr int LOW = (DT == DT_BF16) ? 16 : 0;
    uint32_t prefix = 0, pmask = 0;
    int32_t kk = top_k, eq = 0;
    float rmax = neg_inf();
    for (int shift = 24; shift >= LOW; shift -= 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) L.hist[lane * 4 + q] = 0;
        __builtin_amdgcn_wave_barrier();
        wave_row_blocks<DT>(rowp, vocab, [&](int32_t, const float* f, const bool* ok) {
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e) {
                if (ok[e]) {
                    const uint32_t key = order_key(f[e]);
                    if ((key & pmask) == prefix) atomicAdd(&L.hist[(key >> shift) & 255u], 1u);
                    rmax = fmaxf(rmax, f[e]);
                }
            }
        });
        __builtin_amdgcn_wave_barrier();
        int c4[4], lsum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c4[q] = (int)L.hist[255 - 4 * lane - q];
            lsum += c4[q];
        }
        const int incl = wave_incl_scan_int(lsum);
        const int excl = incl - lsum;
        int found = -1, above = 0, cnt = 0;
        if (excl < kk && incl >= kk) {
            int cc = excl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (found < 0 && cc + c4[q] >= kk) {
                    found = 255 - 4 * lane - q;
                    above = cc;
                    cnt = c4[q];
                }
                cc += c4[q];
            }
        }
        const uint64_t bal = __ballot(found >= 0);
        const int src = bal ? __builtin_ctzll(bal) : 0;
        found = bal ? __shfl(found, src, kWave) : 0;
        above = bal ? __shfl(above, src, kWave) : 0;
        cnt = bal ? __shfl(cnt, src, kWave) : 0;
        prefix |= (uint32_t)found << shift;
        pmask |= 0xffu << shift;
        kk -= above;
        eq = cnt;
        __builtin_amdgcn_wave_barrier();
    }
    if (LOW > 0) prefix |= (prefix & 0x80000000u) ? 0u : ((1u << LOW) - 1u);
    const uint32_t tau_key = prefix;
    const float tau = key_to_float(tau_key);
    const int32_t nkept = (top_k - kk) + eq;
    const float m = __shfl(wave_max(rmax), 0, kWave);
    const float mcc = m * c;
    double ls = 0.0;
    RowDesc d;
    if (nkept <= kKeepCapList) {
        KeptEntry* klist = kept + (int64_t)row * kKeepCapList;
        int32_t base = 0;
        // lanes hold consecutive blocks: count per lane, prefix over the wave,
        // then each lane writes its block's kept ids in order
        wave_row_blocks<DT>(rowp, vocab, [&](int32_t r0, const float* f, const bool* ok) {
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e) cnt += (ok[e] && order_key(f[e]) >= tau_key) ? 1 : 0;
            const int incl = wave_incl_scan_int(cnt);
            int32_t pos = base + incl - cnt;
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e) {
                if (ok[e] && order_key(f[e]) >= tau_key) {
                    if (pos < kKeepCapList) klist[pos] = KeptEntry{r0 + e, f[e]};
                    ++pos;
                    ls += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
                }
            }
            base += __shfl(incl, kWave - 1, kWave);
        });
        d.kept = nkept;
    } else {
        wave_row_blocks<DT>(rowp, vocab, [&](int32_t, const float* f, const bool* ok) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < Dt<DT>::kVec; ++e)
                if (ok[e] && f[e] >= tau) s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
            ls += (double)s;
        });
        d.kept = -1;
    }
    ls = wave_sum(ls);
    if (lane == 0) {
        d.tau = tau;
        d.m = m;
        d.mcc = mcc;
        d.s = ls;
        d.flags = 1;
        d.pad = 0;
        descs[row] = d;
    }
}

// One wave per row.  use_cands = 0: every row takes the exact path.
template <int DT>
__global__ __launch_bounds__(kWave) void topk_select_wave_kernel(RowSet rs, int32_t vocab, int32_t nchunk,
                                                                 int32_t top_k, int32_t cap, float c,
                                                                 const int32_t* __restrict__ counts,
                                                                 const KeptEntry* __restrict__ cands,
                                                                 int32_t use_cands, RowDesc* __restrict__ descs,
                                                                 KeptEntry* __restrict__ kept)
{
    __shared__ WaveSelLds L;
    __shared__ int32_t s_choff[kMaxChunks + 1];
    const int32_t row = blockIdx.x;
    if (use_cands != 0) {
        int32_t base = 0, bad = 0;
        for (int32_t g = 0; g < nchunk; g += kWave) {
            const int32_t ch = g + lane_id();
            const int32_t n = ch < nchunk ? counts[(int64_t)row * nchunk + ch] : 0;
            bad |= n > cap;
            const int32_t nc = min(n, cap);
            const int incl = wave_incl_scan_int(nc);
            if (ch < nchunk) s_choff[ch] = base + incl - nc;
            base += __shfl(incl, kWave - 1, kWave);
        }
        if (lane_id() == 0) s_choff[nchunk] = base;
        __builtin_amdgcn_wave_barrier();
        if (__ballot(bad != 0) == 0 && base >= top_k && base <= kKeepCapList) {
            wave_select_fast<DT>(row, nchunk, top_k, cap, c, counts, cands, descs, kept, L, s_choff, base);
            return;
        }
    }
    wave_select_exact<DT>(row, row_ptr(rs, row), vocab, top_k, c, descs, kept, L);
}

}  // namespace sv
