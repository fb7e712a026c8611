// Per-row top-k selection, one workgroup of four waves per row: the four
// waves share the speculative path's survivor pass (one barrier), and every
// other step runs in one wave with no workgroup barrier.
//
// Input: the candidates the streaming pass wrote for each (row, chunk) (every
// chunk element >= a lower bound of the row's tau, so the candidate set holds
// the whole kept set), or nothing (then the row itself is scanned).
// Output: the row descriptor (tau = the top_k-th largest logit with
// multiplicity, the max, fl32(max * c), the sum of exp2 terms over the kept
// set) and the kept list sorted by id, or kept = -1 ("full row masked by
// tau") when the kept set is larger than the list capacity.
//
// Speculative path (every row of a typical call): only candidates >= the
// largest chunk bound can be kept; the four waves compact those survivors,
// then a ballot radix select over the top key bits finds tau without LDS
// atomics, and the kept entries are compacted with ballots, placed by rank
// (at most 64) or sorted by id with a register bitonic network.
// Chunk-list path (no chunk overflowed, top_k <= candidates <= kKeepCapList):
// the same select over every candidate, found by position.
// With top-p (top_p < 1) both paths also narrow the top-k set to its nucleus
// before writing it, and mark the descriptor (kDescTopP) so that the nucleus
// kernel leaves the row alone.
// Exact path: the same radix select with one pass over the whole row per
// 8-bit digit, then an ordered compaction of the row.
#pragma once

#include "sv_common.hpp"
#include "sv_topk.hpp"

namespace sv {

constexpr int kSelPer = kKeepCapList / kWave;  // candidates per lane on the fast path

// Keys the radix select works on: bf16 logits are fully ordered by the top
// 16 bits of their fp32 order key; fp16 logits by the same sign flip applied
// to their own 16 bits (a widened value narrows back exactly); fp32 needs
// all 32.
template <int DT>
struct SelKey {
    static constexpr int kBits = Dt<DT>::kSize == 2 ? 16 : 32;
    __device__ __forceinline__ static uint32_t of(float v)
    {
        if constexpr (DT == DT_BF16) {
            return order_key(v) >> 16;
        } else if constexpr (DT == DT_F16) {
            const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)v);
            return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
        } else {
            return order_key(v);
        }
    }
    // the logit value of a key (bf16: the low 16 key bits follow from the sign)
    __device__ __forceinline__ static float value(uint32_t k)
    {
        if constexpr (DT == DT_BF16) {
            return key_to_float((k << 16) | ((k & 0x8000u) ? 0u : 0xffffu));
        } else if constexpr (DT == DT_F16) {
            return half_bits_to_float((k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu));
        } else {
            return key_to_float(k);
        }
    }
};

// LDS scratch of one wave.
struct alignas(16) WaveSelLds {
    int32_t kidx[kKeepCapList];
    float kval[kKeepCapList];
    uint32_t hist[256];
};

// Bitonic sort of 64 * P (id, value) entries by ascending id, in the wave's
// registers: entry i = lane * P + r is slot r of lane `lane`.  Compare-and-
// exchange partners closer than P are in the same lane; farther ones are
// fetched from lane ^ (stride / P) with shuffles.  Ids are distinct except
// padding (INT32_MAX).
template <int P>
__device__ __forceinline__ void wave_bitonic_sort(int32_t (&id)[P], float (&val)[P])
{
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= kWave * P; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= P) {
                const int ls = stride / P;  // partner lane distance
                const bool lower = (lane & ls) == 0;
#pragma unroll
                for (int r = 0; r < P; ++r) {
                    const int32_t i = lane * P + r;
                    const bool up = (i & size) == 0;
                    const int32_t oid = __shfl_xor(id[r], ls, kWave);
                    const float ov = __shfl_xor(val[r], ls, kWave);
                    const bool take = (lower == up) ? (oid < id[r]) : (oid > id[r]);
                    if (take) {
                        id[r] = oid;
                        val[r] = ov;
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < P; ++r) {
                    const int r2 = r ^ stride;
                    if (r2 > r) {
                        const bool up = ((lane * P + r) & size) == 0;
                        if ((id[r] > id[r2]) == up) {
                            const int32_t ti = id[r];
                            id[r] = id[r2];
                            id[r2] = ti;
                            const float tv = val[r];
                            val[r] = val[r2];
                            val[r2] = tv;
                        }
                    }
                }
            }
        }
    }
}

// The nk kept entries staged in L.kidx / L.kval (nk <= 64 * P), sorted by id
// in registers and written to klist; returns the lane's fp64 sum of their
// exp2 weights.
template <int P>
__device__ __forceinline__ double sort_write_kept(WaveSelLds& L, int32_t nk, KeptEntry* klist, float c, float mcc)
{
    const int lane = lane_id();
    int32_t id[P];
    float val[P];
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const int32_t i = lane * P + r;
        id[r] = i < nk ? L.kidx[i] : INT32_MAX;
        val[r] = i < nk ? L.kval[i] : neg_inf();
    }
    wave_bitonic_sort<P>(id, val);
    double ls = 0.0;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const int32_t i = lane * P + r;
        if (i < nk) {
            klist[i] = KeptEntry{id[r], val[r]};
            ls += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(val[r], c, -mcc));
        }
    }
    return ls;
}

// The select proper, from NJ candidate slots per lane in registers (idx
// INT32_MAX marks an empty slot): tau by a ballot radix select, the kept
// entries compacted and sorted by id, their max and sum, the descriptor.
// NJ is a template argument so that every per-slot loop is unrolled without
// branches; select_tail picks the smallest NJ that holds the candidates.
template <int DT, int NJ>
__device__ __forceinline__ void select_tail_n(int32_t row, int32_t top_k, float c, float top_p, RowDesc* __restrict__ descs,
                              KeptEntry* __restrict__ kept, WaveSelLds& L, const KeptEntry* e)
{
    using K = SelKey<DT>;
    const int lane = lane_id();
    uint32_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = (e[j].idx != INT32_MAX) ? K::of(e[j].val) : 0u;

    // ballot radix select: the largest h with #{key >= h} >= top_k
    uint32_t h = 0;
#pragma unroll
    for (int bit = K::kBits - 1; bit >= 0; --bit) {
        const uint32_t cand = h | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) cnt += (int)__popcll(__ballot(key[j] >= cand));
        h = cnt >= top_k ? cand : h;
    }

    // top-p after top-k: among the top-k set (key >= h), the largest key hp
    // whose entries at or above it hold top_p of the set's mass, by the same
    // bitwise search, fp32 weights and fp64 wave sums as the kept-list path
    // of the nucleus kernel (which then leaves the row alone).  The row's
    // maximum stays kept, so its reference mcc is the top-k set's.  A set
    // with no finite logit is left unfiltered, for the consumers to report.
    bool nucleus = false;
    float m0 = neg_inf();
    if (top_p < 1.0f) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (key[j] >= h && e[j].idx != INT32_MAX) m0 = fmaxf(m0, e[j].val);
        m0 = wave_max_dpp(m0);
        nucleus = m0 != neg_inf();
    }
    if (nucleus) {
        const float mcc0 = m0 * c;
        float w[NJ];
        double s0 = 0.0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            w[j] = (key[j] >= h && e[j].idx != INT32_MAX) ? __builtin_amdgcn_exp2f(__builtin_fmaf(e[j].val, c, -mcc0))
                                                          : 0.0f;
            s0 += (double)w[j];
        }
        const double target = (double)top_p * wave_sum_dpp(s0);
        // the cut lies in [h, key of the maximum]: the bits above the highest
        // one where those two differ are the cut's too
        const uint32_t kmax = K::of(m0);
        if (kmax != h) {
            const int top = 31 - __builtin_clz(kmax ^ h);
            uint32_t hp = h & ~((2u << top) - 1u);
            for (int bit = top; bit >= 0; --bit) {
                const uint32_t cand = hp | (1u << bit);
                double ls = 0.0;
#pragma unroll
                for (int j = 0; j < NJ; ++j) ls += key[j] >= cand ? (double)w[j] : 0.0;
                if (wave_sum_dpp(ls) >= target) hp = cand;
            }
            h = hp;  // >= the top-k h: the whole set's mass reaches the target
        }
    }

    // kept entries (key >= h), compacted in candidate order
    int32_t nk = 0;
    float lm = neg_inf();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool pred = key[j] >= h && e[j].idx != INT32_MAX;
        const uint64_t m = __ballot(pred);
        if (m != 0) {
            if (pred) {
                const int32_t pos = nk + lanes_below(m);
                L.kidx[pos] = e[j].idx;
                L.kval[pos] = e[j].val;
                lm = fmaxf(lm, e[j].val);
            }
            nk += (int32_t)__popcll(m);
        }
    }
    lm = wave_max_dpp(lm);
    const float mcc = lm * c;

    KeptEntry* klist = kept + (int64_t)row * kKeepCapList;
    double ls = 0.0;
    if (nk <= kWave) {
        // one kept entry per lane; its place in the id-sorted list is the
        // number of kept ids below its own (ids are distinct), counted from
        // 16 broadcast LDS reads of four ids each (slots past nk hold INT32_MAX)
        if (lane >= nk) L.kidx[lane] = INT32_MAX;
        __builtin_amdgcn_wave_barrier();
        const int32_t ix = L.kidx[lane];
        const float v = lane < nk ? L.kval[lane] : neg_inf();
        const int4* k4 = reinterpret_cast<const int4*>(L.kidx);
        int4 q[kWave / 4];
#pragma unroll
        for (int j = 0; j < kWave / 4; ++j) q[j] = k4[j];
        int32_t rank = 0;
#pragma unroll
        for (int j = 0; j < kWave / 4; ++j) rank += (q[j].x < ix) + (q[j].y < ix) + (q[j].z < ix) + (q[j].w < ix);
        if (lane < nk) {
            klist[rank] = KeptEntry{ix, v};
            ls = (double)__builtin_amdgcn_exp2f(__builtin_fmaf(v, c, -mcc));
        }
    } else {
        // more than one per lane: a register bitonic sort of the next power of two
        __builtin_amdgcn_wave_barrier();
        if (nk <= 2 * kWave) ls = sort_write_kept<2>(L, nk, klist, c, mcc);
        else if (nk <= 4 * kWave) ls = sort_write_kept<4>(L, nk, klist, c, mcc);
        else if (nk <= 8 * kWave) ls = sort_write_kept<8>(L, nk, klist, c, mcc);
        else ls = sort_write_kept<16>(L, nk, klist, c, mcc);
    }
    ls = wave_sum_dpp(ls);
    if (lane == 0) {
        RowDesc d;
        d.tau = K::value(h);
        d.m = lm;
        d.mcc = mcc;
        d.kept = nk;
        d.s = ls;
        d.flags = nucleus ? kDescTopP : 0;
        d.pad = 0;
        descs[row] = d;
    }
}

// e[0 .. nj) hold the candidates (nj wave-uniform, at most kSelPer).
template <int DT>
__device__ void select_tail(int32_t row, int32_t top_k, float c, float top_p, RowDesc* __restrict__ descs,
                            KeptEntry* __restrict__ kept, WaveSelLds& L, const KeptEntry* e, int32_t nj)
{
    if (nj <= 1) {
        select_tail_n<DT, 1>(row, top_k, c, top_p, descs, kept, L, e);
    } else if (nj <= 2) {
        select_tail_n<DT, 2>(row, top_k, c, top_p, descs, kept, L, e);
    } else if (nj <= 4) {
        select_tail_n<DT, 4>(row, top_k, c, top_p, descs, kept, L, e);
    } else if (nj <= 8) {
        select_tail_n<DT, 8>(row, top_k, c, top_p, descs, kept, L, e);
    } else {
        select_tail_n<DT, kSelPer>(row, top_k, c, top_p, descs, kept, L, e);
    }
}

// Candidates by global position: the row's chunks hold counts[ch] entries
// each, choff their exclusive prefix sums (in LDS); candidate i is found by a
// binary search over choff.
template <int DT>
__device__ __attribute__((noinline)) void wave_select_fast(int32_t row, int32_t nchunk, int32_t top_k, int32_t cap, float c, float top_p,
                                 const KeptEntry* __restrict__ cands, RowDesc* __restrict__ descs,
                                 KeptEntry* __restrict__ kept, WaveSelLds& L, const int32_t* choff, int32_t total)
{
    const int lane = lane_id();
    const int32_t nj = (total + kWave - 1) / kWave;  // wave-uniform
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
    select_tail<DT>(row, top_k, c, top_p, descs, kept, L, e, nj);
}

// Speculative path, kSelWaves waves per row.  Every chunk bound is a lower
// bound of the row's tau, so only candidates >= their maximum can be kept.
// Each wave reads every count and bound itself (one lane per chunk, 64
// chunks per round), so each knows the largest bound and whether a chunk
// overflowed; wave w then takes the contiguous chunks [w C, (w + 1) C),
// C = ceil(nchunk / kSelWaves), kSpecChunks at a time with the first
// kSpecSlots * 64 slots of each loaded at once (the first batch in flight
// with the counts and bounds) and the rare slots past them kSpecExtra rounds
// at a time, and compacts its survivors in chunk order into an LDS region
// of its own, which holds a whole kept list (survivors need not spread
// evenly over the waves).  Region after region, that is the row's
// chunk order.  After one barrier wave 0 runs the select over them.  Returns
// false (the same in every wave), having written nothing, when a chunk
// overflowed or the survivors do not fit the kept list.
constexpr int kSelWaves = 4;
constexpr int kSelRegion = kKeepCapList;  // survivors a wave can hold

// Survivor regions of the speculative path (32 KB).
struct alignas(16) SpecLds {
    int32_t idx[kSelWaves * kSelRegion];
    float val[kSelWaves * kSelRegion];
};
constexpr int kSpecChunks = 4;
constexpr int kSpecSlots = 2;
constexpr int kSpecExtra = 6;  // slot rounds past kSpecSlots loaded at once (512 slots: all of them)

// The select over the n survivors held in the waves' LDS regions (region v
// holds off[v + 1] - off[v] of them), in region order; n <= NJ * 64.
template <int DT, int NJ>
__device__ __forceinline__ void select_from_regions(int32_t row, int32_t top_k, float c, float top_p, RowDesc* __restrict__ descs,
                                                    KeptEntry* __restrict__ kept, WaveSelLds& L, const SpecLds& R,
                                                    const int32_t* off, int32_t n)
{
    KeptEntry r[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int32_t i = lane_id() + j * kWave;
        int32_t at = i;  // region 0
#pragma unroll
        for (int u = 1; u < kSelWaves; ++u)
            if (i >= off[u]) at = u * kSelRegion + (i - off[u]);
        r[j] = i < n ? KeptEntry{R.idx[at], R.val[at]} : KeptEntry{INT32_MAX, neg_inf()};
    }
    select_tail_n<DT, NJ>(row, top_k, c, top_p, descs, kept, L, r);
}

template <int DT>
__device__ __forceinline__ bool select_spec(int32_t row, int32_t nchunk, int32_t top_k, int32_t cap, float c, float top_p,
                                            const int32_t* __restrict__ counts, const float* __restrict__ bounds,
                                            const KeptEntry* __restrict__ cands, RowDesc* __restrict__ descs,
                                            KeptEntry* __restrict__ kept, WaveSelLds& L, SpecLds& R, int32_t* s_wn)
{
    const int lane = lane_id();
    const int w = wave_id();
    const int64_t t0 = (int64_t)row * nchunk;
    const int32_t C = (nchunk + kSelWaves - 1) / kSelWaves;
    const int32_t cb = min(nchunk, w * C), ce = min(nchunk, cb + C);  // this wave's chunks
    int32_t cnt_l = lane < nchunk ? counts[t0 + lane] : 0;  // chunk `lane` of the first 64
    float bnd_l = lane < nchunk ? bounds[t0 + lane] : neg_inf();
    // the first batch of this wave's candidate slots in flight with the counts and bounds
    KeptEntry e[kSpecChunks][kSpecSlots];
    int32_t cnt_b = lane < kSpecChunks && cb + lane < ce ? counts[t0 + cb + lane] : 0;  // lane ch: chunk c0 + ch
#pragma unroll
    for (int ch = 0; ch < kSpecChunks; ++ch) {
#pragma unroll
        for (int q = 0; q < kSpecSlots; ++q) {
            e[ch][q] = cb + ch < ce ? cands[(t0 + cb + ch) * cap + q * kWave + lane] : KeptEntry{INT32_MAX, neg_inf()};
        }
    }
    bool over = cnt_l > cap;
    for (int32_t g = kWave; g < nchunk; g += kWave) {
        const int32_t ch = g + lane;
        if (ch < nchunk) {
            over |= counts[t0 + ch] > cap;
            bnd_l = fmaxf(bnd_l, bounds[t0 + ch]);
        }
    }
    if (__ballot(over) != 0) return false;
    const float bmax = wave_max_dpp(bnd_l);

    // survivors (candidate >= the largest chunk bound) of this wave's chunks,
    // compacted in chunk order into region w
    const int32_t rbase = w * kSelRegion;
    int32_t ns = 0;
    auto keep = [&](const KeptEntry& x, bool valid) {
        const bool pred = valid && x.val >= bmax;
        const uint64_t m = __ballot(pred);
        if (m != 0) {
            const int32_t pos = ns + lanes_below(m);
            if (pred && pos < kSelRegion) {
                R.idx[rbase + pos] = x.idx;
                R.val[rbase + pos] = x.val;
            }
            ns += (int32_t)__popcll(m);
        }
    };
    for (int32_t c0 = cb; c0 < ce; c0 += kSpecChunks) {
        if (c0 > cb) {
#pragma unroll
            for (int ch = 0; ch < kSpecChunks; ++ch) {
#pragma unroll
                for (int q = 0; q < kSpecSlots; ++q) {
                    e[ch][q] = c0 + ch < ce ? cands[(t0 + c0 + ch) * cap + q * kWave + lane]
                                            : KeptEntry{INT32_MAX, neg_inf()};
                }
            }
            cnt_b = lane < kSpecChunks && c0 + lane < ce ? counts[t0 + c0 + lane] : 0;
        }
#pragma unroll
        for (int ch = 0; ch < kSpecChunks; ++ch) {
            if (c0 + ch < ce) {
                const int32_t cnt = __builtin_amdgcn_readlane(cnt_b, ch);
#pragma unroll
                for (int q = 0; q < kSpecSlots; ++q) keep(e[ch][q], q * kWave + lane < cnt);
                // slots past the first batch (at most cap), kSpecExtra rounds of
                // loads in flight together
                for (int32_t q0 = kSpecSlots; q0 * kWave < cnt; q0 += kSpecExtra) {
                    KeptEntry x[kSpecExtra];
#pragma unroll
                    for (int u = 0; u < kSpecExtra; ++u) {
                        const int32_t i = (q0 + u) * kWave + lane;
                        x[u] = i < cnt ? cands[(t0 + c0 + ch) * cap + i] : KeptEntry{INT32_MAX, neg_inf()};
                    }
#pragma unroll
                    for (int u = 0; u < kSpecExtra; ++u) keep(x[u], (q0 + u) * kWave + lane < cnt);
                }
            }
        }
    }
    if (lane == 0) s_wn[w] = ns;
    __syncthreads();
    int32_t off[kSelWaves + 1];
    int32_t tot = 0;
    bool fit = true;
#pragma unroll
    for (int v = 0; v < kSelWaves; ++v) {
        off[v] = tot;
        tot += s_wn[v];
        fit = fit && s_wn[v] <= kSelRegion;
    }
    off[kSelWaves] = tot;
    if (!fit || tot < top_k || tot > kKeepCapList) return false;
    if (w != 0) return true;
    const int32_t nj = (tot + kWave - 1) / kWave;
    if (nj <= 1) {
        select_from_regions<DT, 1>(row, top_k, c, top_p, descs, kept, L, R, off, tot);
    } else if (nj <= 2) {
        select_from_regions<DT, 2>(row, top_k, c, top_p, descs, kept, L, R, off, tot);
    } else if (nj <= 4) {
        select_from_regions<DT, 4>(row, top_k, c, top_p, descs, kept, L, R, off, tot);
    } else if (nj <= 8) {
        select_from_regions<DT, 8>(row, top_k, c, top_p, descs, kept, L, R, off, tot);
    } else {
        select_from_regions<DT, kSelPer>(row, top_k, c, top_p, descs, kept, L, R, off, tot);
    }
    return true;
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
__device__ __attribute__((noinline)) void wave_select_exact(int32_t row, const char* rowp, int32_t vocab, int32_t top_k, float c,
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

// The select of one row by one wave: the speculative path, else the
// chunk-list path, else the exact path over the full row.  Returns true (in
// every wave) when the speculative path wrote the row; false when wave 0
// took one of the others (the other waves return at once).
template <int DT>
__device__ __forceinline__ bool select_row_wave(const RowSet& rs, int32_t row, int32_t vocab, int32_t nchunk, int32_t top_k,
                                int32_t cap, float c, float top_p, const int32_t* __restrict__ counts,
                                const float* __restrict__ bounds, const KeptEntry* __restrict__ cands,
                                RowDesc* __restrict__ descs, KeptEntry* __restrict__ kept, WaveSelLds& L,
                                SpecLds& R, int32_t* s_choff, int32_t* s_wn)
{
    if (select_spec<DT>(row, nchunk, top_k, cap, c, top_p, counts, bounds, cands, descs, kept, L, R, s_wn)) return true;
    if (wave_id() != 0) return false;  // the paths below are one wave's
    // every wave has passed the barrier of the speculative path (or none has),
    // so wave 0 alone may reuse the LDS from here
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
        wave_select_fast<DT>(row, nchunk, top_k, cap, c, top_p, cands, descs, kept, L, s_choff, base);
        return false;
    }
    wave_select_exact<DT>(row, row_ptr(rs, row), vocab, top_k, c, descs, kept, L);
    return false;
}

// The top-p narrowing of one top-k row by kThreads threads (the nucleus
// kernel's per-row steps; defined with them).  lds: at least the nucleus's
// LDS, 16-byte aligned.
template <int DT>
__device__ __attribute__((noinline)) void nucleus_topk_row(RowSet rs, int32_t vocab, float c, float top_p,
                                                           RowDesc* __restrict__ descs, KeptEntry* __restrict__ kept,
                                                           int32_t row, void* lds);

// One workgroup of kSelWaves waves per row, over the candidates of the top-k
// streaming pass.  TOPP: top_p < 1 narrows the kept sets it writes (without
// it the top-p code is compiled out): the speculative and chunk-list paths
// do it on the set in registers; a row the exact path wrote is narrowed
// after it by the whole workgroup, in the speculative path's LDS.
template <int DT, bool TOPP>
__global__ __launch_bounds__(kSelWaves * kWave) void topk_select_wave_kernel(RowSet rs, int32_t vocab, int32_t nchunk,
                                                                 int32_t top_k, int32_t cap, float c, float top_p,
                                                                 const int32_t* __restrict__ counts,
                                                                 const float* __restrict__ bounds,
                                                                 const KeptEntry* __restrict__ cands,
                                                                 RowDesc* __restrict__ descs,
                                                                 KeptEntry* __restrict__ kept)
{
    __shared__ WaveSelLds L;
    __shared__ int32_t s_choff[kMaxChunks + 1];
    __shared__ SpecLds R;
    __shared__ int32_t s_wn[kSelWaves];
    const bool spec = select_row_wave<DT>(rs, (int32_t)blockIdx.x, vocab, nchunk, top_k, cap, c, TOPP ? top_p : 1.0f,
                                          counts, bounds, cands, descs, kept, L, R, s_choff, s_wn);
    if constexpr (TOPP) {
        if (spec) return;  // (the same in every wave)
        __syncthreads();   // wave 0's descriptor and kept list are written
        nucleus_topk_row<DT>(rs, vocab, c, top_p, descs, kept, (int32_t)blockIdx.x, &R);
    }
}

}  // namespace sv
