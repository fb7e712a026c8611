// Top-p (nucleus) filter, applied after temperature and top-k: the sampling
// filter that the "CS3602_FINAL_SpeDec" report's helpers name next to top-K
// (its module list, and its problem analysis, item 2).  The kept set shrinks
// to every id whose logit is >= tau_p, the largest logit value t for which
// the probability of {v : l_v >= t} reaches top_p (ties at tau_p kept whole),
// and the distribution is renormalised over it.  The row's maximum is always
// kept, so m and fl32(m c) do not change; the kernel rewrites the row
// descriptor (tau, S, kept count) and the kept list.
//
// One workgroup per row:
//  - a row with a kept list (<= 1024 ids) is done by wave 0 in registers: a
//    bitwise radix search on the select key, one wave-wide fp64 sum of the
//    fp32 weights per bit (fixed order), then an order-keeping compaction;
//  - a full row (no top-k, or a kept set that outgrew its list) takes two
//    reads of the row: a histogram of its weights over log-weight buckets,
//    which finds the bucket where the mass from the top reaches top_p; then
//    the entries of that bucket staged in LDS (and the ids above it counted)
//    and resolved by a mass-weighted radix select.  The kept count and mass
//    follow from those; only a kept set that fits the list takes a third
//    read, which writes the list in id order and sums the kept weights.
//    Weights are summed in 2^-43 fixed point with integer LDS atomics, so the
//    sums are exact and the result deterministic.
#pragma once

#include "sv_common.hpp"
#include "sv_select.hpp"
#include "sv_topk.hpp"

namespace sv {

struct NucArgs {
    RowSet rs;
    int32_t vocab;
    int32_t rows;
    float c;
    float top_p;
    const PartialFull* partials;  // full rows: the streaming pass's chunk partials
    int32_t nchunk;
    RowDesc* descs;                // in (top-k) / out
    KeptEntry* kept;               // in (top-k) / out, kKeepCap per row
};

constexpr double kFixScale = 8796093022208.0;  // 2^43: weights <= 1 summed over <= 2^20 ids stay below 2^63

// round(w 2^43) for a weight w in [0, 1] (ties to even): w 2^43 + 2^52 in one
// fp64 fma leaves that integer in the low mantissa bits, since w 2^43 < 2^52.
__device__ __forceinline__ uint64_t fix43(float w)
{
    const double x = __builtin_fma((double)w, kFixScale, 4503599627370496.0);
    return (uint64_t)__double_as_longlong(x) - 0x4330000000000000ull;
}

// Radix key of a logit for the full-row select: ordered like the logit, with
// the meaningful bits on top (16 of them for the 16-bit types).
template <int DT>
__device__ __forceinline__ uint32_t nuc_key(float v)
{
    if constexpr (DT == DT_F16) return SelKey<DT_F16>::of(v) << 16;
    else return order_key(v);
}
template <int DT>
__device__ __forceinline__ float nuc_value(uint32_t k)
{
    if constexpr (DT == DT_F32) return key_to_float(k);
    else return SelKey<DT>::value(k >> 16);
}

// Inclusive scan of a u64 across the wave (shuffles; once per digit).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, o, kWave);
        const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), o, kWave);
        if (lane_id() >= o) v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

// Sum of a u64 across the wave (butterfly; every lane gets it, exactly).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, kWave);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

// Kept-list rows: wave 0 alone.
template <int DT>
__device__ void nucleus_list(const NucArgs& a, int32_t row, const RowDesc& d)
{
    using K = SelKey<DT>;
    constexpr int PER = kKeepCap / kWave;
    const int lane = lane_id();
    KeptEntry* kl = a.kept + (int64_t)row * kKeepCap;
    const int32_t n = d.kept;
    KeptEntry e[PER];
    float w[PER];
    uint32_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int32_t i = j * kWave + lane;  // ascending i: j-major, then lane
        e[j] = i < n ? kl[i] : KeptEntry{INT32_MAX, neg_inf()};
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool ok = e[j].idx != INT32_MAX;
        w[j] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(e[j].val, a.c, -d.mcc)) : 0.0f;
        key[j] = ok ? K::of(e[j].val) : 0u;
    }
    const double target = (double)a.top_p * d.s;
    // the largest key h with sum{w : key >= h} >= target
    uint32_t h = 0;
    for (int bit = K::kBits - 1; bit >= 0; --bit) {
        const uint32_t cand = h | (1u << bit);
        double ls = 0.0;
#pragma unroll
        for (int j = 0; j < PER; ++j) ls += key[j] >= cand ? (double)w[j] : 0.0;
        const double mass = readlane_f64(wave_sum_dpp(ls), 0);
        if (mass >= target) h = cand;
    }
    // order-keeping compaction of the kept entries, in place (all loaded above)
    int32_t nk = 0;
    double ls = 0.0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool pred = e[j].idx != INT32_MAX && key[j] >= h;
        const uint64_t m = __ballot(pred);
        if (m != 0) {
            if (pred) {
                kl[nk + lanes_below(m)] = e[j];
                ls += (double)w[j];
            }
            nk += (int32_t)__popcll(m);
        }
    }
    ls = wave_sum_dpp(ls);
    if (lane == 0) {
        RowDesc o = d;
        o.tau = K::value(h);
        o.s = ls;
        o.kept = nk;
        a.descs[row] = o;
    }
}

// Mass-weighted radix select: the largest radix key h with
// sum{w : key >= h} >= need over the (key, fixed-point weight) pairs that
// visit(fn) presents, 8-bit digits from the top down to `low`.  All threads
// call it; integer sums make it exact and independent of visiting order.
template <class Visit>
__device__ uint32_t mass_radix(Visit&& visit, uint64_t need, int low, uint64_t* s_hist, uint64_t* s_u)
{
    uint32_t prefix = 0, pmask = 0;
    for (int shift = 24; shift >= low; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kThreads) s_hist[i] = 0;
        __syncthreads();
        visit([&](uint32_t k, uint64_t w) {
            if ((k & pmask) == prefix) atomicAdd((unsigned long long*)&s_hist[(k >> shift) & 255u], (unsigned long long)w);
        });
        __syncthreads();
        if (wave_id() == 0) {
            // lane L holds digits 255-4L .. 252-4L (descending)
            const int l = lane_id();
            uint64_t h4[4], lsum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                h4[q] = s_hist[255 - 4 * l - q];
                lsum += h4[q];
            }
            const uint64_t incl = wave_incl_scan_u64(lsum);
            const uint64_t excl = incl - lsum;
            int found = -1;
            uint64_t above = 0;
            if (excl < need && incl >= need) {
                uint64_t cum = excl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (found < 0 && cum + h4[q] >= need) {
                        found = 255 - 4 * l - q;
                        above = cum;
                    }
                    cum += h4[q];
                }
            }
            const uint64_t bal = __ballot(found >= 0);
            if (bal != 0) {
                const int src = __builtin_ctzll(bal);
                found = __shfl(found, src, kWave);
                above = (uint64_t)__shfl((long long)above, src, kWave);
            } else {
                found = 0;  // not reached (need <= the visited mass)
                above = 0;
            }
            if (l == 0) {
                s_u[0] = (uint64_t)found;
                s_u[1] = need - above;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_u[0] << shift;
        pmask |= 0xffu << shift;
        need = s_u[1];
        __syncthreads();
    }
    return prefix;
}

constexpr int kNucBuckets = 256;   // log-weight buckets of 1/8 bit below the row maximum
constexpr int kNucCap = 2048;      // entries of the crossing bucket staged in LDS

// The log-weight bucket of a logit, floor(8 (m - l) c) clamped to the
// buckets (the last one open-ended).  Every step is monotone, so the bucket
// never increases with the logit.
__device__ __forceinline__ uint32_t nuc_bucket(float l, float c, float mcc)
{
    const float e = -__builtin_fmaf(l, c, -mcc) * 8.0f;
    return (uint32_t)__builtin_amdgcn_fmed3f(e, 0.0f, (float)(kNucBuckets - 1));
}

// The smallest logit whose bucket is at most t (a binary search over the
// order keys from -inf to +inf; the bucket of +inf is 0).
__device__ __forceinline__ float nuc_lowest_at_most(uint32_t t, float c, float mcc)
{
    uint32_t lo = order_key(neg_inf()), hi = order_key(__int_as_float(0x7f800000));
    while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (nuc_bucket(key_to_float(mid), c, mcc) <= t) hi = mid;
        else lo = mid + 1;
    }
    return key_to_float(lo);
}

struct NucLds {
    uint64_t hist[256];
    uint64_t u[4];
    int32_t w[kWaves];
    double d[kWaves];
    uint32_t ck[kNucCap];
    uint64_t cw[kNucCap];
    int32_t n;
};

// The crossing bucket's radix select straight from the row, for a bucket
// too large to stage in LDS (kept out of line: it is rare and register-hungry).
template <int DT>
__device__ __attribute__((noinline)) uint32_t nucleus_bucket_radix(const char* rowp, int32_t vocab, float tau,
                                                                    float mcc, float c, uint32_t bstar,
                                                                    uint64_t need, uint64_t* s_hist, uint64_t* s_u)
{
    constexpr int LOW = Dt<DT>::kSize == 2 ? 16 : 0;
    return mass_radix(
        [&](auto&& fn) {
            for_row_blocks<DT>(rowp, vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
                for (int e = 0; e < Dt<DT>::kVec; ++e) {
                    if (ok[e] && f[e] >= tau && nuc_bucket(f[e], c, mcc) == bstar)
                        fn(nuc_key<DT>(f[e]), fix43(__builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc))));
                }
            });
        },
        need, LOW, s_hist, s_u);
}

// Full rows (kept set = {l >= d.tau}): the whole workgroup.  First a
// histogram of the fixed-point weights over log-weight buckets (bucket =
// floor(8 (m - l) c), the last one open-ended): it spreads a row over many
// buckets, so the integer LDS atomics rarely collide, and it finds the
// bucket where the mass from the top reaches top_p.  The bucket is
// monotone in the logit, so every higher bucket is kept whole and every lower
// one dropped.  Its own entries (a small share of the row) are staged in LDS
// by a second read and resolved by a mass-weighted radix select there; if
// they do not fit, the radix select reads the row instead.
template <int DT>
__device__ void nucleus_full(const NucArgs& a, int32_t row, const RowDesc& d, NucLds& S)
{
    constexpr int LOW = Dt<DT>::kSize == 2 ? 16 : 0;
    const char* rowp = row_ptr(a.rs, row);
    const float tau = d.tau, mcc = d.mcc, c = a.c;
    auto fixw = [&](float l) { return fix43(__builtin_amdgcn_exp2f(__builtin_fmaf(l, c, -mcc))); };
    auto bucket = [&](float l) { return nuc_bucket(l, c, mcc); };
    // 1. log-weight histogram
    for (int i = threadIdx.x; i < kNucBuckets; i += kThreads) S.hist[i] = 0;
    if (threadIdx.x == 0) S.n = 0;
    __syncthreads();
    for_row_blocks<DT>(rowp, a.vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e)
            if (ok[e] && f[e] >= tau)
                atomicAdd((unsigned long long*)&S.hist[bucket(f[e])], (unsigned long long)fixw(f[e]));
    });
    __syncthreads();
    if (wave_id() == 0) {
        // ascending buckets = descending weights; lane L holds buckets 4L .. 4L+3
        const int l = lane_id();
        uint64_t h4[4], lsum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h4[q] = S.hist[4 * l + q];
            lsum += h4[q];
        }
        const uint64_t incl = wave_incl_scan_u64(lsum);
        const uint64_t total = (uint64_t)__shfl((long long)incl, kWave - 1, kWave);
        uint64_t need = (uint64_t)((double)a.top_p * (double)total);
        if (need == 0) need = 1;  // at least the maximum is kept
        const uint64_t excl = incl - lsum;
        int found = -1;
        uint64_t above = 0;
        if (excl < need && incl >= need) {
            uint64_t cum = excl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (found < 0 && cum + h4[q] >= need) {
                    found = 4 * l + q;
                    above = cum;
                }
                cum += h4[q];
            }
        }
        const uint64_t bal = __ballot(found >= 0);
        const int src = bal != 0 ? __builtin_ctzll(bal) : 0;
        found = bal != 0 ? __shfl(found, src, kWave) : kNucBuckets - 1;
        above = bal != 0 ? (uint64_t)__shfl((long long)above, src, kWave) : 0;
        if (l == 0) {
            S.u[0] = (uint64_t)found;
            S.u[1] = need - above;
            S.u[2] = above;
        }
    }
    __syncthreads();
    const uint32_t bstar = (uint32_t)S.u[0];
    const uint64_t need_b = S.u[1];
    const uint64_t mass_hi = S.u[2];  // exact mass of the buckets above the crossing one
    __syncthreads();

    // 2. the crossing bucket's entries into LDS, and the count of the ids above
    // it, by the logit bounds of the bucket: l >= l_in is in or above it,
    // l >= l_above above it
    const float l_in = fmaxf(nuc_lowest_at_most(bstar, c, mcc), tau);
    const float l_above = bstar > 0 ? fmaxf(nuc_lowest_at_most(bstar - 1, c, mcc), tau) : __int_as_float(0x7f800000);
    int32_t n_hi = 0;
    for_row_blocks<DT>(rowp, a.vocab, [&](int32_t, int32_t, const float* f, const bool* ok) {
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e) {
            if (ok[e] && f[e] >= l_in) {
                const bool above = f[e] >= l_above;
                n_hi += above;
                if (!above) {
                    const int32_t slot = atomicAdd(&S.n, 1);
                    if (slot < kNucCap) {
                        S.ck[slot] = nuc_key<DT>(f[e]);
                        S.cw[slot] = fixw(f[e]);
                    }
                }
            }
        }
    });
    n_hi = wave_sum_int(n_hi);
    if (lane_id() == 0) S.w[wave_id()] = n_hi;
    __syncthreads();
    n_hi = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) n_hi += S.w[w];
    const int32_t nb = S.n;
    uint32_t prefix;
    if (nb <= kNucCap) {
        prefix = mass_radix(
            [&](auto&& fn) {
                for (int32_t i = threadIdx.x; i < nb; i += kThreads) fn(S.ck[i], S.cw[i]);
            },
            need_b, LOW, S.hist, S.u);
    } else {
        prefix = nucleus_bucket_radix<DT>(rowp, a.vocab, tau, mcc, c, bstar, need_b, S.hist, S.u);
    }
    int32_t* s_w = S.w;
    double* s_d = S.d;
    // the threshold value: the logit whose key has this prefix
    if constexpr (LOW > 0) prefix |= 0xffffu;
    const float tau_p = fmaxf(nuc_value<DT>(prefix), tau);

    // With the bucket staged, the kept count and mass follow without another
    // read: the ids above the crossing bucket, plus its staged entries >= tau_p
    // (exact fixed-point mass).  A kept set larger than the list needs nothing
    // more; the descriptor's S is that mass.
    if (nb <= kNucCap) {
        int32_t nk = 0;
        uint64_t mk = 0;
        for (int32_t i = threadIdx.x; i < nb; i += kThreads) {
            if (nuc_value<DT>(S.ck[i]) >= tau_p) {
                ++nk;
                mk += S.cw[i];
            }
        }
        nk = wave_sum_int(nk);
        mk = wave_sum_u64(mk);
        __syncthreads();  // every thread has read S.w and the staged entries
        if (lane_id() == 0) {
            S.w[wave_id()] = nk;
            S.hist[wave_id()] = mk;
        }
        __syncthreads();
        int32_t kept_n = n_hi;
        uint64_t kept_m = mass_hi;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            kept_n += S.w[w];
            kept_m += S.hist[w];
        }
        if (kept_n > kKeepCap) {
            if (threadIdx.x == 0) {
                RowDesc o = d;
                o.tau = tau_p;
                o.s = (double)kept_m / kFixScale;
                o.kept = -1;
                a.descs[row] = o;
            }
            return;
        }
        __syncthreads();  // S.w is the scan scratch below
    }

    // kept sum, count and (if it fits) the ordered kept list
    KeptEntry* kl = a.kept + (int64_t)row * kKeepCap;
    int32_t base = 0;
    double ls = 0.0;
    for_row_blocks<DT>(rowp, a.vocab, [&](int32_t, int32_t r0, const float* f, const bool* ok) {
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e) cnt += (ok[e] && f[e] >= tau_p);
        int tot;
        int pos = base + block_excl_scan_int(cnt, s_w, &tot);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < Dt<DT>::kVec; ++e) {
            if (ok[e] && f[e] >= tau_p) {
                if (pos < kKeepCap) kl[pos] = KeptEntry{r0 + e, f[e]};
                ++pos;
                s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, -mcc));
            }
        }
        ls += (double)s;
        base += tot;
    });
    const double sum = block_sum_double(ls, s_d);
    if (threadIdx.x == 0) {
        RowDesc o = d;
        o.tau = tau_p;
        o.s = sum;
        o.kept = base <= kKeepCap ? base : -1;
        a.descs[row] = o;
    }
}

template <int DT, bool FROM_DESC>
__global__ __launch_bounds__(kThreads) void nucleus_kernel(NucArgs a)
{
    __shared__ NucLds s_nuc;
    __shared__ RowDesc s_desc;
    const int32_t row = blockIdx.x;
    if constexpr (FROM_DESC) {
        if (threadIdx.x == 0) s_desc = a.descs[row];
    } else {
        // full rows: the row's statistics from the streaming pass's partials
        if (wave_id() == 0) {
            const PartialFull* pp = a.partials + (int64_t)row * a.nchunk;
            float m = neg_inf();
            for (int32_t ch = lane_id(); ch < a.nchunk; ch += kWave) m = fmaxf(m, pp[ch].m);
            m = wave_max_dpp(m);
            const float mcc = m * a.c;
            double s = 0.0;
            for (int32_t ch = lane_id(); ch < a.nchunk; ch += kWave) {
                const PartialFull q = pp[ch];
                if (q.s > 0.0) s += q.s * exp2((double)q.mcc - (double)mcc);
            }
            s = wave_sum_dpp(s);
            if (lane_id() == 0) {
                RowDesc d;
                d.tau = neg_inf();
                d.m = m;
                d.mcc = mcc;
                d.kept = -1;
                d.s = s;
                d.flags = 0;
                d.pad = 0;
                s_desc = d;
            }
        }
    }
    __syncthreads();
    const RowDesc d = s_desc;
    if (!(d.s > 0.0)) {  // no finite kept logit: the consumers report the row
        if (threadIdx.x == 0) a.descs[row] = d;
        return;
    }
    if (d.kept >= 0) {
        if (wave_id() == 0) nucleus_list<DT>(a, row, d);
    } else {
        nucleus_full<DT>(a, row, d, s_nuc);
    }
}

}  // namespace sv
