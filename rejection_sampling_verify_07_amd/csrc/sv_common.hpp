// Device-side building blocks shared by the specverify kernels (gfx950).
//
// Wavefronts are 64 lanes; every kernel runs 256-thread workgroups (4 waves,
// one per SIMD of a CU).  Logit rows are read in 16-byte vector loads
// (8 bf16 or 4 fp32 values); bf16 widens to fp32 exactly (the bf16 bits are
// the top half of the fp32 word).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT>
struct Dt;
template <>
struct Dt<DT_F32> {
    static constexpr int kSize = 4;
    static constexpr int kVec = 4;
};
// 16-bit types also carry the bit patterns the streaming passes write into
// out-of-row slots: -inf (ignored by every max and weight) and a quiet NaN
// (rejected by every compare).
template <>
struct Dt<DT_BF16> {
    static constexpr int kSize = 2;
    static constexpr int kVec = 8;
    static constexpr uint32_t kNegInf = 0xff80u;
    static constexpr uint32_t kNaN = 0x7fc0u;
};
template <>
struct Dt<DT_F16> {
    static constexpr int kSize = 2;
    static constexpr int kVec = 8;
    static constexpr uint32_t kNegInf = 0xfc00u;
    static constexpr uint32_t kNaN = 0x7e00u;
};

// IEEE binary16 bits -> fp32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// The low and high 16-bit element of a 32-bit word, widened to fp32.
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w)
{
    if constexpr (DT == DT_BF16) return __uint_as_float(w << 16);
    else return half_bits_to_float(w & 0xffffu);
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w)
{
    if constexpr (DT == DT_BF16) return __uint_as_float(w & 0xffff0000u);
    else return half_bits_to_float(w >> 16);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// ---------------------------------------------------------------------------
// Loads.  Row pointers reach the kernels inside by-value structs, where the
// compiler can no longer tell they are global memory and would emit FLAT
// instructions (which also occupy the LDS counter, so LDS work waits on HBM
// loads).  Casting to the global address space keeps them GLOBAL loads.
// ---------------------------------------------------------------------------
#define SV_GLOBAL __attribute__((address_space(1)))

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p)
{
    const SV_GLOBAL u32x4* g = (const SV_GLOBAL u32x4*)p;
    if constexpr (NT) {
        return __builtin_nontemporal_load(g);
    } else {
        return *g;
    }
}

// Widen one 16-byte block to kVec fp32 values.
template <int DT>
__device__ __forceinline__ void unpack(const u32x4 w, float* f)
{
    if constexpr (DT == DT_F32) {
        f[0] = __uint_as_float(w.x);
        f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z);
        f[3] = __uint_as_float(w.w);
    } else {
        f[0] = lo16<DT>(w.x);
        f[1] = hi16<DT>(w.x);
        f[2] = lo16<DT>(w.y);
        f[3] = hi16<DT>(w.y);
        f[4] = lo16<DT>(w.z);
        f[5] = hi16<DT>(w.z);
        f[6] = lo16<DT>(w.w);
        f[7] = hi16<DT>(w.w);
    }
}

// One element of a row, widened to fp32.
template <int DT>
__device__ __forceinline__ float load_one(const char* row, int64_t i)
{
    if constexpr (DT == DT_F32) {
        return ((const SV_GLOBAL float*)row)[i];
    } else {
        const uint32_t b = ((const SV_GLOBAL uint16_t*)row)[i];
        return lo16<DT>(b);
    }
}

// ---------------------------------------------------------------------------
// Monotone map float -> uint32 (a < b  <=>  key(a) < key(b), for non-NaN).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
}

// fp32 maximum of three with no NaN canonicalisation of the inputs.  The
// instruction ignores a quiet NaN operand and, in IEEE mode, turns a
// signalling one into a quiet NaN result; callers pass only finite values,
// -inf and quiet NaN fill patterns, so the result is the plain maximum of
// the non-NaN operands.  (fmaxf quiets every operand first: one extra
// instruction per input.)
__device__ __forceinline__ float max3_quiet(float a, float b, float c)
{
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// ---------------------------------------------------------------------------
// Wave primitives (64 lanes).  Reductions run a fixed butterfly, so the
// result is the same on every run; consumers take lane 0's copy.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return __shfl(v, 0, kWave);
}

__device__ __forceinline__ int wave_sum_int(int v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum over the lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_incl_scan(double v)
{
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(v, o, kWave);
        if (l >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_scan_int(int v)
{
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(v, o, kWave);
        if (l >= o) v += t;
    }
    return v;
}

// (value, index) arg-max with the lower index winning ties.
__device__ __forceinline__ void argmax_merge(float& v, int32_t& i, float ov, int32_t oi)
{
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int32_t& i)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, kWave);
        const int32_t oi = __shfl_xor(i, o, kWave);
        argmax_merge(v, i, ov, oi);
    }
}

// ---------------------------------------------------------------------------
// DPP reductions: data moves between lanes inside the VALU (quad permutes,
// row mirrors, row broadcasts) instead of through the LDS crossbar, which
// matters for the latency-bound one-wave-per-row passes.  The combine order
// is fixed; the result is read from lane 63 and returned wave-uniform.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_mov(int old, int v)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror, row_bcast:15 (into rows 1 and 3), row_bcast:31 (into rows 2, 3).
enum { kDppQuad1032 = 0xB1, kDppQuad2301 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
       kDppBcast15 = 0x142, kDppBcast31 = 0x143 };

__device__ __forceinline__ float wave_max_dpp(float v)
{
    const int ninf = __float_as_int(neg_inf());
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuad1032>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuad2301>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppHalfMirror>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppMirror>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppBcast15, 0xa>(ninf, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppBcast31, 0xc>(ninf, __float_as_int(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Wave-wide unsigned max and min, both returned wave-uniform (lane 63).
__device__ __forceinline__ void wave_umax_umin_dpp(uint32_t& mx, uint32_t& mn)
{
    int a = (int)mx, b = (int)mn;
#define SV_UMM_STEP(CTRL, RM)                                               \
    a = (int)max((uint32_t)a, (uint32_t)dpp_mov<CTRL, RM>(0, a));           \
    b = (int)min((uint32_t)b, (uint32_t)dpp_mov<CTRL, RM>(-1, b));
    SV_UMM_STEP(kDppQuad1032, 0xf)
    SV_UMM_STEP(kDppQuad2301, 0xf)
    SV_UMM_STEP(kDppHalfMirror, 0xf)
    SV_UMM_STEP(kDppMirror, 0xf)
    SV_UMM_STEP(kDppBcast15, 0xa)
    SV_UMM_STEP(kDppBcast31, 0xc)
#undef SV_UMM_STEP
    mx = (uint32_t)__builtin_amdgcn_readlane(a, kWave - 1);
    mn = (uint32_t)__builtin_amdgcn_readlane(b, kWave - 1);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_mov_f64(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const int lo = dpp_mov<CTRL, ROW_MASK>(0, (int)(uint32_t)b);
    const int hi = dpp_mov<CTRL, ROW_MASK>(0, (int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double wave_sum_dpp(double v)
{
    v += dpp_mov_f64<kDppQuad1032>(v);
    v += dpp_mov_f64<kDppQuad2301>(v);
    v += dpp_mov_f64<kDppHalfMirror>(v);
    v += dpp_mov_f64<kDppMirror>(v);
    v += dpp_mov_f64<kDppBcast15, 0xa>(v);
    v += dpp_mov_f64<kDppBcast31, 0xc>(v);
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, kWave - 1);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), kWave - 1);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes with DPP (fixed order): within each
// row of 16 the sums of 2, 3 and 4 neighbours, then shifts by 4 and 8; then
// the row totals are carried into rows 1 and 3 (row_bcast:15) and into rows 2
// and 3 (row_bcast:31).  Lanes whose source is outside the row add 0.
enum { kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr3 = 0x113, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118,
       kDppWaveShr1 = 0x138 };

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, BANK_MASK, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, BANK_MASK, true);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double wave_incl_scan_dpp(double v)
{
    double s = v + dpp_f64<kDppRowShr1, 0xf, 0xf>(v);
    s = s + dpp_f64<kDppRowShr2, 0xf, 0xf>(v);
    s = s + dpp_f64<kDppRowShr3, 0xf, 0xf>(v);
    s = s + dpp_f64<kDppRowShr4, 0xf, 0xe>(s);
    s = s + dpp_f64<kDppRowShr8, 0xf, 0xc>(s);
    s = s + dpp_f64<kDppBcast15, 0xa, 0xf>(s);
    s = s + dpp_f64<kDppBcast31, 0xc, 0xf>(s);
    return s;
}

// The same inclusive prefix sum for exact u64 sums (fixed-point masses).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t b)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, BANK_MASK, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, BANK_MASK, true);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64_dpp(uint64_t v)
{
    uint64_t s = v + dpp_u64<kDppRowShr1, 0xf, 0xf>(v);
    s = s + dpp_u64<kDppRowShr2, 0xf, 0xf>(v);
    s = s + dpp_u64<kDppRowShr3, 0xf, 0xf>(v);
    s = s + dpp_u64<kDppRowShr4, 0xf, 0xe>(s);
    s = s + dpp_u64<kDppRowShr8, 0xf, 0xc>(s);
    s = s + dpp_u64<kDppBcast15, 0xa, 0xf>(s);
    s = s + dpp_u64<kDppBcast31, 0xc, 0xf>(s);
    return s;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// The previous lane's value (0 in lane 0).
__device__ __forceinline__ double wave_prev_dpp(double v) { return dpp_f64<kDppWaveShr1, 0xf, 0xf>(v); }

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiplier S-box over a 4-word counter with a Weyl-incremented 2-word
// key.  Only output word 0 is needed here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                                 uint32_t k0, uint32_t k1)
{
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t a_hi = __umulhi(kMulA, x0), a_lo = kMulA * x0;
        const uint32_t b_hi = __umulhi(kMulB, x2), b_lo = kMulB * x2;
        const uint32_t y0 = b_hi ^ x1 ^ k0;
        const uint32_t y2 = a_hi ^ x3 ^ k1;
        x0 = y0;
        x1 = b_lo;
        x2 = y2;
        x3 = a_lo;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return x0;
}

// U(seq, pos, purpose) in [0, 1): 24 high bits of word 0, exact in fp32/fp64.
__device__ __forceinline__ double uniform24(uint64_t seed, uint32_t seq, uint32_t pos,
                                            uint32_t purpose, uint32_t offset)
{
    const uint32_t w = philox_word0(seq, pos, purpose, offset, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    return (double)(w >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------------------------
// Row addressing: rows [0, rows_t) are target rows, the rest draft rows.
// ---------------------------------------------------------------------------
struct RowSet {
    const char* tgt;
    const char* drf;
    int64_t t_stride_bytes;
    int64_t d_stride_bytes;
    int32_t rows_t;
};

__device__ __forceinline__ const char* row_ptr(const RowSet& rs, int32_t row)
{
    return row < rs.rows_t ? rs.tgt + (int64_t)row * rs.t_stride_bytes
                           : rs.drf + (int64_t)(row - rs.rows_t) * rs.d_stride_bytes;
}

// Per-(row, chunk) results of the streaming pass.
struct PartialFull {  // sampling: chunk max and sum of exp2(l*c - mcc) at the chunk's own max
    float m;
    float mcc;
    double s;
};
struct PartialArg {  // greedy: chunk max and its lowest index (row-relative)
    float m;
    int32_t idx;
};

// Per-row description used by the accept/resample pass.
struct RowDesc {
    float tau;      // kept set = { v : l_v >= tau } (-inf keeps every id)
    float m;        // largest kept logit
    float mcc;      // fl32(m * c), c = log2(e) / T in fp32
    int32_t kept;   // >= 0: number of entries in the row's kept list; -1: full row masked by tau
    double s;       // sum over kept v of exp2(fl32(l_v * c - mcc))
    int32_t flags;  // bit 0: candidate overflow took the exact full-row path; bit 1 (kDescTopP): top-p applied
    int32_t pad;
};

constexpr int32_t kDescTopP = 2;  // RowDesc.flags: the select already narrowed the kept set by top-p

struct KeptEntry {
    int32_t idx;
    float val;
};

// ---------------------------------------------------------------------------
// Hand-off between the workgroups of one kernel.  The L2 of each XCD is not
// coherent with the others', so data that one workgroup publishes for
// another travels in relaxed agent-scope atomic stores and loads (global
// store / load with sc1: written through to, and read from, the agent's
// point of coherence) rather than in plain stores, which a release fence
// would have to write back from L2 (buffer_wbl2) in every publishing
// workgroup.  Each publishing wave waits for its stores to complete
// (wait_stores) before the workgroup takes a ticket with an agent-scope
// atomic; the workgroup that takes the last ticket reads with agent loads
// only after its atomic has returned.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_agent_f64(double* p, double v)
{
    __hip_atomic_store((SV_GLOBAL uint64_t*)p, (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent_f64(const double* p)
{
    return __longlong_as_double(
        (long long)__hip_atomic_load((const SV_GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// An agent-scope atomic add that returns the previous value: a ticket.
__device__ __forceinline__ int32_t ticket_agent(int32_t* p)
{
    return __hip_atomic_fetch_add((SV_GLOBAL int32_t*)p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory operation this wave has issued is complete (stores written to
// their level of coherence); the compiler keeps memory operations on their
// side of it.
__device__ __forceinline__ void wait_stores()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Tickets sit 256 bytes apart, one cache line each, so that the atomics of
// different sequences do not contend for a line (measured: 32 tickets in
// one line cost 1.5 us per step at 10 arrivals each).
constexpr int kTicketStride = 64;

}  // namespace sv
