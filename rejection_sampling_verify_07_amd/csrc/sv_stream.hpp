// Walk over the (row, chunk) tiles of the streaming passes.
//
// A chunk is kThreads * LOADS aligned 16-byte blocks of one row; tile c is
// chunk (c mod nchunk) of row (c / nchunk), and workgroup c takes tile c
// (one tile per workgroup: the hardware refills a finished workgroup's slot
// with the next tile, which overlapped the loads better than a persistent
// grid with the next tile's loads in flight, measured on MI355X).
#pragma once

#include "sv_common.hpp"

namespace sv {

// Every field is uniform across the workgroup (kept in scalar registers);
// a thread's first block is cb0 + threadIdx.x.
struct Tile {
    int32_t index;  // global tile index (row * nchunk + chunk)
    int32_t row;
    int32_t cb0;    // the tile's first block (aligned 16-byte units from the row's first block)
    int32_t mis;    // row start offset inside its first block, in elements
    int32_t nblk;   // blocks touched by the row
};

__device__ __forceinline__ int32_t tile_b0(const Tile& t) { return t.cb0 + (int32_t)threadIdx.x; }

template <int DT>
__device__ __forceinline__ Tile make_tile(const RowSet& rs, int32_t vocab, int32_t nchunk, int32_t c, int loads,
                                          const u32x4** base)
{
    constexpr int VEC = Dt<DT>::kVec;
    constexpr int ES = Dt<DT>::kSize;
    Tile t;
    t.index = c;
    t.row = (int32_t)((uint32_t)c / (uint32_t)nchunk);
    const int32_t chunk = c - t.row * nchunk;
    const uintptr_t addr = (uintptr_t)row_ptr(rs, t.row);
    t.mis = (int32_t)((addr & 15u) / ES);
    *base = reinterpret_cast<const u32x4*>(addr - (addr & 15u));
    t.nblk = (t.mis + vocab + VEC - 1) / VEC;
    t.cb0 = chunk * (kThreads * loads);
    return t;
}

template <int DT, int LOADS, bool NT>
__device__ __forceinline__ void issue_tile(const Tile& t, const u32x4* base, u32x4* raw)
{
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int32_t j = tile_b0(t) + i * kThreads;
        raw[i] = (j < t.nblk) ? load16<NT>(base + j) : u32x4{0u, 0u, 0u, 0u};
    }
}

// The tile of workgroup g.  With xcd > 1 the tiles of row r go to the
// workgroups g = r (mod xcd): the dispatcher deals workgroups to the XCDs in
// turn (MI355X: 8 XCDs), so all of a row's tiles run on one XCD, the one that
// also runs workgroup r of a per-row kernel launched next, which then finds
// the row's partial results in that XCD's L2.  The grid holds xcd *
// ceil(rows / xcd) * nchunk workgroups; -1 marks a padding workgroup.
__device__ __forceinline__ int32_t tile_of(int32_t g, int32_t ntiles, int32_t nchunk, int32_t xcd)
{
    if (xcd <= 1) return g < ntiles ? g : -1;
    const int32_t x = g % xcd, local = g / xcd;
    const int32_t row = (local / nchunk) * xcd + x;
    const int32_t c = row * nchunk + local % nchunk;
    return c < ntiles ? c : -1;
}

// body(tile, raw) is called once, by every thread of the workgroup, with the
// thread's LOADS raw words (which the body may overwrite).
template <int DT, int LOADS, bool NT, class Body>
__device__ __forceinline__ void walk_tiles(const RowSet& rs, int32_t vocab, int32_t nchunk, int32_t ntiles,
                                           Body&& body, int32_t xcd = 1)
{
    const int32_t c = tile_of((int32_t)blockIdx.x, ntiles, nchunk, xcd);
    if (c < 0) return;
    const u32x4* base;
    u32x4 raw[LOADS];
    const Tile t = make_tile<DT>(rs, vocab, nchunk, c, LOADS, &base);
    issue_tile<DT, LOADS, NT>(t, base, raw);
    body(t, raw);
}

// A plain read of nblk 16-byte blocks with the loads and tile shape of the
// streaming passes (LOADS loads per thread, one tile per workgroup): the
// practical roof they are measured against.  A thread writes `sink` only
// when the xor of its words equals `never`, which keeps the loads.
template <int LOADS>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, int64_t nblk,
                                                               uint32_t never, uint32_t* __restrict__ sink)
{
    const int64_t b0 = (int64_t)blockIdx.x * (kThreads * LOADS) + threadIdx.x;
    u32x4 raw[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int64_t j = b0 + (int64_t)i * kThreads;
        raw[i] = j < nblk ? load16<true>(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) x ^= raw[i].x ^ raw[i].y ^ raw[i].z ^ raw[i].w;
    if (x == never) *sink = x;
}

// Widen block i of a tile to fp32 and replace elements outside the row by
// `fill`.  The checks are branch-free selects (measured faster here than a
// per-block branch around them).
template <int DT>
__device__ __forceinline__ void tile_block(const Tile& t, const u32x4* raw, int i, int32_t vocab, float fill,
                                           float* f)
{
    constexpr int VEC = Dt<DT>::kVec;
    const int32_t j = tile_b0(t) + i * kThreads;
    unpack<DT>(raw[i], f);
    const int32_t r0 = j * VEC - t.mis;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const uint32_t r = (uint32_t)(r0 + e);
        f[e] = ((j < t.nblk) & (r < (uint32_t)vocab)) ? f[e] : fill;
    }
}

}  // namespace sv
