// Shared pieces of the prefill kernels that stream each selected block through
// LDS once per group of 16 consecutive query rows (forward attention and the
// row pass of its backward): the union of the rows' selected blocks (ascending
// list of distinct blocks and, per block, the mask of the rows that selected
// it) and the swizzled LDS tiles of a 64-key block.
#pragma once

#include "common.hpp"

namespace infv2 {

constexpr int kURows = 16;        // query rows per group
constexpr int kUWaves = 16;       // most waves of the thread blocks that build it
constexpr int kUThreads = kUWaves * 64;
constexpr int kUMaxWords = 512;   // bitmap words: up to 16384 blocks
constexpr int kUnionCap = 2048;   // union entries: 16 rows x top-k, top-k <= 128

// Union of the selected blocks of kRows consecutive rows (one wave per row),
// at most kCap entries.
template <int kRows, int kCap>
struct UnionSmemT {
    int32_t list[kCap];               // union of the rows' blocks, ascending (<= kRows * topk)
    uint32_t mask[kCap];              // which of the kRows rows selected each union block
    uint16_t order[kCap];             // balance_union scratch: the streaming order
    uint32_t bcount[2][kRows][5];     // balance_union: per-wave bucket counts, then their prefix
    uint32_t bsize[5];                // balance_union: bucket sizes
    uint32_t bits[kUMaxWords];
    uint32_t wbase[kUMaxWords];
    uint32_t scan_tmp[kUWaves + 1];
};
using UnionSmem = UnionSmemT<kURows, kUnionCap>;

// Called by all kThreads threads (kThreads >= 512, so that one bitmap word per
// thread covers 16384 blocks); returns the number of union blocks (the list and
// masks are valid after the call's final barrier).  Entries < 0 or >= nblk are
// ignored; rows >= rows_total contribute nothing.
template <int kThreads = kUThreads, int kRows, int kCap>
__device__ inline int build_union(UnionSmemT<kRows, kCap>& sm, const int32_t* __restrict__ idx,
                                  int rows_total, int r0, int hkv, int g, int topk, int64_t nblk) {
    static_assert(kThreads >= kUMaxWords && kThreads <= kUThreads && kThreads % 64 == 0, "threads");
    static_assert(kRows <= 32, "one mask bit per row");
    constexpr int kWaves = kThreads / 64;
    const int t = threadIdx.x;
    const int nwords = static_cast<int>((nblk + 31) / 32);
    for (int x = t; x < nwords; x += kThreads) sm.bits[x] = 0u;
    __syncthreads();
    const int nent = kRows * topk;
    for (int e = t; e < nent; e += kThreads) {
        const int row = r0 + e / topk;
        if (row >= rows_total) continue;
        const int32_t blk = idx[(static_cast<size_t>(row) * hkv + g) * topk + e % topk];
        if (blk >= 0 && blk < nblk) atomicOr(&sm.bits[blk >> 5], 1u << (blk & 31));
    }
    __syncthreads();
    const uint32_t word_t = t < nwords ? sm.bits[t] : 0u;      // one bitmap word per thread
    const uint32_t cnt_t = __popc(word_t);
    const uint32_t base_t = block_incl_scan<kWaves>(cnt_t, sm.scan_tmp) - cnt_t;
    if (t < nwords) {
        sm.wbase[t] = base_t;
        uint32_t bw = word_t, pos = base_t;
        while (bw) {
            const int bit = __ffs(bw) - 1;
            bw &= bw - 1;
            sm.list[pos] = t * 32 + bit;
            sm.mask[pos] = 0u;
            ++pos;
        }
    }
    if (t == kThreads - 1) sm.scan_tmp[kUWaves] = base_t + cnt_t;
    __syncthreads();
    const int n_u = static_cast<int>(sm.scan_tmp[kUWaves]);
    for (int e = t; e < nent; e += kThreads) {
        const int tok = e / topk, row = r0 + tok;
        if (row >= rows_total) continue;
        const int32_t blk = idx[(static_cast<size_t>(row) * hkv + g) * topk + e % topk];
        if (blk < 0 || blk >= nblk) continue;
        const uint32_t word = sm.bits[blk >> 5];
        const uint32_t pos = sm.wbase[blk >> 5] + __popc(word & ((1u << (blk & 31)) - 1u));
        atomicOr(&sm.mask[pos], 1u << tok);
    }
    __syncthreads();
    return n_u;
}

constexpr int kPB = 64;           // KV block size of the matrix-core prefill kernels

// LDS transpose read of 8 bytes per lane: inside each group of 16 lanes, lane i
// receives as its element e (e = 0..3) halfword i % 4 of the 8 bytes that lane
// 4 e + i / 4 addresses.
__device__ __forceinline__ uint2 lds_read_tr16(uint32_t byte_offset) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_s16x4*>(static_cast<uintptr_t>(byte_offset)));
    return __builtin_bit_cast(uint2, v);
}


// K / V tile: 64 keys x 16 chunks of 16 B; chunk c of key r sits at c ^ (r & 15),
// which makes 16-lane 16-byte column reads conflict-free.  Transposed operands
// (d along M, keys along K) are read from the same tile with lds_read_tr16.
typedef bf16_t BlockTile[kPB * kHeadDim];            // 16 KB

__device__ __forceinline__ uint4 k_frag(const BlockTile& t, int key, int chunk) {
    return *reinterpret_cast<const uint4*>(&t[key * kHeadDim + 8 * (chunk ^ (key & 15))]);
}

// Streaming order of the union that spreads each barrier interval's work over
// the SIMDs.  Wave w of the block runs on SIMD w % 4 and owns row w, so a
// block's work on SIMD s is the number of rows w = s (mod 4) in its mask.  Each
// block goes to the bucket of its busiest SIMD (a fifth bucket for blocks whose
// SIMD counts differ by at most one), and the buckets are interleaved round
// robin, so consecutive blocks -- the blocks of one interval -- load different
// SIMDs.  The order is stable within a bucket.  Called by all kThreads threads
// after build_union; on return list[] and mask[] hold the union in streaming
// order (order[] is scratch).
template <int kThreads = kUThreads, int kRows, int kCap>
__device__ inline void balance_union(UnionSmemT<kRows, kCap>& sm, int n_u) {
    constexpr int kWaves = kThreads / 64, kB = 5;
    static_assert(kThreads * 2 >= kCap, "two entries per thread at most");
    static_assert(kWaves == kRows && kRows % 4 == 0, "one row per wave, waves w and w + 4 on one SIMD");
    // rows on SIMD 0: 0, 4, 8, ...
    constexpr uint32_t kSimd0 = kRows == 4 ? 0x1u : kRows == 8 ? 0x11u : kRows == 12 ? 0x111u
                              : kRows == 16 ? 0x1111u : kRows == 20 ? 0x11111u : kRows == 24 ? 0x111111u
                              : kRows == 28 ? 0x1111111u : 0x11111111u;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int bk[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int u = rd * kThreads + t;
        int b = -1;
        if (u < n_u) {
            const uint32_t m = sm.mask[u];
            int best = 0, bc = __popc(m & kSimd0), mn = bc;
#pragma unroll
            for (int x = 1; x < 4; ++x) {
                const int c = __popc(m & (kSimd0 << x));
                if (c > bc) { bc = c; best = x; }
                mn = c < mn ? c : mn;
            }
            b = (bc - mn <= 1) ? 4 : best;
        }
        bk[rd] = b;
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            const uint64_t bal = __ballot(b == x);
            if (lane == 0) sm.bcount[rd][w][x] = static_cast<uint32_t>(__popcll(bal));
        }
    }
    __syncthreads();
    // exclusive prefix of the bucket counts over (round, wave), and the bucket sizes
    if (t < 5) {
        uint32_t run = 0;
        for (int rd = 0; rd < 2; ++rd)
            for (int y = 0; y < kWaves; ++y) {
                const uint32_t c = sm.bcount[rd][y][t];
                sm.bcount[rd][y][t] = run;
                run += c;
            }
        sm.bsize[t] = run;
    }
    __syncthreads();
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int u = rd * kThreads + t;
        const int b = bk[rd];
        uint32_t i = 0;                              // index of u inside its bucket
#pragma unroll
        for (int x = 0; x < kB; ++x) {
            const uint64_t bx = __ballot(b == x);
            if (b == x) i = sm.bcount[rd][w][x] + __popcll(bx & ((uint64_t(1) << lane) - 1));
        }
        if (u < n_u) {
            // round robin over the buckets: every bucket's items before index i,
            // then the buckets before b that still have an item i
            uint32_t pos = 0;
#pragma unroll
            for (int x = 0; x < kB; ++x) {
                const uint32_t nx = sm.bsize[x];
                pos += nx < i ? nx : i;
                if (x < b && nx > i) ++pos;
            }
            sm.order[pos] = static_cast<uint16_t>(u);
        }
    }
    __syncthreads();
    // apply the order: list[] and mask[] become the streaming order itself, so
    // a consumer finds block u with one LDS read
    int32_t bl[2];
    uint32_t bm[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int u = rd * kThreads + t;
        if (u < n_u) {
            const int o = sm.order[u];
            bl[rd] = sm.list[o];
            bm[rd] = sm.mask[o];
        }
    }
    __syncthreads();
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const int u = rd * kThreads + t;
        if (u < n_u) {
            sm.list[u] = bl[rd];
            sm.mask[u] = bm[rd];
        }
    }
    __syncthreads();
}

// Two-block barrier intervals (blocks 2 i and 2 i + 1): one pass of pairwise
// exchanges between intervals i and i + d (d = 1, 2, 3) that lowers the sum of
// the two intervals' costs.  An interval's cost is the largest SIMD load, with
// a wave that owns both blocks counted 1.6x per block (its two products run
// back to back); the exchange takes the cheaper of swapping the second blocks
// or swapping A's second block with B's first.  Intervals of one sub-pass are
// disjoint (i mod 2d < d, then >= d), so the threads do not race.  Called by all
// kThreads threads after balance_union; list[] and mask[] are updated in place.
template <int kThreads = kUThreads, int kRows, int kCap>
__device__ inline void refine_pairs(UnionSmemT<kRows, kCap>& sm, int n_u) {
    static_assert(kThreads * 2 >= kCap, "one interval per thread");
    constexpr uint32_t kSimd0 = kRows == 4 ? 0x1u : kRows == 8 ? 0x11u : kRows == 12 ? 0x111u
                              : kRows == 16 ? 0x1111u : kRows == 20 ? 0x11111u : kRows == 24 ? 0x111111u
                              : kRows == 28 ? 0x1111111u : 0x11111111u;
    auto cost = [](uint32_t a, uint32_t b) {   // 5 x (SIMD load), 8 x (2 products of one wave)
        uint32_t c = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t sx = kSimd0 << x;
            const uint32_t sum = 5u * (__popc(a & sx) + __popc(b & sx));
            const uint32_t two = (a & b & sx) ? 16u : (((a | b) & sx) ? 8u : 0u);
            const uint32_t v = sum > two ? sum : two;
            c = v > c ? v : c;
        }
        return c;
    };
    const int t = threadIdx.x;
    const int n_full = n_u / 2;                 // intervals with two blocks
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = t;
            if (i + d < n_full && (i % (2 * d)) / d == h) {
                const int pa = 2 * i, pb = 2 * (i + d);
                const uint32_t a0 = sm.mask[pa], a1 = sm.mask[pa + 1];
                const uint32_t b0 = sm.mask[pb], b1 = sm.mask[pb + 1];
                const uint32_t cur = cost(a0, a1) + cost(b0, b1);
                const uint32_t o1 = cost(a0, b1) + cost(b0, a1);   // swap the second blocks
                const uint32_t o2 = cost(a0, b0) + cost(a1, b1);   // swap A's second with B's first
                if (o1 < cur && o1 <= o2) {
                    const int32_t la = sm.list[pa + 1];
                    sm.list[pa + 1] = sm.list[pb + 1]; sm.mask[pa + 1] = b1;
                    sm.list[pb + 1] = la;              sm.mask[pb + 1] = a1;
                } else if (o2 < cur) {
                    const int32_t la = sm.list[pa + 1];
                    sm.list[pa + 1] = sm.list[pb]; sm.mask[pa + 1] = b0;
                    sm.list[pb] = la;              sm.mask[pb] = a1;
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace infv2
