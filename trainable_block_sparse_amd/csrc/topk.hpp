// Block-wide top-k selection with forced blocks, for one (query row, KV head).
// MiniCPM4 summary page, "InfLLM v2" section: paragraph "Top-K implementation
// and the LSE bottleneck" (select the K blocks with the highest group score)
// and paragraph "Initial and local tokens always selected" (block 0 and the
// local window are always kept; shorter than k*m degenerates to dense).
//
// Candidates are the blocks 0..c that are not forced.  Scores arrive as sortable
// 32-bit keys (score_to_key).  Thread t owns the contiguous blocks
// [t*per, t*per + per) and holds their keys in registers for the whole
// selection.  The k' = k - |F| largest keys, ties to the lower block, are
// found by narrowing a key window [lo, hi]:
//   1. lo, hi = min and max candidate key;
//   2. histogram of the candidates in the window over at most 1024 bins of
//      2^sh consecutive key values (sh chosen so the window fits), which
//      adapts to the data: the bins spread even when every score shares its
//      exponent;
//   3. the bin holding the k'-th largest key becomes the new window; every key
//      above it is taken.
// The loop stops when the window's keys are all needed, when the window holds
// at most kThreads keys (each is then ranked against the others by (key desc,
// block asc)), or when the window is a single key value (the lowest blocks are
// taken).  Each step shrinks the window by 2^10 (a 32-bit key range needs at
// most four steps; typical inputs need one).  The ascending output needs one
// block scan because ownership is contiguous.  Barriers: one for the min / max,
// two per narrowing step, three for the rank step, one for the output scan.
// A caller that only needs to find given slots of the selection can take it
// as a bitmap instead (kBitmap: bit j = block j, set with one LDS atomic OR per
// thread, no output scan), read with wave-level popcounts (BitmapLanes).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace infv2 {

constexpr int kTopkBins = 1024;

template <int kThreads>
struct TopkSmem {
    uint32_t hist[kTopkBins];
    uint32_t scan_tmp[3][kThreads / 64];   // wave totals: narrowing, window, output scans
    uint32_t rmin[kThreads / 64], rmax[kThreads / 64];
    uint32_t ckey[kThreads + 4] __attribute__((aligned(16)));   // the window's keys (rank step)
    int32_t cidx[kThreads + 4] __attribute__((aligned(16)));    // and their blocks
    uint32_t keep[kThreads];        // and whether each is taken
    uint32_t bstar, above, ebin;
};

// keys per thread held in registers for a block of kThreads and nblk blocks
__host__ __device__ constexpr int topk_per(int64_t nblk, int threads) {
    return static_cast<int>((nblk + threads - 1) / threads);
}
// the register-array sizes the top-k kernels are built for: the smallest one
// that holds `per` keys
__host__ __device__ constexpr int topk_kper(int per) {
    return per <= 2 ? 2 : per <= 8 ? 8 : per <= 16 ? 16 : 64;
}

// words of the selection bitmap for kThreads threads of kPer blocks
__host__ __device__ constexpr int topk_bm_words(int threads, int per) { return (threads * per + 31) / 32; }

// key[u] is the key of block jb + u for u < cnt (cnt = valid blocks of this
// thread, 0 if none).  Must be called by all kThreads threads of the block.
// Writes idx[k] ascending, padded with -1 (and score[k] if non-null); with
// kBitmap, instead sets bit j of the LDS words bits[] (cleared here) for every
// selected block j, and the caller's barrier makes them visible (no ordered
// output scan).
template <int kThreads, int kPer, bool kBitmap = false, typename Smem>
__device__ inline void block_topk_regs(const uint32_t (&key)[kPer], int jb, int cnt, int c, int k,
                                       int init, int local, int32_t* __restrict__ idx,
                                       float* __restrict__ score, Smem& sm,
                                       uint32_t* __restrict__ bits = nullptr) {
    static_assert(kThreads % 64 == 0 && kThreads <= kTopkBins && kTopkBins % kThreads == 0,
                  "block size");
    static_assert(kPer <= 64, "at most 64 keys per thread");
    using Mask = typename std::conditional<(kPer > 32), uint64_t, uint32_t>::type;
    constexpr int kWaves = kThreads / 64;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int nb = c + 1;
    const float kNaN = __uint_as_float(0x7fc00000u);
    static_assert(!kBitmap || (kPer <= 32 && 32 % kPer == 0), "a thread's blocks lie in one bitmap word");
    if constexpr (kBitmap) {
        for (int x = t; x < topk_bm_words(kThreads, kPer); x += kThreads) bits[x] = 0;
        if (nb <= k) {                  // dense: every block
            __syncthreads();            // orders the clearing
            const uint32_t all = cnt > 0 ? (cnt >= 32 ? 0xffffffffu : (1u << cnt) - 1u) : 0u;
            if (all != 0u) atomicOr(&bits[jb >> 5], all << (jb & 31));
            return;
        }
    }
    if (nb <= k) {                      // dense: every block, then -1 padding
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (u < cnt) {
                idx[jb + u] = jb + u;
                if (score) score[jb + u] = key_to_score(key[u]);
            }
        }
        for (int r = nb + t; r < k; r += kThreads) {
            idx[r] = -1;
            if (score) score[r] = kNaN;
        }
        return;
    }
    const int a = init < nb ? init : nb;
    const int lo_loc = c - local + 1 > 0 ? c - local + 1 : 0;
    const int nforced = a + (nb - (lo_loc > a ? lo_loc : a));
    const uint32_t kp = static_cast<uint32_t>(k - nforced);
    // candidate mask of this thread's blocks
    Mask cmask = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int j = jb + u;
        if (u < cnt && j >= init && j <= c - local) cmask |= Mask(1) << u;
    }
    auto cand = [&](int u) { return ((cmask >> u) & 1u) != 0; };

    // window [lo, hi] of undecided keys; keys above hi are taken.
    // mode: 0 = take every candidate in the window, 1 = rank the window,
    //       2 = single key value: the lowest `need` blocks, 3 = none.
    uint32_t lo = 0, hi = 0, need = kp;
    int mode = 3;
    if (kBitmap && kp == 0) __syncthreads();   // orders the bitmap's clearing
    if (kp > 0) {
        // the first histogram is cleared here; the barrier after the min / max
        // orders the clearing before its increments
#pragma unroll
        for (int x = t; x < kTopkBins; x += kThreads) sm.hist[x] = 0;
        uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (cand(u)) {
                mn = key[u] < mn ? key[u] : mn;
                mx = key[u] > mx ? key[u] : mx;
            }
        }
        mn = wave_umin(mn);
        mx = wave_umax(mx);
        if (lane == 0) { sm.rmin[w] = mn; sm.rmax[w] = mx; }
        __syncthreads();
        lo = 0xffffffffu; hi = 0u;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
            lo = sm.rmin[x] < lo ? sm.rmin[x] : lo;
            hi = sm.rmax[x] > hi ? sm.rmax[x] : hi;
        }
        for (bool first = true;; first = false) {
            const uint32_t span = hi - lo;
            if (span == 0) { mode = 2; break; }
            const int bits = 32 - __clz(span);
            const int sh = bits > 10 ? bits - 10 : 0;
            if (!first) {
                // every read of the previous histogram came before the last barrier
#pragma unroll
                for (int x = t; x < kTopkBins; x += kThreads) sm.hist[x] = 0;
                __syncthreads();
            }
#pragma unroll
            for (int u = 0; u < kPer; ++u)
                if (cand(u) && key[u] >= lo && key[u] <= hi) atomicAdd(&sm.hist[(key[u] - lo) >> sh], 1u);
            __syncthreads();
            // descending bins: thread t owns bins [1024 - kB (t+1), 1024 - kB t)
            constexpr int kB = kTopkBins / kThreads;
            uint32_t cntb[kB];
            uint32_t sum = 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                cntb[u] = sm.hist[kTopkBins - 1 - (t * kB + u)];
                sum += cntb[u];
            }
            uint32_t total_w;
            const uint32_t incl = block_incl_scan_1b<kWaves>(sum, sm.scan_tmp[0], total_w);
            uint32_t run = incl - sum;            // candidates in higher bins
            // exactly one thread owns the bin of the need-th largest key
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                if (run < need && need <= run + cntb[u]) {
                    sm.bstar = static_cast<uint32_t>(kTopkBins - 1 - (t * kB + u));
                    sm.above = run;
                    sm.ebin = cntb[u];
                }
                run += cntb[u];
            }
            __syncthreads();
            const uint32_t bstar = sm.bstar;
            need -= sm.above;
            const uint32_t e = sm.ebin;
            const uint32_t nlo = lo + (bstar << sh);
            const uint32_t width = (sh >= 32) ? 0xffffffffu : ((1u << sh) - 1u);
            hi = (hi - nlo > width) ? nlo + width : hi;
            lo = nlo;
            if (e == need) { mode = 0; break; }
            if (e <= static_cast<uint32_t>(kThreads)) { mode = 1; break; }
        }
    }
    auto in_window = [&](int u) { return cand(u) && key[u] >= lo && key[u] <= hi; };
    int16_t slot_of[kPer];                // mode 1: where each window key was collected
#pragma unroll
    for (int u = 0; u < kPer; ++u) slot_of[u] = -1;
    if (mode == 1) {                      // collect the window's keys in block order, rank them
        uint32_t nw = 0;
#pragma unroll
        for (int u = 0; u < kPer; ++u) nw += in_window(u) ? 1u : 0u;
        uint32_t ncol;
        const uint32_t incl_w = block_incl_scan_1b<kWaves>(nw, sm.scan_tmp[1], ncol);
        uint32_t slot = incl_w - nw;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (in_window(u)) {
                sm.ckey[slot] = key[u];
                sm.cidx[slot] = jb + u;
                slot_of[u] = static_cast<int16_t>(slot);
                ++slot;
            }
        }
        // pad the collected keys to a multiple of four with entries that rank
        // below every key (key 0 at a block past every real one)
        if (static_cast<uint32_t>(t) < ((4u - (ncol & 3u)) & 3u)) {
            sm.ckey[ncol + t] = 0u;
            sm.cidx[ncol + t] = 0x7fffffff;
        }
        __syncthreads();
        if (static_cast<uint32_t>(t) < ncol) {
            const uint32_t mk = sm.ckey[t];
            const int32_t mj = sm.cidx[t];
            uint32_t rank = 0;
            const uint4* ck4 = reinterpret_cast<const uint4*>(sm.ckey);
            const int4* cj4 = reinterpret_cast<const int4*>(sm.cidx);
            for (uint32_t x = 0; x < (ncol + 3u) / 4u; ++x) {
                const uint4 ok = ck4[x];
                const int4 oj = cj4[x];
                rank += (ok.x > mk || (ok.x == mk && oj.x < mj)) ? 1u : 0u;
                rank += (ok.y > mk || (ok.y == mk && oj.y < mj)) ? 1u : 0u;
                rank += (ok.z > mk || (ok.z == mk && oj.z < mj)) ? 1u : 0u;
                rank += (ok.w > mk || (ok.w == mk && oj.w < mj)) ? 1u : 0u;
            }
            sm.keep[t] = rank < need ? 1u : 0u;
        }
        __syncthreads();
    }
    // selection flags of this thread's blocks
    Mask smask = 0;
    if (mode == 2) {                      // keys above the window, and its lowest `need` blocks
        uint32_t n_eq = 0;
#pragma unroll
        for (int u = 0; u < kPer; ++u) n_eq += in_window(u) ? 1u : 0u;
        uint32_t n_all;
        uint32_t r = block_incl_scan_1b<kWaves>(n_eq, sm.scan_tmp[1], n_all) - n_eq;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (cand(u) && key[u] > hi) smask |= Mask(1) << u;
            if (in_window(u)) {
                if (r < need) smask |= Mask(1) << u;
                ++r;
            }
        }
    } else if (mode != 3) {
        // keys above the window are taken; window keys by mode (all, or their keep
        // flags, read for every block at once without branches)
        uint32_t kf[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) kf[u] = (mode == 1) ? sm.keep[slot_of[u] < 0 ? 0 : slot_of[u]] : 1u;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const bool s = cand(u) && (key[u] > hi || (in_window(u) && kf[u] != 0u));
            if (s) smask |= Mask(1) << u;
        }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if (u < cnt && !cand(u)) smask |= Mask(1) << u;     // forced
    if constexpr (kBitmap) {
        if (smask != 0) atomicOr(&bits[jb >> 5], static_cast<uint32_t>(smask) << (jb & 31));
        return;
    }
    const uint32_t n_sel = sizeof(Mask) == 8 ? __popcll(static_cast<uint64_t>(smask))
                                             : __popc(static_cast<uint32_t>(smask));
    uint32_t n_total;
    const uint32_t incl = block_incl_scan_1b<kWaves>(n_sel, sm.scan_tmp[2], n_total);
    uint32_t pos = incl - n_sel;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        if ((smask >> u) & 1u) {
            if (pos < static_cast<uint32_t>(k)) {
                idx[pos] = jb + u;
                if (score) score[pos] = key_to_score(key[u]);
            }
            ++pos;
        }
    }
    // slots past the total are padding
    for (int r = static_cast<int>(n_total) + t; r < k; r += kThreads) {
        idx[r] = -1;
        if (score) score[r] = kNaN;
    }
}

// Wave-level reads of the selection bitmap (kWords words, bit j = block j):
// lane l holds words [l kWpl, (l + 1) kWpl) and their inclusive set-bit count.
template <int kWords>
struct BitmapLanes {
    static constexpr int kWpl = (kWords + 63) / 64;
    uint32_t wv[kWpl];
    uint32_t excl, incl;
    __device__ explicit BitmapLanes(const uint32_t* bits) {
        const int lane = threadIdx.x & 63;
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < kWpl; ++i) {
            const int x = lane * kWpl + i;
            wv[i] = x < kWords ? bits[x] : 0u;
            cnt += __popc(wv[i]);
        }
        incl = wave_incl_sum(cnt);
        excl = incl - cnt;
    }
    // block of the e-th (0-based, ascending) selected slot, -1 past the last;
    // e wave-uniform, the result in every lane.  The lane whose words hold that
    // slot is found by a ballot; its word and the slot's rank in it are read
    // into every lane, and lane b < 32 tests whether bit b is that set bit.
    __device__ int32_t nth(int e) const {
        const int lane = threadIdx.x & 63;
        const uint32_t ue = static_cast<uint32_t>(e);
        const uint64_t ball = __ballot(excl <= ue && ue < incl);
        if (ball == 0) return -1;
        const int src = static_cast<int>(__builtin_ctzll(ball));
        uint32_t r = ue - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(excl), src));
        uint32_t word = 0;
        int wi = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < kWpl; ++i) {
            const uint32_t wvi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wv[i]), src));
            const uint32_t p = __popc(wvi);
            if (!found && r < p) { word = wvi; wi = i; found = true; }
            else if (!found) r -= p;
        }
        const uint32_t below = lane < 32 ? (1u << lane) - 1u : 0xffffffffu;
        const uint64_t hit = __ballot(lane < 32 && ((word >> lane) & 1u) != 0u && __popc(word & below) == r);
        return (src * kWpl + wi) * 32 + static_cast<int>(__builtin_ctzll(hit));
    }
    // the selection as an ascending list of k slots, padded with -1 (one wave)
    __device__ void write_list(int32_t* __restrict__ out, int k) const {
        const int lane = threadIdx.x & 63;
        uint32_t pos = excl;
#pragma unroll
        for (int i = 0; i < kWpl; ++i) {
            uint32_t word = wv[i];
            while (word != 0u) {
                const int b = __builtin_ctz(word);
                if (pos < static_cast<uint32_t>(k)) out[pos] = (lane * kWpl + i) * 32 + b;
                ++pos;
                word &= word - 1u;
            }
        }
        const int total = __builtin_amdgcn_readlane(static_cast<int>(incl), 63);
        for (int r = total + lane; r < k; r += 64) out[r] = -1;
    }
};

}  // namespace infv2
