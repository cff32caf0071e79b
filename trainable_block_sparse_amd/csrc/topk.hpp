// Block-wide top-k selection with forced blocks, for one (query row, KV head).
// MiniCPM4 summary page, "InfLLM v2" section: paragraph "Top-K implementation
// and the LSE bottleneck" (select the K blocks with the highest group score)
// and paragraph "Initial and local tokens always selected" (block 0 and the
// local window are always kept; shorter than k*m degenerates to dense).
//
// Candidates are the blocks 0..c that are not forced.  Scores arrive as sortable
// 32-bit keys (score_to_key) in LDS.  The k' = k - |F| largest keys are found
// by an MSB-first radix select (four 8-bit digits, histogram in LDS), which
// yields the exact k'-th largest key T and how many candidates equal to T are
// still needed; those are taken in increasing block order, so ties go to the
// lower block.  Each thread owns a contiguous range of block indices, so the
// ascending output needs only two block-wide scans.  Must be called by all
// kThreads threads of the block (kThreads a multiple of 256).
#pragma once

#include "common.hpp"

namespace infv2 {

struct TopkSmem {
    uint32_t hist[256];
    uint32_t scan_tmp[24];
    uint32_t prefix, need;
};

__device__ __forceinline__ bool is_forced(int64_t j, int64_t c, int init, int local) {
    return j < init || j > c - local;
}

// lk: [c+1] sortable scores in LDS.  Writes idx[k] (and score[k] if non-null).
template <int kThreads>
__device__ inline void block_topk_lds(const uint32_t* lk, int64_t c, int k, int init, int local,
                                      int32_t* __restrict__ idx, float* __restrict__ score,
                                      TopkSmem& sm) {
    constexpr int kWaves = kThreads / 64;
    const int t = threadIdx.x;
    const int nb = static_cast<int>(c + 1);
    const float kNaN = __uint_as_float(0x7fc00000u);
    if (nb <= k) {                      // dense: every block, then -1 padding
        for (int r = t; r < k; r += kThreads) {
            idx[r] = r < nb ? r : -1;
            if (score) score[r] = r < nb ? key_to_score(lk[r]) : kNaN;
        }
        return;
    }
    const int a = init < nb ? init : nb;
    const int lo = c - local + 1 > 0 ? static_cast<int>(c - local + 1) : 0;
    const int nforced = a + (nb - (lo > a ? lo : a));
    const uint32_t kp = static_cast<uint32_t>(k - nforced);
    const int per = (nb + kThreads - 1) / kThreads;
    const int jb = t * per;
    const int je = jb + per < nb ? jb + per : nb;

    uint32_t prefix = 0, mask = 0, need = kp;
    if (kp > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (t < 256) sm.hist[t] = 0;
            __syncthreads();
            for (int j = jb; j < je; ++j) {
                if (is_forced(j, c, init, local)) continue;
                const uint32_t key = lk[j];
                if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // thread t < 256 looks at digit 255 - t; incl = #candidates with digit >= it
            const uint32_t v = t < 256 ? sm.hist[255 - t] : 0u;
            const uint32_t incl = block_incl_scan<kWaves>(v, sm.scan_tmp);
            const uint32_t excl = incl - v;
            if (t < 256 && excl < need && need <= incl) {
                sm.prefix = prefix | (static_cast<uint32_t>(255 - t) << shift);
                sm.need = need - excl;
            }
            __syncthreads();
            prefix = sm.prefix;
            need = sm.need;
            mask |= 255u << shift;
            __syncthreads();
        }
    }
    // selected = forced, strictly above T, and the first `need` candidates equal to T
    uint32_t n_eq = 0;
    if (kp > 0)
        for (int j = jb; j < je; ++j)
            n_eq += (!is_forced(j, c, init, local) && lk[j] == prefix) ? 1u : 0u;
    const uint32_t eq_base = block_incl_scan<kWaves>(n_eq, sm.scan_tmp) - n_eq;
    uint32_t n_sel = 0;
    {
        uint32_t r = eq_base;
        for (int j = jb; j < je; ++j) {
            const bool f = is_forced(j, c, init, local);
            const uint32_t key = lk[j];
            const bool eq = !f && kp > 0 && key == prefix;
            const bool sel = f || (!f && kp > 0 && key > prefix) || (eq && r < need);
            r += eq ? 1u : 0u;
            n_sel += sel ? 1u : 0u;
        }
    }
    uint32_t pos = block_incl_scan<kWaves>(n_sel, sm.scan_tmp) - n_sel;
    {
        uint32_t r = eq_base;
        for (int j = jb; j < je; ++j) {
            const bool f = is_forced(j, c, init, local);
            const uint32_t key = lk[j];
            const bool eq = !f && kp > 0 && key == prefix;
            const bool sel = f || (!f && kp > 0 && key > prefix) || (eq && r < need);
            r += eq ? 1u : 0u;
            if (sel && pos < static_cast<uint32_t>(k)) {
                idx[pos] = j;
                if (score) score[pos] = key_to_score(key);
            }
            pos += sel ? 1u : 0u;
        }
    }
    // every selected block is written above; slots past the total stay padding
    if (t == kThreads - 1) sm.scan_tmp[kWaves] = pos;
    __syncthreads();
    for (int r = static_cast<int>(sm.scan_tmp[kWaves]) + t; r < k; r += kThreads) {
        idx[r] = -1;
        if (score) score[r] = kNaN;
    }
}

// keys in global memory: staged into the LDS scratch `lk` (>= c+1 words) first
template <int kThreads>
__device__ inline void block_topk(const uint32_t* gkeys, int64_t c, int k, int init, int local,
                                  int32_t* __restrict__ idx, float* __restrict__ score,
                                  TopkSmem& sm, uint32_t* lk) {
    const int nb = static_cast<int>(c + 1);
    if (nb > k) {
        // batches of independent loads, then the LDS stores
        for (int j0 = threadIdx.x; j0 < nb; j0 += 8 * kThreads) {
            uint32_t r[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * kThreads;
                r[u] = j < nb ? gkeys[j] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * kThreads;
                if (j < nb) lk[j] = r[u];
            }
        }
        __syncthreads();
        block_topk_lds<kThreads>(lk, c, k, init, local, idx, score, sm);
    } else {
        block_topk_lds<kThreads>(gkeys, c, k, init, local, idx, score, sm);
    }
}

}  // namespace infv2
