// Block-wide top-k selection with forced blocks, for one (query row, KV head).
// MiniCPM4 summary page, "InfLLM v2" section: paragraph "Top-K implementation
// and the LSE bottleneck" (select the K blocks with the highest group score)
// and paragraph "Initial and local tokens always selected" (block 0 and the
// local window are always kept; shorter than k*m degenerates to dense).
//
// Candidates are the blocks 0..c that are not forced.  Scores arrive as sortable
// 32-bit keys (score_to_key) and are staged once in LDS.  The k' = k - |F|
// largest keys are found by an MSB-first radix select (four 8-bit digits,
// histogram in LDS), which yields the exact k'-th largest key T and how many
// candidates equal to T are still needed; those are taken in increasing block
// order, so ties go to the lower block.  Each thread owns a contiguous range of
// block indices, so the ascending output needs only two block-wide scans.
// Must be called by all 256 threads of the block.
#pragma once

#include "common.hpp"

namespace infv2 {

struct TopkSmem {
    uint32_t hist[256];
    uint32_t scan_tmp[8];
    uint32_t prefix, need;
};

__device__ __forceinline__ bool is_forced(int64_t j, int64_t c, int init, int local) {
    return j < init || j > c - local;
}

// gkeys: [c+1] sortable scores in global memory; lk: LDS scratch of >= c+1 words.
// Writes idx[k] (and score[k] if non-null).
__device__ inline void block_topk(const uint32_t* gkeys, int64_t c, int k, int init, int local,
                                  int32_t* __restrict__ idx, float* __restrict__ score,
                                  TopkSmem& sm, uint32_t* lk) {
    const int t = threadIdx.x;
    const int nb = static_cast<int>(c + 1);
    const float kNaN = __uint_as_float(0x7fc00000u);
    if (nb <= k) {                      // dense: every block, then -1 padding
        for (int r = t; r < k; r += 256) {
            idx[r] = r < nb ? r : -1;
            if (score) score[r] = r < nb ? key_to_score(gkeys[r]) : kNaN;
        }
        return;
    }
    for (int j = t; j < nb; j += 256) lk[j] = gkeys[j];
    const int a = init < nb ? init : nb;
    const int lo = c - local + 1 > 0 ? static_cast<int>(c - local + 1) : 0;
    const int nforced = a + (nb - (lo > a ? lo : a));
    const uint32_t kp = static_cast<uint32_t>(k - nforced);
    const int per = (nb + 255) / 256;
    const int jb = t * per;
    const int je = jb + per < nb ? jb + per : nb;
    __syncthreads();

    uint32_t prefix = 0, mask = 0, need = kp;
    if (kp > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            sm.hist[t] = 0;
            __syncthreads();
            for (int j = jb; j < je; ++j) {
                if (is_forced(j, c, init, local)) continue;
                const uint32_t key = lk[j];
                if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // thread t looks at digit 255 - t; incl = #candidates with digit >= it
            const uint32_t v = sm.hist[255 - t];
            const uint32_t incl = block_incl_scan256(v, sm.scan_tmp);
            const uint32_t excl = incl - v;
            if (excl < need && need <= incl) {
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
    const uint32_t eq_base = block_incl_scan256(n_eq, sm.scan_tmp) - n_eq;
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
    uint32_t pos = block_incl_scan256(n_sel, sm.scan_tmp) - n_sel;
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
    if (t == 255) sm.scan_tmp[4] = pos;
    __syncthreads();
    for (int r = static_cast<int>(sm.scan_tmp[4]) + t; r < k; r += 256) {
        idx[r] = -1;
        if (score) score[r] = kNaN;
    }
}

}  // namespace infv2
