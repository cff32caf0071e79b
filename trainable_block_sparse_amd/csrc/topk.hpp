// Block-wide top-k selection with forced blocks, for one (query row, KV head).
// MiniCPM4 summary page, "InfLLM v2" section: paragraph "Top-K implementation
// and the LSE bottleneck" (select the K blocks with the highest group score)
// and paragraph "Initial and local tokens always selected" (block 0 and the
// local window are always kept; shorter than k*m degenerates to dense).
//
// Candidates are the blocks 0..c that are not forced.  Scores arrive as sortable
// 32-bit keys (score_to_key).  The k' = k - |F| largest keys are found by an
// MSB-first radix select (four 8-bit digits, histogram in LDS), which yields the
// exact k'-th largest key T and how many candidates equal to T are still
// needed; those are taken in increasing block order, so ties go to the lower
// block.  The output is written in ascending block order by a block-wide scan.
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

// keys: [c+1] sortable scores in global memory; writes idx[k] (and score[k] if non-null).
__device__ inline void block_topk(const uint32_t* keys, int64_t c, int k, int init, int local,
                                  int32_t* __restrict__ idx, float* __restrict__ score,
                                  TopkSmem& sm) {
    const int t = threadIdx.x;
    const int64_t nb = c + 1;
    if (nb <= k) {                      // dense: every block, then -1 padding
        for (int r = t; r < k; r += 256) {
            idx[r] = r < nb ? r : -1;
            if (score) score[r] = r < nb ? key_to_score(keys[r]) : __uint_as_float(0x7fc00000u);
        }
        return;
    }
    const int64_t a = init < nb ? init : nb;
    const int64_t lo = c - local + 1 > 0 ? c - local + 1 : 0;
    const int64_t nforced = a + (nb - (lo > a ? lo : a));
    const uint32_t kp = static_cast<uint32_t>(k - nforced);

    uint32_t prefix = 0, mask = 0, need = kp;
    if (kp > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            sm.hist[t] = 0;
            __syncthreads();
            for (int64_t j = t; j < nb; j += 256) {
                if (is_forced(j, c, init, local)) continue;
                const uint32_t key = keys[j];
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
    // output pass in block order: forced, strictly above T, then the first
    // `need` candidates equal to T
    uint32_t base_eq = 0, base_out = 0;
    for (int64_t j0 = 0; j0 < nb; j0 += 256) {
        const int64_t j = j0 + t;
        const bool valid = j < nb;
        const bool f = valid && is_forced(j, c, init, local);
        const uint32_t key = valid ? keys[j] : 0u;
        const bool cand = valid && !f && kp > 0;
        const bool eq = cand && key == prefix;
        const uint32_t eq_incl = block_incl_scan256(eq ? 1u : 0u, sm.scan_tmp);
        const uint32_t eq_rank = base_eq + eq_incl - (eq ? 1u : 0u);
        const bool sel = f || (cand && key > prefix) || (eq && eq_rank < need);
        const uint32_t sel_incl = block_incl_scan256(sel ? 1u : 0u, sm.scan_tmp);
        const uint32_t pos = base_out + sel_incl - 1u;
        if (sel && pos < static_cast<uint32_t>(k)) {
            idx[pos] = static_cast<int32_t>(j);
            if (score) score[pos] = key_to_score(key);
        }
        // totals of this chunk live in the last thread's inclusive scans
        if (t == 255) { sm.scan_tmp[4] = eq_incl; sm.scan_tmp[5] = sel_incl; }
        __syncthreads();
        base_eq += sm.scan_tmp[4];
        base_out += sm.scan_tmp[5];
        __syncthreads();
    }
    for (int r = static_cast<int>(base_out) + t; r < k; r += 256) {
        idx[r] = -1;
        if (score) score[r] = __uint_as_float(0x7fc00000u);
    }
}

}  // namespace infv2
