// Prefill attention over the selected blocks on the matrix cores (bf16, KV block 64).
// MiniCPM4 summary page, "InfLLM v2" section: "Complexity analysis" (Stage 2,
// each query token attends the k*m tokens of its own selected blocks), "Design
// principles summary" (token-level queries, block-level keys/values) and "Query
// group sharing" (the group's 16 heads form the 16-wide matrix tile of a token).
//
// Every query row picks its own 64 blocks, so the matrix tile of a (row, block)
// pair is 16 heads x 64 keys.  A thread block owns 16 consecutive rows of one
// KV head, one row per wave (16 waves, four per SIMD, so that the latency of
// one wave's dependent MFMA / softmax chain hides behind the others).  The
// block builds the union of the rows' selected blocks and streams it through
// LDS with direct global->LDS loads (K and V as stored; the V^T operand comes
// from the V tile by transpose reads), two blocks per barrier interval with the
// next interval's loads in flight under the current one's products.  The
// streaming order spreads each interval's (row, block) pairs over the SIMDs
// (balance_union, refine_pairs).
// For each block the waves whose row selected it run:
//   S^T[key][head] = K_blk . Q_row^T          16 MFMA 16x16x32
//   O^T[d][head]  += V^T_blk . P_row^T        16 MFMA 16x16x32
// One head sits in each lane column, so softmax state is per lane.  The
// reference max of a row is only raised when a block exceeds it by more than
// 2^8 (then the output is rescaled); otherwise probabilities are taken against
// the old reference (p <= 256, exact in fp32 and bf16), which skips the
// cross-lane max and the rescale on almost every block.  Row sums stay per lane
// until the end.  Keys after the row (t > i) are masked in the row's own block.
// Thread blocks are placed so that each XCD (own L2) serves row groups of one
// KV head, the later (larger) ones first.
#include "common.hpp"
#include "kernels.hpp"
#include "prefill_tiles.hpp"

namespace infv2 {

constexpr int kPRows = 16;       // query rows per thread block
constexpr int kPWaves = 16;      // one query row per wave, four waves per SIMD
constexpr int kPRowsW = 16 / kPWaves;                // query rows per wave
constexpr int kKBatch = 2;       // K-steps whose fragments are read from LDS at once
constexpr int kVBatch = 2;       // V^T d-tiles whose fragments are read from LDS at once
constexpr int kTileLoads = 16 / kPWaves;             // 1 KB global->LDS loads per wave per tile
constexpr int kPThreads = kPWaves * 64;
static_assert(kPThreads == kUThreads && kPRows == kURows, "rows and threads of the union build");
constexpr int kGroup2 = 2;       // union blocks per LDS stage = per barrier interval; two stages
constexpr int kXcds = 8;         // thread blocks are dealt round-robin to the 8 XCDs
constexpr float kRescaleSlack = 8.f;   // log2 units

typedef BlockTile StageTiles[kGroup2];              // 2 x 16 KB (K) or 2 x 16 KB (V^T)

__global__ __launch_bounds__(kPThreads, 1) void attn_prefill_mfma(
    const PrefillSeqs seqs, const bf16_t* __restrict__ q_all, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const int64_t* __restrict__ kv_off_all,
    const int32_t* __restrict__ idx_all, bf16_t* __restrict__ out_all, int hq, int hkv, int topk,
    float scale_log2) {
    __shared__ __attribute__((aligned(16))) StageTiles kst[2], vst[2];   // two stages
    __shared__ UnionSmem sm;
    // XCD-aware placement: thread block b runs on XCD b % 8 and the blocks of
    // one XCD start in the order of b.  When the KV heads divide the XCDs, each
    // head gets 8 / hkv XCDs of its own (its K / V prefix in their L2), they take
    // its row groups in turn, and each XCD runs its share from the last row
    // group down: later rows see more blocks, so the largest unions start first
    // and the small ones fill in behind them (a per-XCD tail of +2 % in a host
    // model of config 3's unions, against +11 % for contiguous ranges in row
    // order).  Otherwise each XCD gets a contiguous range of work items.
    const int nrg = seqs.grp_end[seqs.n - 1];
    const int xcd = static_cast<int>(blockIdx.x) % kXcds, kx = static_cast<int>(blockIdx.x) / kXcds;
    int g, grp;
    if (kXcds % hkv == 0) {
        const int xh = kXcds / hkv;                        // XCDs per KV head
        g = xcd / xh;
        const int rank = kx * xh + xcd % xh;
        if (rank >= nrg) return;                           // grid padding (whole block)
        grp = nrg - 1 - rank;
    } else {
        const int nwg = static_cast<int>(gridDim.x);
        const int qx = nwg / kXcds, rx = nwg % kXcds;
        const int lid = xcd * qx + (xcd < rx ? xcd : rx) + kx;
        g = lid / nrg;
        grp = lid % nrg;
    }
    int si = 0;
    while (si + 1 < seqs.n && grp >= seqs.grp_end[si]) ++si;
    const int r0 = (grp - (si > 0 ? seqs.grp_end[si - 1] : 0)) * kPRows;
    const int rows = seqs.rows[si];
    const int64_t q_start = seqs.q_start[si];
    const size_t row0 = static_cast<size_t>(seqs.row0[si]);
    const bf16_t* q = q_all + row0 * hq * kHeadDim;
    bf16_t* out = out_all + row0 * hq * kHeadDim;
    const int32_t* idx = idx_all + row0 * hkv * topk;
    const int64_t* kv_off = kv_off_all + seqs.seq[si];
    const int64_t nblk = (q_start + rows + kPB - 1) / kPB;
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const int64_t cap = kv_off[1] - kv_off[0];
    const bf16_t* kh = k + (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const bf16_t* vh = v + (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const int64_t nlim = q_start + rows;                     // keys needed are < nlim

    // ---- union of the 16 rows' selected blocks (ascending list + row masks)
    const int n_u = build_union(sm, idx, rows, r0, hkv, g, topk, nblk);
    balance_union(sm, n_u);                   // intervals spread their work over the SIMDs
    refine_pairs(sm, n_u);                    // and exchanges between intervals even it out further

    // ---- per-wave row state: wave w owns rows r0 + 8 i + w (i < 2)
    bf16x8_t qf[kPRowsW][4];
    f32x4_t o[kPRowsW][8];
    float mref[kPRowsW], lsum[kPRowsW];       // per lane: reference max of head lc, partial row sum
    int32_t qpos[kPRowsW];
#pragma unroll
    for (int i = 0; i < kPRowsW; ++i) {
        const int row = r0 + kPWaves * i + w;
        const int rr = row < rows ? row : rows - 1;
        qpos[i] = static_cast<int32_t>(q_start + row);
        const bf16_t* qrow = q + (static_cast<size_t>(rr) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[i][ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[i][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mref[i] = -INFINITY;
        lsum[i] = 0.f;
    }
    // make the compiler wait for the q fragments here, where it sees the use;
    // otherwise it keeps them pending and waits for all loads (the next
    // interval's tile loads included) inside the products
#pragma unroll
    for (int i = 0; i < kPRowsW; ++i)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" :: "v"(qf[i][ks]));

    // ---- stream the union through LDS with direct global->LDS loads.  Each
    // wave fills 1 KB of each K and V tile; the lane part of the address is
    // fixed, only the block part (wave-uniform) changes.
    int koff_l[kTileLoads], key_l[kTileLoads];
#pragma unroll
    for (int j = 0; j < kTileLoads; ++j) {
        const int sg = kTileLoads * w + j;
        key_l[j] = 4 * sg + (l >> 4);                       // keys 4 sg .. 4 sg + 3
        koff_l[j] = key_l[j] * kHeadDim + 8 * ((l & 15) ^ (key_l[j] & 15));
    }
    auto issue = [&](StageTiles& kt, StageTiles& vs, int u) {
        const int slot = u % kGroup2;
        const int32_t blk = sm.list[u];
        const int64_t k0 = static_cast<int64_t>(blk) * kPB;
        const bool partial = k0 + kPB > nlim;               // last block of the chunk
#pragma unroll
        for (int j = 0; j < kTileLoads; ++j) {
            const int sg = kTileLoads * w + j;
            int64_t off = k0 * kHeadDim + koff_l[j];
            if (partial) {                                  // clamp: keys past the chunk get P = 0
                int64_t gk = k0 + key_l[j];
                gk = gk < nlim ? gk : nlim - 1;
                off = gk * kHeadDim + 8 * ((l & 15) ^ (key_l[j] & 15));
            }
            dma16(kh + off, lds_offset(&kt[slot][sg * 512]));
            dma16(vh + off, lds_offset(&vs[slot][sg * 512]));
        }
    };
    // V^T operands of O^T = V^T P^T come from the V tile by transpose reads:
    // for d-tile mt and keys 32 kk + 16 a + 4 lg + 0..3 this lane reads the 4
    // values d = 16 mt + 4 (lc % 4) .. + 3 of key 32 kk + 16 a + kq, which hands
    // lane lc element e = V[key 32 kk + 16 a + 4 lg + e][d = 16 mt + lc] -- the
    // key order of the P^T operand (the accumulator layout of S^T)
    const int kq = 4 * lg + (lc >> 2), kqb = (lc >> 1) & 1;
    const uint32_t kq0 = static_cast<uint32_t>(kq * kHeadDim * 2 + 8 * (lc & 1));
    auto compute = [&](const StageTiles& kt, const StageTiles& vs, int u) {
        const int slot = u % kGroup2;
        const int32_t blk = sm.list[u];
        const uint32_t msk = sm.mask[u];
        uint32_t act = 0;
        int cntr[kPRowsW];
#pragma unroll
        for (int i = 0; i < kPRowsW; ++i) {
            cntr[i] = qpos[i] + 1 - blk * kPB;               // keys of the block at or before the row
            if (((msk >> (kPWaves * i + w)) & 1u) && cntr[i] > 0) act |= 1u << i;
        }
        act = __builtin_amdgcn_readfirstlane(act);          // wave-uniform by construction
        if (!act) return;
        // K fragments, kKBatch K-steps at a time (their LDS latencies overlap);
        // lane holds K[key 16 mt + lc][32 ks + 8 lg ..]
        f32x4_t s[kPRowsW][4];
#pragma unroll
        for (int i = 0; i < kPRowsW; ++i)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[i][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; kb += kKBatch) {
            uint4 kf[kKBatch][4];
#pragma unroll
            for (int ks = 0; ks < kKBatch; ++ks)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) kf[ks][mt] = k_frag(kt[slot], 16 * mt + lc, 4 * (kb + ks) + lg);
#pragma unroll
            for (int i = 0; i < kPRowsW; ++i) {
                if (!((act >> i) & 1u)) continue;
#pragma unroll
                for (int ks = 0; ks < kKBatch; ++ks)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        s[i][mt] = mfma32(as_bf16x8(kf[ks][mt]), qf[i][kb + ks], s[i][mt]);
            }
        }
        bf16x8_t pf[kPRowsW][2];
#pragma unroll
        for (int i = 0; i < kPRowsW; ++i) {
            if (!((act >> i) & 1u)) continue;
            // raw logits; the scale (> 0) is applied to the max and inside the exp
            float lm = -INFINITY;
            if (__builtin_amdgcn_readfirstlane(cntr[i]) >= kPB) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) lm = fmaxf(lm, s[i][mt][r]);
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = (16 * mt + 4 * lg + r) < cntr[i] ? s[i][mt][r] : -INFINITY;
                        s[i][mt][r] = x;
                        lm = fmaxf(lm, x);
                    }
            }
            lm *= scale_log2;
            // raise the reference only when some head of the row overshoots it
            if (__any(lm > mref[i] + kRescaleSlack)) {
                const float mx = max_xor32(max_xor16(lm));
                const float mnew = fmaxf(mref[i], mx);
                const float alpha = (mref[i] == -INFINITY) ? 0.f : fast_exp2(mref[i] - mnew);
                lsum[i] *= alpha;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[i][mt][r] *= alpha;
                mref[i] = mnew;
            }
            float ls = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(fmaf(s[i][mt][r], scale_log2, -mref[i]));   // masked: 2^-inf = 0
                    s[i][mt][r] = p;
                    ls += p;
                }
            lsum[i] += ls;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 pu;
                pu.x = pack_rne(s[i][2 * kk][0], s[i][2 * kk][1]);
                pu.y = pack_rne(s[i][2 * kk][2], s[i][2 * kk][3]);
                pu.z = pack_rne(s[i][2 * kk + 1][0], s[i][2 * kk + 1][1]);
                pu.w = pack_rne(s[i][2 * kk + 1][2], s[i][2 * kk + 1][3]);
                pf[i][kk] = as_bf16x8(pu);
            }
        }
        // V^T fragments, kVBatch d-tiles at a time
        const uint32_t vb0 = lds_offset(&vs[slot][0]) + kq0;
#pragma unroll
        for (int mb = 0; mb < 8; mb += kVBatch) {
            uint4 vf[kVBatch][2];
#pragma unroll
            for (int x = 0; x < kVBatch; ++x) {
                // chunk 2 mt + kqb of key 32 kk + 16 a + kq sits at chunk (2 mt + kqb) ^ kq
                const uint32_t o = vb0 + 16u * static_cast<uint32_t>((2 * (mb + x) + kqb) ^ kq);
                const uint2 a0 = lds_read_tr16(o), a1 = lds_read_tr16(o + 16u * kHeadDim * 2);
                const uint2 b0 = lds_read_tr16(o + 32u * kHeadDim * 2), b1 = lds_read_tr16(o + 48u * kHeadDim * 2);
                vf[x][0] = make_uint4(a0.x, a0.y, a1.x, a1.y);
                vf[x][1] = make_uint4(b0.x, b0.y, b1.x, b1.y);
            }
#pragma unroll
            for (int x = 0; x < kVBatch; ++x)
#pragma unroll
                for (int i = 0; i < kPRowsW; ++i) {
                    if (!((act >> i) & 1u)) continue;
                    o[i][mb + x] = mfma32(as_bf16x8(vf[x][0]), pf[i][0], o[i][mb + x]);
                    o[i][mb + x] = mfma32(as_bf16x8(vf[x][1]), pf[i][1], o[i][mb + x]);
                }
        }
    };
    // Two-block barrier intervals, double-buffered: the loads of interval iv + 1
    // run under the products of interval iv.
    const int n_iv = (n_u + kGroup2 - 1) / kGroup2;
    for (int x = 0; x < kGroup2 && x < n_u; ++x) issue(kst[0], vst[0], x);
    for (int iv = 0; iv < n_iv; ++iv) {
        // interval iv landed (the only loads in flight); every wave is done
        // with interval iv - 1, whose stage now takes interval iv + 1, one
        // block's loads before each block of products
        dma_wait_barrier();
        const int sx = (iv + 1) & 1, sc = iv & 1;
#pragma unroll
        for (int b = 0; b < kGroup2; ++b) {
            const int xn = (iv + 1) * kGroup2 + b, u = iv * kGroup2 + b;
            if (xn < n_u) issue(kst[sx], vst[sx], xn);
            if (u < n_u) compute(kst[sc], vst[sc], u);
        }
    }

    // ---- epilogue: row sum over the four lanes of each head; lane holds
    // O[head lc][d = 16 mt + 4 lg + r]
#pragma unroll
    for (int i = 0; i < kPRowsW; ++i) {
        const float lt = add_xor32(add_xor16(lsum[i]));
        const int row = r0 + kPWaves * i + w;
        if (row >= rows) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        bf16_t* dst = out + (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            uint2 pk;
            pk.x = pack_rne(o[i][mt][0] * inv, o[i][mt][1] * inv);
            pk.y = pack_rne(o[i][mt][2] * inv, o[i][mt][3] * inv);
            *reinterpret_cast<uint2*>(dst + 16 * mt) = pk;
        }
    }
}

// blocks of the launch: 8 per (8 / hkv) row groups when the KV heads divide the
// XCDs (the kernel maps them head by head), else one per (KV head, row group)
static unsigned prefill_grid(int nrg, int hkv) {
    if (kXcds % hkv == 0) {
        const int xh = kXcds / hkv;
        return static_cast<unsigned>(kXcds) * static_cast<unsigned>((nrg + xh - 1) / xh);
    }
    return static_cast<unsigned>(nrg) * static_cast<unsigned>(hkv);
}

bool attn_prefill_mfma_ok(const Shape& sh) {
    return sh.io_bf16 && sh.m == kPB && kPRows * sh.topk <= kUnionCap;
}

size_t attn_prefill_ws_bytes(const Shape&, int64_t) { return 0; }   // no workspace

hipError_t launch_attn_prefill_mfma_seqs(const Shape& sh, const PrefillSeqs& seqs, const void* q,
                                         const void* k, const void* v, const int64_t* kv_off,
                                         const int32_t* idx, void* out, hipStream_t st) {
    if (seqs.n < 1 || seqs.n > kVarlenMax) return hipErrorInvalidValue;
    const int nrg = seqs.grp_end[seqs.n - 1];
    if (nrg < 1) return hipSuccess;
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    launch_timed(INFV2_KERNEL_ATTN_PREFILL, attn_prefill_mfma,
                 dim3(prefill_grid(nrg, sh.hkv)), dim3(kPThreads), 0, st, seqs,
        static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
        static_cast<const bf16_t*>(v), kv_off, idx, static_cast<bf16_t*>(out), sh.hq, sh.hkv,
        sh.topk, scale_log2);
    return hipGetLastError();
}

hipError_t launch_attn_prefill_mfma(const Shape& sh, const void* q, int rows, int64_t q_start,
                                    const void* k, const void* v, const int64_t* kv_off,
                                    const int32_t* idx, void* out, void* ws, hipStream_t st) {
    (void)ws;
    PrefillSeqs seqs{};
    seqs.n = 1;
    seqs.grp_end[0] = (rows + kPRows - 1) / kPRows;
    seqs.seq[0] = 0;
    seqs.row0[0] = 0;
    seqs.rows[0] = rows;
    seqs.q_start[0] = q_start;
    return launch_attn_prefill_mfma_seqs(sh, seqs, q, k, v, kv_off, idx, out, st);
}

}  // namespace infv2
