// Decode attention over the selected blocks on the matrix cores (bf16 K/V/Q).
// MiniCPM4 summary page, "InfLLM v2" section: "Complexity analysis" (Stage 2,
// each query token attends the k*m tokens of its selected blocks) and "Query
// group sharing" (the 16 heads of a group read each selected block once, which
// is what makes the 16-row matrix tile a real contraction).
//
// The work is cut into 16-key tiles of the selected blocks, and every wave makes
// two dependent memory round trips before its first product: (offsets, length,
// block ids, queries), then its first tile's K and V rows.  At batch 1 (64
// blocks per KV head, 4 MiB in all, latency-bound) each wave takes one tile;
// at large batches a run of tiles, loading the next tile while it computes
// the current one.  Per tile and wave, all in registers:
//   S^T[key][head] = K_tile (16x128) . Q^T (128x16)      4 MFMA 16x16x32
//   V^T tiles      = V_tile . I  (identity MFMA, exact)    8 MFMA 16x16x16
//   O^T[d][head]  += V^T (128x16) . P^T (16x16)           8 MFMA 16x16x16
// K rows are the A operand as stored (16 contiguous bytes per lane), so K and V
// stream from HBM with 16-byte coalesced loads.  The S^T layout puts one query
// head per lane column; it is also exactly the B-operand layout of P^T.  The
// thread block merges its four waves' (max, sum, output) in LDS in a fixed
// order (results are deterministic) and writes one partial per split;
// attn_decode_merge combines the splits by their LogSumExp in a second kernel.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace infv2 {

struct DecSmem {
    float o[4][kGroup][kHeadDim + 4];     // each wave's partial output, [head][d]
    float m[4][kGroup];                   // each wave's running max per head (log2 units)
    float l[4][kGroup];                   // each wave's running sum per head
};

// One wave's run of tpw 16-key tiles of selected block `blk` (< 0: none), from
// piece st0 of the block, with an online softmax (running max, sum, output),
// loading tile x + 1 while it computes tile x; then the thread block's merge of
// its four waves in LDS, in wave order, into the split's partial at pbase.
// kRun = false: one tile per wave (tpw == 1), no second set of K / V registers.
template <bool kRun>
__device__ __forceinline__ void decode_run(DecSmem& sm, const bf16x8_t (&qf)[4], int32_t blk, int st0,
                                           int tpw_arg, int m, int64_t n, const bf16_t* kh,
                                           const bf16_t* vh, float scale_log2,
                                           float* __restrict__ part_o, float2* __restrict__ part_ml,
                                           size_t pbase) {
    const int tpw = kRun ? tpw_arg : 1;
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    // identity B operand for the transpose MFMA: B[4 lg + j][lc] = (4 lg + j == lc)
    s16x4_t ident;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident[j] = (4 * lg + j == lc) ? static_cast<short>(0x3f80) : 0;
    // piece x of the run: its first key and its keys below n (<= 0: nothing to do)
    auto piece = [&](int x, int64_t& t0, int64_t& cnt) {
        t0 = static_cast<int64_t>(blk) * m + 16 * (st0 + x);
        cnt = blk < 0 ? 0 : n - t0;
        cnt = cnt < 16 ? cnt : 16;
    };
    auto load_tile = [&](int64_t t0, int64_t cnt, uint4 (&kr)[4], uint4 (&vr)[4]) {
        if (cnt > 0) {                               // wave-uniform
            int64_t key = t0 + lc;
            key = key < n ? key : n - 1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kr[c] = ldg16_nt(kh + key * kHeadDim + 32 * c);
                vr[c] = ldg16_nt(vh + key * kHeadDim + 32 * c);
            }
        }
    };

    f32x4_t o[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) o[c][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    uint4 kr[4], vr[4], kn[4], vn[4];
    int64_t t0, cnt;
    piece(0, t0, cnt);
    load_tile(t0, cnt, kr, vr);
    for (int x = 0; x < tpw; ++x) {
        // the next piece's K / V, in flight under this piece's products
        int64_t t1 = 0, cnt1 = 0;
        if (kRun && x + 1 < tpw) {
            piece(x + 1, t1, cnt1);
            load_tile(t1, cnt1, kn, vn);
        }
        if (cnt > 0) {
            // S^T: lane holds S[key 4 lg + r][head lc]
            f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s = mfma32(as_bf16x8(kr[ks]), qf[ks], s);
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float xv = (4 * lg + r < cnt) ? s[r] * scale_log2 : -INFINITY;
                s[r] = xv;
                mx = fmaxf(mx, xv);
            }
            mx = max_xor32(max_xor16(mx));
            const float mnew = fmaxf(mrun, mx);      // finite: key 0 of the tile is below n
            const float alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mnew);
            float p[4], ls = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = (s[r] == -INFINITY) ? 0.f : exp2f(s[r] - mnew);
                ls += p[r];
            }
            ls = add_xor32(add_xor16(ls));
            lrun = lrun * alpha + ls;
            mrun = mnew;
            // P^T as the B operand: lane holds P[key 4 lg + j][head lc]
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(pack_rne(p[0], p[1]), pack_rne(p[2], p[3])));
            // V^T tile (d column block c, half hf), then O^T = alpha O^T + V^T . P^T.
            // Transpose output: lane holds V[key 4 lg + r][d(lc)], d(x) = 32 c + 8 (x/4) + 4 hf + x%4
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[c][hf][r] *= alpha;
                    const uint2 half = hf ? make_uint2(vr[c].z, vr[c].w) : make_uint2(vr[c].x, vr[c].y);
                    const f32x4_t vt = mfma16(__builtin_bit_cast(s16x4_t, half), ident, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    const s16x4_t va = __builtin_bit_cast(s16x4_t, make_uint2(pack_exact(vt[0], vt[1]), pack_exact(vt[2], vt[3])));
                    o[c][hf] = mfma16(va, pb, o[c][hf]);
                }
            }
        }
        if (kRun && x + 1 < tpw) {
#pragma unroll
            for (int c = 0; c < 4; ++c) { kr[c] = kn[c]; vr[c] = vn[c]; }
            t0 = t1;
            cnt = cnt1;
        }
    }
    // O^T lane layout: O[head lc][d = 32 c + 8 lg + 4 hf + r]
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            *reinterpret_cast<float4*>(&sm.o[w][lc][32 * c + 8 * lg + 4 * hf]) =
                make_float4(o[c][hf][0], o[c][hf][1], o[c][hf][2], o[c][hf][3]);
    if (lg == 0) { sm.m[w][lc] = mrun; sm.l[w][lc] = lrun; }
    __syncthreads();
    // merge the waves in wave order: thread -> 4 columns of one head
    for (int x = t; x < kGroup * kHeadDim / 4; x += 256) {
        const int h = x >> 5, c4 = (x & 31) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int y = 0; y < 4; ++y) M = fmaxf(M, sm.m[y][h]);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                if (sm.m[y][h] == -INFINITY) continue;
                const float wgt = exp2f(sm.m[y][h] - M);
                const float4 a = *reinterpret_cast<const float4*>(&sm.o[y][h][c4]);
                acc.x = fmaf(wgt, a.x, acc.x); acc.y = fmaf(wgt, a.y, acc.y);
                acc.z = fmaf(wgt, a.z, acc.z); acc.w = fmaf(wgt, a.w, acc.w);
            }
        }
        *reinterpret_cast<float4*>(part_o + (pbase + h) * kHeadDim + c4) = acc;
    }
    if (t < kGroup) {
        float M = -INFINITY, L = 0.f;
#pragma unroll
        for (int y = 0; y < 4; ++y) M = fmaxf(M, sm.m[y][t]);
        if (M != -INFINITY) {
#pragma unroll
            for (int y = 0; y < 4; ++y)
                if (sm.m[y][t] != -INFINITY) L += sm.l[y][t] * exp2f(sm.m[y][t] - M);
        }
        part_ml[pbase + t] = make_float2(M, L);
    }
}

// Grid (split, KV head, sequence), four waves per thread block.  The tiles of a
// (sequence, KV head) are its selected blocks cut into 16-key pieces, in slot
// order; split sp covers tiles [4 tpw sp, 4 tpw (sp + 1)), wave w of it the run
// of tpw tiles starting at 4 tpw sp + w tpw, all in one block (tpw divides the
// block's m / 16 tiles).
template <bool kRun>
__global__ __launch_bounds__(256) void attn_decode_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ lens, int lens_end,
    const int32_t* __restrict__ idx, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int hq, int hkv, int m, int topk, int nsplit, int tpw_arg, float scale_log2) {
    const int tpw = kRun ? tpw_arg : 1;
    __shared__ DecSmem sm;
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const int tpb = m >> 4;                          // 16-key tiles per block
    const int ntiles = topk * tpb;
    const int u0 = (sp * 4 + w) * tpw;               // this wave's first tile
    // round trip 1: every load below depends only on the kernel arguments
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
    // the wave's tiles are tpw consecutive 16-key pieces of ONE selected block
    // (tpw divides the block's tile count)
    const int e = u0 / tpb, st0 = u0 - e * tpb;
    const int32_t blk_raw = idx[bg * topk + (e < topk ? e : topk - 1)];
    const bf16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    const int64_t cap = o1 - o0;
    const int64_t n = seq_len(o0, o1, lv, lens_end);     // decode row i = n - 1 sees keys t < n
    const bf16_t* kh = k + (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * cap) * kHeadDim + 8 * lg;
    const bf16_t* vh = v + (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * cap) * kHeadDim + 8 * lg;
    const int32_t blk = (u0 < ntiles && e < topk) ? blk_raw : -1;
    decode_run<kRun>(sm, qf, blk, st0, tpw, m, n, kh, vh, scale_log2, part_o, part_ml,
                     (bg * nsplit + sp) * kGroup);
}

// Decode step: the top-k of the (sequence, KV head) runs in every thread block
// of its attention, before the tiles, so the step needs no separate top-k launch
// and no round trip of the block list through memory.  The selection is the
// one the top-k kernel makes (same code, same keys); single-tile grids keep it
// as a bitmap of the selected blocks, read by each wave for its own block
// (cheaper than the ordered list at batch 1, dearer in the larger grids where
// waves run several tiles); split 0 also stores the list.  Tiles as attn_decode_mfma.  Keys: the
// block-score keys of the scoring pass, rows of kld entries padded to 256 kPer.
constexpr int kFusedTopkMax = 256;       // largest top-k the fused kernel serves

template <int kPer, bool kRun>
__global__ __launch_bounds__(256) void attn_decode_topk_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ lens, int lens_end,
    const uint32_t* __restrict__ keys, int64_t kld, int64_t nblk_max, int init, int local,
    int32_t* __restrict__ idx_out, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int hq, int hkv, int m, int topk, int nsplit, int tpw_arg, float scale_log2) {
    const int tpw = kRun ? tpw_arg : 1;
    static_assert(kPer % 2 == 0, "keys load in pairs");
    constexpr int kWords = topk_bm_words(256, kPer);
    __shared__ union { TopkSmem<256> tk; DecSmem dec; } sm;
    __shared__ uint32_t sel_bits[kWords];     // single tiles: the selection, bit j = block j
    __shared__ int32_t sel[kFusedTopkMax];    // runs: the selection as a list
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    // round trip 1: offsets, length, the block keys and the queries
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
    const int jb = t * kPer;
    const uint32_t* gk = keys + bg * kld + jb;
    uint32_t key[kPer];
    if constexpr (kPer % 4 == 0) {
#pragma unroll
        for (int u = 0; u < kPer; u += 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(gk + u);
            key[u] = x.x; key[u + 1] = x.y; key[u + 2] = x.z; key[u + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kPer; u += 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(gk + u);
            key[u] = x.x; key[u + 1] = x.y;
        }
    }
    const bf16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    const int64_t cap = o1 - o0;
    const int64_t n = seq_len(o0, o1, lv, lens_end);
    int64_t c = n > 0 ? (n - 1) / m : -1;
    c = c < nblk_max - 1 ? c : nblk_max - 1;
    int cnt = static_cast<int>(c + 1) - jb;
    cnt = cnt < 0 ? 0 : (cnt > kPer ? kPer : cnt);
    const int tpb = m >> 4;
    const int u0 = (sp * 4 + w) * tpw;   // this wave's first tile
    const int e = u0 / tpb, st0 = u0 - e * tpb;
    int32_t blk;
    if constexpr (!kRun) {
        // small grids: the selection as a bitmap (no ordered output scan); each
        // wave finds its own block in it
        block_topk_regs<256, kPer, true>(key, jb, cnt, static_cast<int>(c), topk, init, local, nullptr,
                                         static_cast<float*>(nullptr), sm.tk, sel_bits);
        __syncthreads();                 // the bitmap is complete; the top-k's LDS is free
        const BitmapLanes<kWords> bm(sel_bits);
        if (sp == 0 && w == 0) bm.write_list(idx_out + bg * topk, topk);
        blk = (e < topk) ? bm.nth(e) : -1;
    } else {
        block_topk_regs<256>(key, jb, cnt, static_cast<int>(c), topk, init, local, sel,
                             static_cast<float*>(nullptr), sm.tk);
        __syncthreads();                 // the list is complete; the top-k's LDS is free
        if (sp == 0)
            for (int r = t; r < topk; r += 256) idx_out[bg * topk + r] = sel[r];
        blk = (e < topk) ? sel[e] : -1;
    }
    const bf16_t* kh = k + (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * cap) * kHeadDim + 8 * lg;
    const bf16_t* vh = v + (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * cap) * kHeadDim + 8 * lg;
    decode_run<kRun>(sm.dec, qf, blk, st0, tpw, m, n, kh, vh, scale_log2, part_o, part_ml,
                     (bg * nsplit + sp) * kGroup);
}

// Merge of the split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// m in log2 units.  Grid (query head of the group, KV head, sequence), 256
// threads.  Thread t folds the (m, l) pairs of splits t, t + 256, ..; for the
// outputs, thread t takes columns 4 (t % 32) .. +3 of splits t / 32, t / 32 + 8,
// .. (the first eight of them loaded together with the pairs), and the eight
// split groups are summed in LDS in a fixed order.  Up to 64 splits (the batch-1
// grids) every wave folds all the pairs itself, one split per lane, and takes
// the weights from their lanes: the final sum is then the only barrier.
template <typename Tout>
__global__ __launch_bounds__(256) void attn_decode_merge(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         Tout* __restrict__ out, int hq, int hkv,
                                                         int nsplit, int64_t* __restrict__ lens_adv,
                                                         const int64_t* __restrict__ kv_off) {
    constexpr int kSg = 8;                 // split groups
    constexpr int kPre = 8;                // splits per thread loaded with the (m, l) pairs
    constexpr int kMlPer = kDecodeMaxSplit / 256;
    __shared__ float wgt[kDecodeMaxSplit];
    __shared__ float red[2][4];
    __shared__ float4 part[kSg][kHeadDim / 4];
    const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
    const int sg = t >> 5, cq = t & 31, wv = t >> 6;
    // a step that appended its token: the sequence's length moves on by one here,
    // in the step's last kernel, which no longer reads it
    if (lens_adv && h == 0 && g == 0 && t == 0) {
        const int64_t lv = lens_adv[b];
        if (lv < kv_off[b + 1] - kv_off[b]) lens_adv[b] = lv + 1;
    }
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const size_t stride = static_cast<size_t>(kGroup) * kHeadDim / 4;     // float4 per split
    const float4* po = reinterpret_cast<const float4*>(part_o) +
                       (bg * nsplit * kGroup + h) * (kHeadDim / 4) + cq;
    float4 pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (sg + kSg * i < nsplit) pre[i] = po[(sg + kSg * i) * stride];
    auto add = [&](float4& acc, float w, const float4& a) {
        acc.x = fmaf(w, a.x, acc.x); acc.y = fmaf(w, a.y, acc.y);
        acc.z = fmaf(w, a.z, acc.z); acc.w = fmaf(w, a.w, acc.w);
    };
    auto finish = [&](const float4& acc, float den) {
        part[sg][cq] = acc;
        __syncthreads();
        if (t < kHeadDim / 4) {
            float4 r = part[0][t];
#pragma unroll
            for (int j = 1; j < kSg; ++j) {
                const float4 a = part[j][t];
                r.x += a.x; r.y += a.y; r.z += a.z; r.w += a.w;
            }
            const float inv = den > 0.f ? 1.f / den : 0.f;
            Tout* dst = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + h) * kHeadDim + 4 * t;
            io<Tout>::store(dst + 0, r.x * inv);
            io<Tout>::store(dst + 1, r.y * inv);
            io<Tout>::store(dst + 2, r.z * inv);
            io<Tout>::store(dst + 3, r.w * inv);
        }
    };
    if (nsplit <= 64) {
        // one split per lane: every wave folds all the (m, l) pairs itself with
        // wave reductions and takes the weights of its splits from their lanes,
        // so the only barrier is the final sum over split groups (the same
        // arithmetic in the same order as the general path below)
        const int lane = t & 63;
        const float2 mlv = lane < nsplit ? part_ml[(bg * nsplit + lane) * kGroup + h] : make_float2(-INFINITY, 0.f);
        const float gm1 = wave_max(mlv.x);
        const float wt = (mlv.x == -INFINITY) ? 0.f : exp2f(mlv.x - gm1);
        const float den1 = wave_sum(wt * mlv.y);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const float wx = __shfl(wt, sg + kSg * i, 64);
            if (sg + kSg * i < nsplit) add(acc, wx, pre[i]);
        }
        finish(acc, den1);
        return;
    }
    float2 ml[kMlPer];
#pragma unroll
    for (int i = 0; i < kMlPer; ++i) {
        const int sx = t + 256 * i;
        ml[i] = sx < nsplit ? part_ml[(bg * nsplit + sx) * kGroup + h] : make_float2(-INFINITY, 0.f);
    }
    float gm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMlPer; ++i) gm = fmaxf(gm, ml[i].x);
    gm = wave_max(gm);
    if ((t & 63) == 0) red[0][wv] = gm;
    __syncthreads();
    gm = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float den_t = 0.f;
#pragma unroll
    for (int i = 0; i < kMlPer; ++i) {
        const int sx = t + 256 * i;
        const float wt = (ml[i].x == -INFINITY) ? 0.f : exp2f(ml[i].x - gm);
        if (sx < nsplit) wgt[sx] = wt;
        den_t += wt * ml[i].y;
    }
    const float den_w = wave_sum(den_t);
    if ((t & 63) == 0) red[1][wv] = den_w;
    __syncthreads();
    const float den = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (sg + kSg * i < nsplit) add(acc, wgt[sg + kSg * i], pre[i]);
#pragma unroll 4
    for (int x = sg + kSg * kPre; x < nsplit; x += kSg) add(acc, wgt[x], po[x * stride]);
    finish(acc, den);
}

hipError_t launch_attn_decode_mfma(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int tpw, hipStream_t st) {
    dim3 grid(nsplit, sh.hkv, batch);
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    const int64_t* lens = kv_lens ? kv_lens : kv_off + 1;
    const int lens_end = kv_lens ? (sh.lens_plus_one ? 2 : 0) : 1;
    if (tpw > 1)
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<true>, grid, dim3(256), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
            kv_off, lens, lens_end, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, tpw,
            scale_log2);
    else
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<false>, grid, dim3(256), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
            kv_off, lens, lens_end, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, 1,
            scale_log2);
    return hipGetLastError();
}

bool attn_decode_topk_ok(const Shape& sh, int64_t nblk_max) {
    return sh.io_bf16 && sh.topk <= kFusedTopkMax && topk_per(nblk_max, 256) <= 16 && (sh.m & 15) == 0;
}

hipError_t launch_attn_decode_topk(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const uint32_t* keys, int64_t kld, int64_t nblk_max,
                                   int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int tpw, hipStream_t st) {
    dim3 grid(nsplit, sh.hkv, batch);
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    const int64_t* lens = kv_lens ? kv_lens : kv_off + 1;
    const int lens_end = kv_lens ? (sh.lens_plus_one ? 2 : 0) : 1;
    const int per = topk_per(nblk_max, 256);
#define INFV2_L(P, R) launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_topk_mfma<P, R>, grid, dim3(256), 0, st, \
        static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), \
        kv_off, lens, lens_end, keys, kld, nblk_max, sh.init, sh.local, idx, part_o, part_ml, \
        sh.hq, sh.hkv, sh.m, sh.topk, nsplit, tpw, scale_log2)
    if (tpw > 1) {
        if (per <= 2) INFV2_L(2, true); else if (per <= 8) INFV2_L(8, true); else if (per <= 16) INFV2_L(16, true);
        else return hipErrorInvalidValue;
    } else {
        if (per <= 2) INFV2_L(2, false); else if (per <= 8) INFV2_L(8, false); else if (per <= 16) INFV2_L(16, false);
        else return hipErrorInvalidValue;
    }
#undef INFV2_L
    return hipGetLastError();
}

hipError_t launch_attn_decode_merge(const Shape& sh, const float* part_o, const float2* part_ml,
                                    void* out, int batch, int nsplit, hipStream_t st,
                                    int64_t* lens_adv, const int64_t* kv_off) {
    dim3 grid(kGroup, sh.hkv, batch);
    if (sh.io_bf16)
        launch_timed(INFV2_KERNEL_ATTN_MERGE, attn_decode_merge<bf16_t>, grid, dim3(256), 0, st,
                     part_o, part_ml, static_cast<bf16_t*>(out), sh.hq, sh.hkv, nsplit, lens_adv, kv_off);
    else
        launch_timed(INFV2_KERNEL_ATTN_MERGE, attn_decode_merge<float>, grid, dim3(256), 0, st,
                     part_o, part_ml, static_cast<float*>(out), sh.hq, sh.hkv, nsplit, lens_adv, kv_off);
    return hipGetLastError();
}

}  // namespace infv2
