// Decode attention over the selected blocks on the matrix cores (bf16 K/V/Q).
// MiniCPM4 summary page, "InfLLM v2" section: "Complexity analysis" (Stage 2,
// each query token attends the k*m tokens of its selected blocks) and "Query
// group sharing" (the 16 heads of a group read each selected block once, which
// is what makes the 16-row matrix tile a real contraction).
//
// A decode step at batch 1 is latency-bound: 64 blocks per KV head, 4 MiB in
// all.  So the work is cut into 16-key tiles, one per wave, and every wave makes
// exactly two dependent memory round trips: (offsets, length, block id,
// queries), then its tile's K and V rows.  Grid (split, KV head, sequence); a
// thread block of T waves covers T consecutive tiles of the (KV head,
// sequence)'s selection (T = 4: one 64-key block; T = 16 at large batches,
// fewer partials).  Per wave, all in registers:
//   S^T[key][head] = K_tile (16x128) . Q^T (128x16)      4 MFMA 16x16x32
//   V^T tiles      = V_tile . I  (identity MFMA, exact)    8 MFMA 16x16x16
//   O^T[d][head]  += V^T (128x16) . P^T (16x16)           8 MFMA 16x16x16
// K rows are the A operand as stored (16 contiguous bytes per lane), so K and V
// stream from HBM with 16-byte coalesced loads.  The S^T layout puts one query
// head per lane column; it is also exactly the B-operand layout of P^T.  The
// waves share one reference max per head (exchanged in LDS), so their partial
// outputs add up directly; the thread block sums them in a fixed order (results
// are deterministic) and writes one partial (max, sum, output).
// attn_decode_merge combines the splits by their LogSumExp in a second kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

template <int T>
struct DecSmem {
    float o[T][kGroup][kHeadDim + 4];     // each wave's partial output, [head][d]
    float m[T][kGroup];                   // each wave's max per head (log2 units)
    float l[T][kGroup];                   // each wave's sum per head
};

template <int T>
__global__ __launch_bounds__(64 * T) void attn_decode_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ lens, int lens_end,
    const int32_t* __restrict__ idx, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int hq, int hkv, int m, int topk, int nsplit, float scale_log2) {
    static_assert(T == 4 || T == 16, "four or sixteen waves");
    __shared__ DecSmem<T> sm;
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const int tpb = m >> 4;                          // 16-key tiles per block
    const int u = sp * T + w;                        // this wave's tile
    const int e = u / tpb, st = u - e * tpb;         // its selection slot and sub-tile
    // round trip 1: every load below depends only on the kernel arguments
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
    const int32_t blk_raw = idx[bg * topk + (e < topk ? e : topk - 1)];
    const bf16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    // identity B operand for the transpose MFMA: B[4 lg + j][lc] = (4 lg + j == lc)
    s16x4_t ident;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident[j] = (4 * lg + j == lc) ? static_cast<short>(0x3f80) : 0;

    const int64_t cap = o1 - o0;
    const int64_t n = seq_len(o0, o1, lv, lens_end);     // decode row i = n - 1 sees keys t < n
    const int32_t blk = e < topk ? blk_raw : -1;
    const int64_t t0 = static_cast<int64_t>(blk) * m + 16 * st;
    int64_t cnt = n - t0;
    cnt = cnt < 16 ? cnt : 16;
    const bool act = blk >= 0 && cnt > 0;                // wave-uniform

    f32x4_t o[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) o[c][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 vr[4];
    float mx = -INFINITY;
    if (act) {
        // round trip 2: K (A operand) and V rows of the tile, 16 B per lane each
        int64_t key = t0 + lc;
        key = key < n ? key : n - 1;
        const size_t base = (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * cap + key) * kHeadDim + 8 * lg;
        uint4 kr[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kr[c] = ldg16_nt(k + base + 32 * c);
            vr[c] = ldg16_nt(v + base + 32 * c);
        }
        // S^T: lane holds S[key 4 lg + r][head lc]
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s = mfma32(as_bf16x8(kr[ks]), qf[ks], s);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = (4 * lg + r < cnt) ? s[r] * scale_log2 : -INFINITY;
            s[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) vr[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (lg == 0) sm.m[w][lc] = mx;
    __syncthreads();
    float M = -INFINITY;                                 // the thread block's max of head lc
#pragma unroll
    for (int x = 0; x < T; ++x) M = fmaxf(M, sm.m[x][lc]);
    float ls = 0.f;
    if (act) {
        // M >= mx > -inf: probabilities against the shared reference
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = (s[r] == -INFINITY) ? 0.f : exp2f(s[r] - M);
            ls += p[r];
        }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        // P^T as the B operand: lane holds P[key 4 lg + j][head lc]
        const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(pack_rne(p[0], p[1]), pack_rne(p[2], p[3])));
        // V^T tile (d column block c, half hf), then O^T += V^T . P^T.  Transpose
        // output: lane holds V[key 4 lg + r][d(lc)], d(x) = 32 c + 8 (x/4) + 4 hf + x%4
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const uint2 half = hf ? make_uint2(vr[c].z, vr[c].w) : make_uint2(vr[c].x, vr[c].y);
                const f32x4_t vt = mfma16(__builtin_bit_cast(s16x4_t, half), ident, f32x4_t{0.f, 0.f, 0.f, 0.f});
                const s16x4_t va = __builtin_bit_cast(s16x4_t, make_uint2(pack_exact(vt[0], vt[1]), pack_exact(vt[2], vt[3])));
                o[c][hf] = mfma16(va, pb, o[c][hf]);
            }
        }
    }
    // O^T lane layout: O[head lc][d = 32 c + 8 lg + 4 hf + r]
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            *reinterpret_cast<float4*>(&sm.o[w][lc][32 * c + 8 * lg + 4 * hf]) =
                make_float4(o[c][hf][0], o[c][hf][1], o[c][hf][2], o[c][hf][3]);
    if (lg == 0) sm.l[w][lc] = ls;
    __syncthreads();
    // the waves' outputs, summed in wave order: thread -> 4 columns of one head
    const size_t pbase = (bg * nsplit + sp) * kGroup;
    for (int x = t; x < kGroup * kHeadDim / 4; x += 64 * T) {
        const int h = x >> 5, c4 = (x & 31) * 4;
        float4 acc = *reinterpret_cast<const float4*>(&sm.o[0][h][c4]);
#pragma unroll
        for (int y = 1; y < T; ++y) {
            const float4 a = *reinterpret_cast<const float4*>(&sm.o[y][h][c4]);
            acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
        }
        *reinterpret_cast<float4*>(part_o + (pbase + h) * kHeadDim + c4) = acc;
    }
    if (t < kGroup) {
        float mh = -INFINITY, lh = 0.f;
#pragma unroll
        for (int y = 0; y < T; ++y) {
            mh = fmaxf(mh, sm.m[y][t]);
            lh += sm.l[y][t];
        }
        part_ml[pbase + t] = make_float2(mh, lh);
    }
}

// Merge of the split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// m in log2 units.  Grid (query head of the group, KV head, sequence), 256
// threads.  Thread t folds the (m, l) pairs of splits t, t + 256, ..; for the
// outputs, thread t takes columns 4 (t % 32) .. +3 of splits t / 32, t / 32 + 8,
// .. (the first eight of them loaded together with the pairs), and the eight
// split groups are summed in LDS in a fixed order.
template <typename Tout>
__global__ __launch_bounds__(256) void attn_decode_merge(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         Tout* __restrict__ out, int hq, int hkv,
                                                         int nsplit) {
    constexpr int kSg = 8;                 // split groups
    constexpr int kPre = 8;                // splits per thread loaded with the (m, l) pairs
    constexpr int kMlPer = kDecodeMaxSplit / 256;
    __shared__ float wgt[kDecodeMaxSplit];
    __shared__ float red[2][4];
    __shared__ float4 part[kSg][kHeadDim / 4];
    const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
    const int sg = t >> 5, cq = t & 31, wv = t >> 6;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const size_t stride = static_cast<size_t>(kGroup) * kHeadDim / 4;     // float4 per split
    const float4* po = reinterpret_cast<const float4*>(part_o) +
                       (bg * nsplit * kGroup + h) * (kHeadDim / 4) + cq;
    float4 pre[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (sg + kSg * i < nsplit) pre[i] = po[(sg + kSg * i) * stride];
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
    auto add = [&](float w, const float4& a) {
        acc.x = fmaf(w, a.x, acc.x); acc.y = fmaf(w, a.y, acc.y);
        acc.z = fmaf(w, a.z, acc.z); acc.w = fmaf(w, a.w, acc.w);
    };
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (sg + kSg * i < nsplit) add(wgt[sg + kSg * i], pre[i]);
#pragma unroll 4
    for (int x = sg + kSg * kPre; x < nsplit; x += kSg) add(wgt[x], po[x * stride]);
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
}

hipError_t launch_attn_decode_mfma(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int tiles_wg, hipStream_t st) {
    dim3 grid(nsplit, sh.hkv, batch);
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    const int64_t* lens = kv_lens ? kv_lens : kv_off + 1;
    const int lens_end = kv_lens ? 0 : 1;
    if (tiles_wg == 4)
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<4>, grid, dim3(256), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
            kv_off, lens, lens_end, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, scale_log2);
    else
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<16>, grid, dim3(1024), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
            kv_off, lens, lens_end, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, scale_log2);
    return hipGetLastError();
}

hipError_t launch_attn_decode_merge(const Shape& sh, const float* part_o, const float2* part_ml,
                                    void* out, int batch, int nsplit, hipStream_t st) {
    dim3 grid(kGroup, sh.hkv, batch);
    if (sh.io_bf16)
        launch_timed(INFV2_KERNEL_ATTN_MERGE, attn_decode_merge<bf16_t>, grid, dim3(256), 0, st,
                     part_o, part_ml, static_cast<bf16_t*>(out), sh.hq, sh.hkv, nsplit);
    else
        launch_timed(INFV2_KERNEL_ATTN_MERGE, attn_decode_merge<float>, grid, dim3(256), 0, st,
                     part_o, part_ml, static_cast<float*>(out), sh.hq, sh.hkv, nsplit);
    return hipGetLastError();
}

}  // namespace infv2
