// Decode attention over the selected blocks on the matrix cores (bf16 K/V/Q).
// MiniCPM4 summary page, "InfLLM v2" section: "Complexity analysis" (Stage 2,
// each query token attends the k*m tokens of its selected blocks) and "Query
// group sharing" (the 16 heads of a group read each selected block once, which
// is what makes the 16-row matrix tile a real contraction).
//
// Grid (split, KV head, sequence), W waves per block and one selected block per
// wave: W = 4, or W = 1 when four-block splits would leave most compute units
// idle (small batches).  Each wave owns whole 64-token pieces of its block and
// keeps everything in registers:
//   S^T[key][head] = K_blk (64x128) . Q^T (128x16)      16 MFMA 16x16x32
//   V^T tiles      = V_blk . I  (identity MFMA, exact)  32 MFMA 16x16x16
//   O^T[d][head]  += V^T (128x64) . P^T (64x16)         16 MFMA 16x16x32
// K rows are the A operand exactly as stored (16 contiguous bytes per lane), so
// K and V stream from HBM with 16-byte coalesced loads and never touch LDS.
// The S^T layout puts one query head per lane column, so the online softmax
// rescale is a per-lane scalar.  The waves of a block merge in LDS and each
// block writes one partial (max, sum, output); attn_decode_merge combines the
// splits by their LogSumExp in a second kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

template <int W>
struct DecSmem {
    float o[W][kGroup][kHeadDim + 4];
    float m[W][kGroup];
    float l[W][kGroup];
};

template <int W>
__global__ __launch_bounds__(64 * W) void attn_decode_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ kv_lens,
    const int32_t* __restrict__ idx, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int hq, int hkv, int m, int topk, int nsplit, float scale_log2) {
    static_assert(W == 1 || W == 4, "one or four waves");
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const int e0 = sp * W;
    const int e1 = (e0 + W < topk) ? e0 + W : topk;
    // the wave's first block id is loaded together with the offsets (one round trip)
    const int32_t blk_first = (e0 + w < e1) ? idx[bg * topk + e0 + w] : -1;
    const int64_t o0 = kv_off[b], cap = kv_off[b + 1] - o0;
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const int64_t lim = n;                       // decode row i = n - 1 sees keys t < n
    const bf16_t* kh = k + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const bf16_t* vh = v + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;

    // Q^T as the B operand: lane holds Q[head lc][32 ks + 8 lg .. +7]
    const bf16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    // identity B operand for the transpose MFMA: B[4 lg + j][lc] = (4 lg + j == lc)
    s16x4_t ident;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident[j] = (4 * lg + j == lc) ? static_cast<short>(0x3f80) : 0;

    f32x4_t o[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) o[c][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;

    for (int e = e0 + w; e < e1; e += W) {
        const int32_t blk = e == e0 + w ? blk_first : idx[bg * topk + e];
        if (blk < 0) continue;
        for (int sub = 0; sub < m; sub += 64) {
            const int64_t t0 = static_cast<int64_t>(blk) * m + sub;
            int64_t cnt = lim - t0;
            cnt = cnt < m - sub ? cnt : m - sub;
            cnt = cnt < 64 ? cnt : 64;
            if (cnt <= 0) continue;
            // issue every load of the piece first: K (A operand) and V rows, 16 B per lane each
            uint4 kr[4][4], vr[4][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                int64_t key = t0 + 16 * mt + lc;
                key = key < lim ? key : lim - 1;
                const bf16_t* kp = kh + key * kHeadDim + 8 * lg;
                const bf16_t* vp = vh + key * kHeadDim + 8 * lg;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    kr[mt][c] = ldg16(kp + 32 * c);
                    vr[mt][c] = ldg16(vp + 32 * c);
                }
            }
            // S^T: lane holds S[head lc][key 16 mt + 4 lg + r]
            f32x4_t s[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) s[mt] = mfma32(as_bf16x8(kr[mt][ks]), qf[ks], s[mt]);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = (16 * mt + 4 * lg + r) < cnt;
                    const float x = ok ? s[mt][r] * scale_log2 : -INFINITY;
                    s[mt][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrun, mx);
            const float alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mnew);
            float ls = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = (s[mt][r] == -INFINITY) ? 0.f : exp2f(s[mt][r] - mnew);
                    s[mt][r] = p;
                    ls += p;
                }
            ls += __shfl_xor(ls, 16, 64);
            ls += __shfl_xor(ls, 32, 64);
            lrun = lrun * alpha + ls;
            mrun = mnew;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[c][h][r] *= alpha;
            // P^T as the B operand of K-step kk: slot e <-> key 32 kk + 16 (e/4) + 4 lg + e%4
            bf16x8_t pf[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 u;
                u.x = pack_rne(s[2 * kk][0], s[2 * kk][1]);
                u.y = pack_rne(s[2 * kk][2], s[2 * kk][3]);
                u.z = pack_rne(s[2 * kk + 1][0], s[2 * kk + 1][1]);
                u.w = pack_rne(s[2 * kk + 1][2], s[2 * kk + 1][3]);
                pf[kk] = as_bf16x8(u);
            }
            // V^T tiles (d column block c, half hf) then O^T += V^T . P^T.
            // transpose MFMA output: lane holds V[key 16 mt + 4 lg + r][d(lc)],
            // d(n) = 32 c + 8 (n/4) + 4 hf + n%4
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    f32x4_t vt[4];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const uint2 half = hf ? make_uint2(vr[mt][c].z, vr[mt][c].w)
                                              : make_uint2(vr[mt][c].x, vr[mt][c].y);
                        vt[mt] = mfma16(__builtin_bit_cast(s16x4_t, half), ident,
                                        f32x4_t{0.f, 0.f, 0.f, 0.f});
                    }
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        uint4 u;
                        u.x = pack_exact(vt[2 * kk][0], vt[2 * kk][1]);
                        u.y = pack_exact(vt[2 * kk][2], vt[2 * kk][3]);
                        u.z = pack_exact(vt[2 * kk + 1][0], vt[2 * kk + 1][1]);
                        u.w = pack_exact(vt[2 * kk + 1][2], vt[2 * kk + 1][3]);
                        o[c][hf] = mfma32(as_bf16x8(u), pf[kk], o[c][hf]);
                    }
                }
            }
        }
    }
    // O^T lane layout: O[head lc][d = 32 c + 8 lg + 4 hf + r]
    if constexpr (W == 1) {
        float* po = part_o + ((bg * nsplit + sp) * kGroup + lc) * kHeadDim + 8 * lg;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                *reinterpret_cast<float4*>(po + 32 * c + 4 * hf) =
                    make_float4(o[c][hf][0], o[c][hf][1], o[c][hf][2], o[c][hf][3]);
        if (lg == 0) part_ml[(bg * nsplit + sp) * kGroup + lc] = make_float2(mrun, lrun);
        return;
    } else {
        __shared__ DecSmem<W> sm;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                *reinterpret_cast<float4*>(&sm.o[w][lc][32 * c + 8 * lg + 4 * hf]) =
                    make_float4(o[c][hf][0], o[c][hf][1], o[c][hf][2], o[c][hf][3]);
        if (lg == 0) { sm.m[w][lc] = mrun; sm.l[w][lc] = lrun; }
        __syncthreads();

        // merge the waves: thread -> head h, 8 columns
        const int h = t >> 4, c0 = (t & 15) * 8;
        float mx = -INFINITY;
#pragma unroll
        for (int x = 0; x < W; ++x) mx = fmaxf(mx, sm.m[x][h]);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
            for (int x = 0; x < W; ++x) {
                if (sm.m[x][h] == -INFINITY) continue;
                const float wgt = exp2f(sm.m[x][h] - mx);
                den += wgt * sm.l[x][h];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(wgt, sm.o[x][h][c0 + e], acc[e]);
            }
        }
        float* po = part_o + ((bg * nsplit + sp) * kGroup + h) * kHeadDim + c0;
        *reinterpret_cast<float4*>(po) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>(po + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if ((t & 15) == 0) part_ml[(bg * nsplit + sp) * kGroup + h] = make_float2(mx, den);
    }
}

// Merge of the split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// m in log2 units.  Grid (query head of the group, KV head, sequence).  Thread t
// takes the (m, l) pair of split t, and output columns 4 (t % 32) .. +3 of the
// splits t / 32, t / 32 + 8, ...; the eight split groups are summed in LDS.
template <typename T>
__global__ __launch_bounds__(256) void attn_decode_merge(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         T* __restrict__ out, int hq, int hkv,
                                                         int nsplit) {
    constexpr int kSg = 8;                 // split groups
    constexpr int kPre = 8;                // splits per thread loaded with the (m, l) pairs
    static_assert(kDecodeMaxSplit <= 256, "one (m, l) pair per thread");
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
    float2 ml = make_float2(-INFINITY, 0.f);
    if (t < nsplit) ml = part_ml[(bg * nsplit + t) * kGroup + h];
    float gm = wave_max(ml.x);
    if ((t & 63) == 0) red[0][wv] = gm;
    __syncthreads();
    gm = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    const float wt = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - gm);
    if (t < nsplit) wgt[t] = wt;
    const float den_w = wave_sum(wt * ml.y);
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
        T* dst = out + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + h) * kHeadDim + 4 * t;
        io<T>::store(dst + 0, r.x * inv);
        io<T>::store(dst + 1, r.y * inv);
        io<T>::store(dst + 2, r.z * inv);
        io<T>::store(dst + 3, r.w * inv);
    }
}

hipError_t launch_attn_decode_mfma(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int bps, hipStream_t st) {
    dim3 grid(nsplit, sh.hkv, batch);
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    if (bps == 1)
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<1>, grid, dim3(64), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
            kv_off, kv_lens, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, scale_log2);
    else
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_mfma<4>, grid, dim3(256), 0, st,
        static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
        kv_off, kv_lens, idx, part_o, part_ml, sh.hq, sh.hkv, sh.m, sh.topk, nsplit, scale_log2);
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
