// Block selection: kernel logits, per-head LogSumExp, group score, block max,
// top-k with forced blocks.  MiniCPM4 summary page, "InfLLM v2" section:
// "Semantic kernels" (eqs. r_kernel, r_block), "Query group sharing" (eq.
// r_group), "Top-K implementation and the LSE bottleneck" (pass 1: LogSumExp
// over all kernels; pass 2: normalised scores), "Initial and local tokens".
//
// Decode (one row per sequence, thousands of kernels per row):
//   sel_dec_logits  grid (kernel chunk, KV head, sequence).  Each block scores
//                   64 kernels against the group's 16 heads (matrix cores for
//                   bf16 queries), stores the logits (fp32 scratch, 16 x n_c
//                   floats per KV head: an eighth of a fp32 compressed-key
//                   re-read) and a partial (max, sum-exp) per head.
//   sel_dec_scores  grid (kernel chunk, KV head, sequence): 256 kernels per
//                   block, 1024 in large grids.  Each block folds the partials
//                   into the per-head LogSumExp, forms the group score
//                   R_j = mean_h exp(z_hj - LSE_h) and the block max by
//                   atomicMax on sortable keys.
//   sel_dec_topk    one block per (sequence, KV head).
// Cross-block results are handed over at kernel boundaries only: a device-scope
// fence inside a kernel costs a write-back and invalidation of the whole L2 of
// the XCD on gfx950, once per block.
// Prefill (rows of one sequence, causal visibility per row):
//   ck_split_hilo   fp32 compressed keys, times score_scale log2 e -> hi / lo
//                   bf16 rows, once per call.
//   sel_pre_mfma<1> 16 rows per block on the matrix cores: per-head LogSumExp.
//   sel_pre_mfma<2> the same logits again: group score, block max.
//   (sel_pre_lse / sel_pre_scores: the vector-ALU versions for fp32 queries)
//   sel_pre_topk    one block per (row, KV head).
// Rows shorter than k*m without requested scores: sel_dense_ids only.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

#include <type_traits>

namespace infv2 {

constexpr float kLog2eF = 1.4426950408889634f;   // exp(x) = 2^(x log2 e) on the transcendental unit
constexpr float kLn2F = 0.6931471805599453f;
constexpr int kChunkA = 64;      // kernels per block in sel_dec_logits
constexpr int kLogitsNtMaxBlocks = 1024;   // nontemporal key loads up to this many logits blocks
constexpr int kLogWaves = 2;     // waves per 64-kernel chunk in sel_dec_logits_mfma (4 was no faster)
constexpr int kLogTiles = 4 / kLogWaves;   // 16-kernel tiles per wave
constexpr int kChunkB = 256;     // kernels per block in sel_dec_scores (1024 in large grids)
constexpr int kScoresTwoMinBlocks = 512;   // grids above this take 1024-kernel blocks
constexpr int kRowsPre = 4;      // query rows per block in the prefill passes
constexpr int kTilePre = 64;     // kernels per LDS tile in the prefill passes

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// first / last kernel meeting block `blk`: [j s, j s + p) and [blk m, (blk+1) m) share a token
__device__ __forceinline__ int64_t first_kernel_of_block(int64_t blk, int m, int p, int s) {
    const int64_t v = floor_div(blk * m - p, s) + 1;
    return v > 0 ? v : 0;
}
__device__ __forceinline__ int64_t last_kernel_of_block(int64_t blk, int m, int s) {
    return ((blk + 1) * m - 1) / s;
}

// the coarse-kernel variant adds the coarse pass-1 logits and partials (sized for
// the smallest coarse size it accepts, the fine kernel size) and the normalisers
static size_t coarse_extra(const Shape& sh, int batch, int64_t max_len, size_t* lc, size_t* pc, size_t* ls) {
    const int64_t nc = max_len < sh.p ? 1 : (max_len - sh.p) / sh.p + 1;
    const int64_t ld = (nc + 3) & ~int64_t(3);
    const int64_t nch = (nc + kChunkA - 1) / kChunkA;
    const size_t bg = static_cast<size_t>(batch) * sh.hkv;
    size_t off = 0;
    *lc = off; off += align256(bg * ld * kGroup * sizeof(float));
    *pc = off; off += align256(bg * nch * kGroup * sizeof(float2));
    *ls = off; off += align256(bg * kGroup * sizeof(float));
    return off;
}

SelectDecodeWs select_decode_ws(const Shape& sh, int batch, int64_t max_len) {
    SelectDecodeWs w{};
    w.nc_max = max_len < sh.p ? 0 : (max_len - sh.p) / sh.s + 1;
    w.nblk_max = (max_len + sh.m - 1) / sh.m;
    if (w.nblk_max < 1) w.nblk_max = 1;
    const int64_t ncm = w.nc_max > 0 ? w.nc_max : 1;
    w.nc_ld = (ncm + 3) & ~int64_t(3);
    w.nchunk_a = static_cast<int>((ncm + kChunkA - 1) / kChunkA);
    w.nchunk_b = static_cast<int>((ncm + kChunkB - 1) / kChunkB);
    const size_t bg = static_cast<size_t>(batch) * sh.hkv;
    size_t off = 0;
    w.logits = off;   off += align256(bg * w.nc_ld * kGroup * sizeof(float));
    w.partial = off;  off += align256(bg * w.nchunk_a * kGroup * sizeof(float2));
    // key rows padded to the top-k's register tile (256 threads x kPer keys), so
    // that its loads need no bounds
    w.keys_ld = static_cast<int64_t>(256) * topk_kper(topk_per(w.nblk_max, 256));
    w.keys = off;     off += align256(bg * w.keys_ld * sizeof(uint32_t));
    w.total = off;
    size_t lc, pc, ls;
    w.total_coarse = off + coarse_extra(sh, batch, max_len, &lc, &pc, &ls);
    w.logits_c = off + lc; w.partial_c = off + pc; w.lse_c = off + ls;
    return w;
}

PrefillSeqs one_seq(int rows, int64_t q_start) {
    PrefillSeqs t{};
    t.n = 1;
    t.grp_end[0] = (rows + 15) / 16;
    t.rows[0] = rows;
    t.q_start[0] = q_start;
    return t;
}

SelectPrefillWs select_prefill_ws(const Shape& sh, int rows, int64_t max_len, int nseq) {
    SelectPrefillWs w{};
    w.nblk_max = (max_len + sh.m - 1) / sh.m;
    if (w.nblk_max < 1) w.nblk_max = 1;
    size_t off = 0;
    w.lse = off;  off += align256(static_cast<size_t>(rows) * sh.hq * sizeof(float));
    w.keys = off; off += align256(static_cast<size_t>(rows) * sh.hkv * w.nblk_max * sizeof(uint32_t));
    if (!sh.ck_bf16) {
        // every kernel a row below max_len can see; a coarse kernel (size and
        // stride >= p) is at most one per p tokens
        w.ld = num_kernels(max_len, sh.p, sh.s);
        w.ld = w.ld < 1 ? 1 : w.ld;
        w.ldc = max_len / sh.p + 1;
        w.hl = off;   off += align256(static_cast<size_t>(nseq) * 2 * sh.hkv * w.ld * kHeadDim * sizeof(bf16_t));
        w.total = off;
        w.hlc = off;  off += align256(static_cast<size_t>(2) * sh.hkv * w.ldc * kHeadDim * sizeof(bf16_t));
        w.total_coarse = off;
    } else {
        w.total = w.total_coarse = off;
    }
    return w;
}

// ------------------------------------------------------------------ decode, pass 1
template <typename Tq, typename Tck>
__global__ __launch_bounds__(256) void sel_dec_logits(
    const Tq* __restrict__ q, const Tck* __restrict__ ck, const int64_t* __restrict__ ck_off,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ kv_lens, int hq, int hkv,
    int p, int s, float score_scale, int64_t nc_max, int64_t nc_ld, int nchunk, int64_t nblk_max,
    int64_t kld, float* __restrict__ logits, float2* __restrict__ partial, uint32_t* __restrict__ keys) {
    __shared__ float qs[kGroup][kHeadDim];
    const int b = blockIdx.z, g = blockIdx.y, ch = blockIdx.x, t = threadIdx.x;
    const int64_t cap = kv_off[b + 1] - kv_off[b];
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const int64_t ccap = ck_off[b + 1] - ck_off[b];
    int64_t nvis = num_kernels(n, p, s);          // row n-1 sees every complete kernel
    nvis = nvis < ccap ? nvis : ccap;
    nvis = nvis < nc_max ? nvis : nc_max;
    const size_t bg = static_cast<size_t>(b) * hkv + g;

    // clear this block's share of the block-score keys (filled by pass 2)
    {
        uint32_t* kb = keys + bg * kld;
        const int64_t per = (nblk_max + nchunk - 1) / nchunk;
        const int64_t e = (ch + 1) * per < nblk_max ? (ch + 1) * per : nblk_max;
        for (int64_t j = ch * per + t; j < e; j += 256) kb[j] = 0u;
    }
    const Tq* qg = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim;
    for (int e = t; e < kGroup * kHeadDim; e += 256) qs[e / kHeadDim][e % kHeadDim] = io<Tq>::load(qg + e);
    __syncthreads();

    const int w = t >> 6, lane = t & 63;
    const int64_t j = static_cast<int64_t>(ch) * kChunkA + lane;
    float z[4];
    if (j < nvis) {
        const Tck* row = ck + ((ck_off[b] * hkv + static_cast<int64_t>(g) * ccap) + j) * kHeadDim;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int d = 0; d < kHeadDim; d += 4) {
            float kv[4];
            load4(row + d, kv);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float* qh = qs[w + 4 * u];
                acc[u] = fmaf(qh[d], kv[0], acc[u]);
                acc[u] = fmaf(qh[d + 1], kv[1], acc[u]);
                acc[u] = fmaf(qh[d + 2], kv[2], acc[u]);
                acc[u] = fmaf(qh[d + 3], kv[3], acc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            z[u] = score_scale * acc[u];
            logits[(bg * kGroup + w + 4 * u) * nc_ld + j] = z[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) z[u] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float mx = wave_max(z[u]);
        const float e = (j < nvis) ? expf(z[u] - mx) : 0.f;
        const float sm = wave_sum(e);
        if (lane == 0) partial[(bg * nchunk + ch) * kGroup + w + 4 * u] = make_float2(mx, sm);
    }

}

// ------------------------------------------------------------------ decode step: the newest kernel
// The compressed key of kernel j_new (the one token n - 1 completes) from the
// cached keys: float64 sum of its p rows, rounded once, as infv2_compress_keys
// does (a sum of bf16 rows is exact in float64, so the order does not matter).
// kThreads threads: thread t sums d-octet t % 16 over rows t / 16,
// t / 16 + kThreads / 16, ...; stores the key to ck_w[dst ..] and its stored
// value, widened, to fkey.  Called by the whole block; ends with a barrier.
template <bool kCkBf16, int kThreads>
__device__ __forceinline__ void new_compressed_key(const bf16_t* __restrict__ src, int p,
                                                   double (*fpart)[kHeadDim], float* fkey,
                                                   void* __restrict__ ck_w, size_t dst,
                                                   const bf16_t* __restrict__ newest) {
    constexpr int kParts = kThreads / 16;            // row groups
    const int t = threadIdx.x, oc = t & 15, rg = t >> 4;
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int r0 = rg; r0 < p; r0 += 4 * kParts) {    // four rows per batch of loads
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + kParts * u;
            // the last row is the newest token, read from the step's input when
            // it is being appended in the same launch
            const bf16_t* row = (newest && r == p - 1) ? newest : src + static_cast<size_t>(r) * kHeadDim;
            x[u] = r < p ? ldg16(row + 8 * oc) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t w4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += static_cast<double>(__uint_as_float(w4[e] << 16));
                acc[2 * e + 1] += static_cast<double>(__uint_as_float(w4[e] & 0xffff0000u));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) fpart[rg][8 * oc + e] = acc[e];
    __syncthreads();
    if (t < kHeadDim) {
        double sum = 0.0;
#pragma unroll
        for (int x = 0; x < kParts; ++x) sum += fpart[x][t];
        const double mean = sum / static_cast<double>(p);
        if (kCkBf16) {
            const bf16_t h = f64_to_bf16(mean);
            static_cast<bf16_t*>(ck_w)[dst + t] = h;
            fkey[t] = bf16_to_f32(h);
        } else {
            const float f = static_cast<float>(mean);
            static_cast<float*>(ck_w)[dst + t] = f;
            fkey[t] = f;
        }
    }
    __syncthreads();
}

// the A-operand registers of a compressed-key row held widened in LDS (f), for
// the lane of 8-dim group lg: bf16 keys 4 x 16 B, fp32 keys 8 x 16 B
template <bool kCkBf16, int kU>
__device__ __forceinline__ void key_regs_from(const float* f, int lg, uint4 (&raw)[kU]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float* x = &f[32 * ks + 8 * lg];
        if (kCkBf16) {
            raw[ks] = make_uint4(pack_exact(x[0], x[1]), pack_exact(x[2], x[3]),
                                 pack_exact(x[4], x[5]), pack_exact(x[6], x[7]));
        } else {
            raw[2 * ks] = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                     __float_as_uint(x[2]), __float_as_uint(x[3]));
            raw[2 * ks + 1] = make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]),
                                         __float_as_uint(x[6]), __float_as_uint(x[7]));
        }
    }
}

// Z^T tile (16 kernels x 16 heads) from the A-operand registers: bf16 keys one
// MFMA per 32-dim step; fp32 keys split into bf16 hi + lo (x = hi + lo +
// O(2^-17 |x|)), two MFMAs per step, products exact in fp32
template <bool kCkBf16, int kU>
__device__ __forceinline__ f32x4_t key_tile_logits(const uint4 (&raw)[kU], const bf16x8_t (&qf)[4]) {
    f32x4_t zt = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (kCkBf16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) zt = mfma32(as_bf16x8(raw[ks]), qf[ks], zt);
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 a = raw[2 * ks], c = raw[2 * ks + 1];
            const float x[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w),
                                __uint_as_float(c.x), __uint_as_float(c.y), __uint_as_float(c.z), __uint_as_float(c.w)};
            float hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = bf16_to_f32(f32_to_bf16(x[e]));
                lo[e] = x[e] - hi[e];
            }
            uint4 uh, ul;
            uh.x = pack_exact(hi[0], hi[1]); uh.y = pack_exact(hi[2], hi[3]);
            uh.z = pack_exact(hi[4], hi[5]); uh.w = pack_exact(hi[6], hi[7]);
            ul.x = pack_rne(lo[0], lo[1]); ul.y = pack_rne(lo[2], lo[3]);
            ul.z = pack_rne(lo[4], lo[5]); ul.w = pack_rne(lo[6], lo[7]);
            zt = mfma32(as_bf16x8(uh), qf[ks], zt);
            zt = mfma32(as_bf16x8(ul), qf[ks], zt);
        }
    }
    return zt;
}

// ------------------------------------------------------------------ decode, pass 1 on the matrix cores
// kLogWaves waves per block score 64 kernels (64 / kLogWaves each).  Z^T[kernel][head] = CK (64x128) . Q^T:
// the compressed keys are the A operand as stored (lane: 8 consecutive d of one
// kernel); fp32 keys are split into bf16 hi + lo (x = hi + lo + O(2^-17 |x|)),
// two MFMAs per tile, products exact in fp32.  Z^T puts one head per lane column.
//
// kNt: nontemporal loads of the compressed keys.  They stream faster when the
// grid is small (one sequence: a few hundred blocks) and slower when thousands
// of blocks read at once (a batch), so the launcher picks by grid size.
//
// kFuse (decode step): the block whose chunk holds the kernel that the newest
// token n - 1 completes (n >= p, s divides n - p) first computes that kernel's
// compressed key from the cached keys -- float64 sum of the p rows, rounded
// once, as infv2_compress_keys does -- stores it for later steps, and scores it
// from LDS, so the step needs no separate compression launch.
template <bool kCkBf16, bool kFuse, bool kNt>
__global__ __launch_bounds__(kLogWaves * 64) void sel_dec_logits_mfma(
    const bf16_t* __restrict__ q, const void* __restrict__ ck, const int64_t* __restrict__ ck_off,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ lens, int lens_end, int hq,
    int hkv, int p, int s, float score_scale, int64_t nc_max, int64_t nc_ld, int nchunk,
    int64_t nblk_max, int64_t kld, float* __restrict__ logits, float2* __restrict__ partial,
    uint32_t* __restrict__ keys, const bf16_t* __restrict__ kcache, void* __restrict__ ck_w,
    const bf16_t* __restrict__ knew, const bf16_t* __restrict__ vnew, bf16_t* __restrict__ kapp,
    bf16_t* __restrict__ vapp) {
    __shared__ float2 xm[kLogWaves][kGroup];   // each wave's (max, sum) per head
    constexpr int kFuseParts = kLogWaves * 64 / 16;     // row groups of the fused key sum
    __shared__ double fpart[kFuse ? kFuseParts : 1][kHeadDim];
    __shared__ float fkey[kHeadDim];                    // the new key as stored, widened
    const int b = blockIdx.z, g = blockIdx.y, ch = blockIdx.x, t = threadIdx.x;
    const int l = t & 63, wv = t >> 6, lg = l >> 4, lc = l & 15;
    // round trip 1: offsets, length and the queries (independent loads)
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
    const int64_t c0 = ck_off[b], c1 = ck_off[b + 1];
    const bf16_t* qrow = q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    const int64_t n = seq_len(o0, o1, lv, lens_end);
    const int64_t ccap = c1 - c0;
    int64_t nvis = num_kernels(n, p, s);           // row n-1 sees every complete kernel
    nvis = nvis < ccap ? nvis : ccap;
    nvis = nvis < nc_max ? nvis : nc_max;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const int64_t j0 = static_cast<int64_t>(ch) * kChunkA;
    const int64_t cbase = (c0 * hkv + static_cast<int64_t>(g) * ccap);
    // round trip 2: both tiles of the wave (kernels j0 + 16 mt + lc, rows clamped
    // to the last visible kernel; a tile wholly past it loads nothing)
    constexpr int kU = kCkBf16 ? 4 : 8;             // 16-byte loads per tile and lane
    uint4 raw[kLogTiles][kU];
#pragma unroll
    for (int m2 = 0; m2 < kLogTiles; ++m2) {
        const int mt = kLogTiles * wv + m2;
        int64_t j = j0 + 16 * mt + lc;
        j = j < nvis ? j : nvis - 1;
        if (j0 + 16 * mt < nvis) {                  // wave-uniform
            if (kCkBf16) {
                const bf16_t* row = static_cast<const bf16_t*>(ck) + (cbase + j) * kHeadDim + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) raw[m2][ks] = kNt ? ldg16_nt(row + 32 * ks) : ldg16(row + 32 * ks);
            } else {
                const float* row = static_cast<const float*>(ck) + (cbase + j) * kHeadDim + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    raw[m2][2 * ks] = kNt ? ldg16_nt(row + 32 * ks) : ldg16(row + 32 * ks);
                    raw[m2][2 * ks + 1] = kNt ? ldg16_nt(row + 32 * ks + 4) : ldg16(row + 32 * ks + 4);
                }
            }
        } else {
#pragma unroll
            for (int x = 0; x < kU; ++x) raw[m2][x] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    // appending step (lens_end = 2, lv = the length before the step): the new
    // token enters the caches at position lv when there is room; the block of
    // chunk 0 writes it, and the compression below takes that row from the input
    const bool app = kFuse && knew != nullptr && lv < o1 - o0;
    if (app && ch == 0 && t < 32) {
        const size_t sx = (static_cast<size_t>(b) * hkv + g) * kHeadDim + 8 * (t & 15);
        const size_t dx = (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * (o1 - o0) +
                           static_cast<size_t>(lv)) * kHeadDim + 8 * (t & 15);
        if (t < 16) *reinterpret_cast<uint4*>(kapp + dx) = *reinterpret_cast<const uint4*>(knew + sx);
        else *reinterpret_cast<uint4*>(vapp + dx) = *reinterpret_cast<const uint4*>(vnew + sx);
    }
    // fused compression: the kernel j_new = nvis - 1 completed by token n - 1
    const int64_t j_new = nvis - 1;
    const bool fuse = kFuse && n >= p && (n - p) % s == 0 && j_new < ccap && j_new >= j0 &&
                      j_new < j0 + kChunkA;               // uniform over the block
    if (kFuse && fuse) {
        const bf16_t* src = kcache + (static_cast<size_t>(o0) * hkv + static_cast<size_t>(g) * (o1 - o0) +
                                      static_cast<size_t>(j_new) * s) * kHeadDim;
        new_compressed_key<kCkBf16, kLogWaves * 64>(src, p, fpart, fkey, ck_w,
                                                    static_cast<size_t>(cbase + j_new) * kHeadDim,
                                                    app ? knew + (static_cast<size_t>(b) * hkv + g) * kHeadDim
                                                        : nullptr);
        // the lanes holding row j_new take it from LDS instead of the stale load
#pragma unroll
        for (int m2 = 0; m2 < kLogTiles; ++m2) {
            const int mt = kLogTiles * wv + m2;
            if (j0 + 16 * mt + lc == j_new) key_regs_from<kCkBf16>(fkey, lg, raw[m2]);
        }
    }
    // clear this block's share of the block-score keys (filled by pass 2)
    {
        uint32_t* kb = keys + bg * kld;
        const int64_t per = (nblk_max + nchunk - 1) / nchunk;
        const int64_t e = (ch + 1) * per < nblk_max ? (ch + 1) * per : nblk_max;
        for (int64_t j = ch * per + t; j < e; j += kLogWaves * 64) kb[j] = 0u;
    }
    // Z^T tiles
    f32x4_t z[kLogTiles];
#pragma unroll
    for (int m2 = 0; m2 < kLogTiles; ++m2) z[m2] = key_tile_logits<kCkBf16>(raw[m2], qf);
    // lane holds Z[head lc][kernel j0 + 16 mt + 4 lg + r]
    float mx = -INFINITY;
#pragma unroll
    for (int m2 = 0; m2 < kLogTiles; ++m2) {
        const int mt = kLogTiles * wv + m2;
        const int64_t jb = j0 + 16 * mt + 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = (jb + r < nvis) ? score_scale * z[m2][r] : -INFINITY;
            z[m2][r] = v;
            mx = fmaxf(mx, v);
        }
        float* dst = logits + (bg * kGroup + lc) * nc_ld + jb;
        if (jb + 3 < nvis) {
            *reinterpret_cast<float4*>(dst) = make_float4(z[m2][0], z[m2][1], z[m2][2], z[m2][3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) if (jb + r < nvis) dst[r] = z[m2][r];
        }
    }
    mx = max_xor32(max_xor16(mx));
    float sm = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int m2 = 0; m2 < kLogTiles; ++m2)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm += fast_exp2((z[m2][r] - mx) * kLog2eF);   // exp(-inf) = 0
    }
    sm = add_xor32(add_xor16(sm));
    // the waves' (max, sum) of each head combine into the chunk's partial
    if (lg == 0) xm[wv][lc] = make_float2(mx, sm);
    __syncthreads();
    if (wv == 0 && lg == 0) {
        float m2 = -INFINITY;
#pragma unroll
        for (int x = 0; x < kLogWaves; ++x) m2 = fmaxf(m2, xm[x][lc].x);
        float s2 = 0.f;
        if (m2 != -INFINITY) {
#pragma unroll
            for (int x = 0; x < kLogWaves; ++x) {
                const float2 o = xm[x][lc];
                s2 += (o.x == -INFINITY) ? 0.f : o.y * fast_exp2((o.x - m2) * kLog2eF);
            }
        }
        partial[(bg * nchunk + ch) * kGroup + lc] = make_float2(m2, s2);
    }

}

// ------------------------------------------------------------------ decode, pass 2
// Per-head LogSumExp from pass 1's per-chunk (max, sum-exp) partials of one
// (sequence, KV head): called by 256 threads, 16 per head; thread t folds head
// t / 16 and the result is valid in every thread of that head.
__device__ __forceinline__ float fold_partials(const float2* __restrict__ pp, int nchunk, int t) {
    const int r = t & 15;
    constexpr int kPer = 8;              // partials per thread and load batch (128 chunks)
    // loads are unconditional (index clamped, value masked after): no branch, so
    // a batch is in flight at once (and the first batch with the caller's loads)
    auto batch = [&](int base, float2 (&pm)[kPer]) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = base + r + 16 * u;
            pm[u] = pp[static_cast<size_t>(c < nchunk ? c : nchunk - 1) * kGroup];
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (base + r + 16 * u >= nchunk) pm[u] = make_float2(-INFINITY, 0.f);
    };
    float2 pm[kPer];
    batch(0, pm);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) mx = fmaxf(mx, pm[u].x);
    for (int base = 16 * kPer; base < nchunk; base += 16 * kPer) {      // beyond 128 chunks
        float2 px[kPer];
        batch(base, px);
#pragma unroll
        for (int u = 0; u < kPer; ++u) mx = fmaxf(mx, px[u].x);
    }
    mx = max16(mx);
    float sm = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) sm += (pm[u].x == -INFINITY) ? 0.f : pm[u].y * fast_exp2((pm[u].x - mx) * kLog2eF);
        for (int base = 16 * kPer; base < nchunk; base += 16 * kPer) {
            float2 px[kPer];
            batch(base, px);
#pragma unroll
            for (int u = 0; u < kPer; ++u) sm += (px[u].x == -INFINITY) ? 0.f : px[u].y * fast_exp2((px[u].x - mx) * kLog2eF);
        }
    }
    sm = sum16(sm);
    return (mx == -INFINITY) ? -INFINITY : mx + __log2f(sm) * kLn2F;
}

// lse_in: a per-(sequence, KV head, head) normaliser to use instead of the one
// folded from `partial` (the coarse-kernel approximation), or NULL.
// kJ kernels per thread: 256 kJ kernels per block (kJ = 4 for large grids:
// a quarter of the blocks, so a quarter of the re-reads of the partials).
template <int kJ>
__global__ __launch_bounds__(256) void sel_dec_scores(
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ lens, int lens_end,
    const int64_t* __restrict__ ck_off, int hkv, int m, int p, int s, int64_t nc_max,
    int64_t nc_ld, int nchunk_a, int64_t kld, const float* __restrict__ logits,
    const float2* __restrict__ partial, const float* __restrict__ lse_in,
    uint32_t* __restrict__ keys) {
    __shared__ float ls[kGroup];
    constexpr int kCh = 256 * kJ;                 // kernels per block
    __shared__ float rs[kCh];
    const int b = blockIdx.z, g = blockIdx.y, ch = blockIdx.x, t = threadIdx.x;
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
    const int64_t c0 = ck_off[b], c1 = ck_off[b + 1];
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    uint32_t* kb = keys + bg * kld;
    const int64_t j0 = static_cast<int64_t>(ch) * kCh;

    // this thread's 16 logits and the (max, sum-exp) partials are independent
    // loads: issue them together (one memory round trip)
    float zz[kJ][kGroup];
#pragma unroll
    for (int x = 0; x < kJ; ++x) {
        // clamped to the row, not to nvis: the address does not wait for the length
        const int64_t j = j0 + t + 256 * x;
        const float* z = logits + bg * kGroup * nc_ld + (j < nc_ld ? j : nc_ld - 1);
#pragma unroll
        for (int h = 0; h < kGroup; ++h) zz[x][h] = z[h * nc_ld];
    }
    // per-head LogSumExp from the partials of pass 1 (16 threads per head)
    if (lse_in) {
        if (t < kGroup) ls[t] = lse_in[bg * kGroup + t];
    } else {
        const float v = fold_partials(partial + bg * nchunk_a * kGroup + (t >> 4), nchunk_a, t);
        if ((t & 15) == 0) ls[t >> 4] = v;
    }
    const int64_t n = seq_len(o0, o1, lv, lens_end);
    const int64_t ccap = c1 - c0;
    int64_t nvis = num_kernels(n, p, s);
    nvis = nvis < ccap ? nvis : ccap;
    nvis = nvis < nc_max ? nvis : nc_max;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kJ; ++x) {
        const int64_t j = j0 + t + 256 * x;
        float R = -INFINITY;
        if (j < nvis) {
            float acc = 0.f;
#pragma unroll
            for (int h = 0; h < kGroup; ++h) acc += fast_exp2((zz[x][h] - ls[h]) * kLog2eF);
            R = acc * (1.0f / kGroup);
        }
        rs[t + 256 * x] = R;
    }
    __syncthreads();
    const int64_t jhi = (j0 + kCh < nvis ? j0 + kCh : nvis) - 1;
    if (j0 <= jhi) {
        const int64_t blo = (j0 * s) / m, bhi = (jhi * s + p - 1) / m;
        for (int64_t blk = blo + t; blk <= bhi; blk += 256) {
            int64_t k0 = first_kernel_of_block(blk, m, p, s), k1 = last_kernel_of_block(blk, m, s);
            k0 = k0 > j0 ? k0 : j0;
            k1 = k1 < jhi ? k1 : jhi;
            if (k0 > k1) continue;
            float mx = rs[k0 - j0];
            for (int64_t kk = k0 + 1; kk <= k1; ++kk) mx = fmaxf(mx, rs[kk - j0]);
            atomicMax(&kb[blk], score_to_key(mx));
        }
    }
}

// ------------------------------------------------------------------ decode, coarse LSE
// "Efficient LSE approximation": the per-head normaliser of a (sequence, KV
// head) from the partials of pass 1 run over the coarse kernels (size and
// stride `coarse`); a row that sees no coarse kernel keeps the exact one from
// the fine partials.  grid (KV head, sequence), 256 threads.
__global__ __launch_bounds__(256) void sel_dec_lse_coarse(
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ kv_lens,
    const int64_t* __restrict__ ckc_off, int hkv, int coarse, int nchunk_c, int nchunk_f,
    const float2* __restrict__ partial_c, const float2* __restrict__ partial_f,
    float* __restrict__ lse_out) {
    const int b = blockIdx.y, g = blockIdx.x, t = threadIdx.x;
    const int64_t cap = kv_off[b + 1] - kv_off[b];
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const int64_t ccap = ckc_off[b + 1] - ckc_off[b];
    int64_t nvis = num_kernels(n, coarse, coarse);
    nvis = nvis < ccap ? nvis : ccap;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const float v = nvis > 0 ? fold_partials(partial_c + bg * nchunk_c * kGroup + (t >> 4), nchunk_c, t)
                             : fold_partials(partial_f + bg * nchunk_f * kGroup + (t >> 4), nchunk_f, t);
    if ((t & 15) == 0) lse_out[bg * kGroup + (t >> 4)] = v;
}

// ------------------------------------------------------------------ decode, top-k
// Thread t owns blocks [t kPer, t kPer + kPer) of the (sequence, KV head); the key
// row is padded to 256 kPer entries, so the keys load as whole vectors with no
// bounds, in the same memory round trip as the offsets and the length.
template <int kPer>
__global__ __launch_bounds__(256) void sel_dec_topk(const int64_t* __restrict__ kv_off,
                                                    const int64_t* __restrict__ lens, int lens_end,
                                                    int hkv, int m, int topk, int init, int local,
                                                    int64_t nblk_max, int64_t kld,
                                                    const uint32_t* __restrict__ keys,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ score) {
    static_assert(kPer % 2 == 0, "keys load in pairs");
    __shared__ TopkSmem<256> sm;
    const int b = blockIdx.y, g = blockIdx.x;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const int jb = static_cast<int>(threadIdx.x) * kPer;
    const uint32_t* gk = keys + bg * kld + jb;
    const int64_t o0 = kv_off[b], o1 = kv_off[b + 1], lv = lens[b];
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
    const int64_t n = seq_len(o0, o1, lv, lens_end);
    int64_t c = n > 0 ? (n - 1) / m : -1;
    c = c < nblk_max - 1 ? c : nblk_max - 1;
    int cnt = static_cast<int>(c + 1) - jb;
    cnt = cnt < 0 ? 0 : (cnt > kPer ? kPer : cnt);
    block_topk_regs<256>(key, jb, cnt, static_cast<int>(c), topk, init, local, idx + bg * topk,
                         score ? score + bg * topk : nullptr, sm);
}

// ------------------------------------------------------------------ prefill, pass 1
template <typename Tq, typename Tck>
__device__ __forceinline__ void load_ck_tile(float (*cks)[kHeadDim + 1], const Tck* base,
                                             int64_t j0, int64_t jn) {
    // rows j0 .. j0+63 (those < jn) of a [.][128] compressed-key array into LDS
    for (int e = threadIdx.x * 4; e < kTilePre * kHeadDim; e += 256 * 4) {
        const int r = e / kHeadDim, c = e % kHeadDim;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (j0 + r < jn) load4(base + (j0 + r) * kHeadDim + c, v);
        cks[r][c] = v[0]; cks[r][c + 1] = v[1]; cks[r][c + 2] = v[2]; cks[r][c + 3] = v[3];
    }
}

template <typename Tq, typename Tck>
__global__ __launch_bounds__(256) void sel_pre_lse(
    const Tq* __restrict__ q, int rows, int64_t q_start, const Tck* __restrict__ ck,
    const int64_t* __restrict__ ck_off, int hq, int hkv, int p, int s, float score_scale,
    int64_t nblk_max, float* __restrict__ lse, uint32_t* __restrict__ keys) {
    __shared__ float qs[kRowsPre][kGroup][kHeadDim];
    __shared__ float cks[kTilePre][kHeadDim + 1];
    const int g = blockIdx.y, t = threadIdx.x;
    const int r0 = blockIdx.x * kRowsPre;
    const int64_t ccap = ck_off[1] - ck_off[0];
    const Tck* ckh = ck + (ck_off[0] * hkv + static_cast<int64_t>(g) * ccap) * kHeadDim;
    int64_t vis[kRowsPre];
    int64_t vmax = 0;
#pragma unroll
    for (int rr = 0; rr < kRowsPre; ++rr) {
        const int row = r0 + rr;
        int64_t v = row < rows ? num_kernels(q_start + row + 1, p, s) : 0;
        v = v < ccap ? v : ccap;
        vis[rr] = v;
        vmax = v > vmax ? v : vmax;
        if (row < rows) {
            uint32_t* kb = keys + (static_cast<size_t>(row) * hkv + g) * nblk_max;
            for (int64_t jb = t; jb < nblk_max; jb += 256) kb[jb] = 0u;
        }
    }
    for (int e = t; e < kRowsPre * kGroup * kHeadDim; e += 256) {
        const int rr = e / (kGroup * kHeadDim), rem = e % (kGroup * kHeadDim);
        const int row = r0 + rr;
        qs[rr][rem / kHeadDim][rem % kHeadDim] =
            row < rows ? io<Tq>::load(q + (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim + rem) : 0.f;
    }
    const int w = t >> 6, lane = t & 63;
    // this thread's 16 (row, head) pairs: pair u -> row u/4, head w + 4*(u%4)
    float mrun[16], lrun[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) { mrun[u] = -INFINITY; lrun[u] = 0.f; }
    for (int64_t j0 = 0; j0 < vmax; j0 += kTilePre) {
        __syncthreads();
        load_ck_tile<Tq, Tck>(cks, ckh, j0, vmax);
        __syncthreads();
        const int64_t j = j0 + lane;
        float acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = 0.f;
        for (int d = 0; d < kHeadDim; ++d) {
            const float kd = cks[lane][d];
#pragma unroll
            for (int u = 0; u < 16; ++u) acc[u] = fmaf(qs[u >> 2][w + 4 * (u & 3)][d], kd, acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (j < vis[u >> 2]) {
                const float z = score_scale * acc[u];
                if (z > mrun[u]) {
                    lrun[u] = lrun[u] * expf(mrun[u] - z) + 1.f;
                    mrun[u] = z;
                } else {
                    lrun[u] += expf(z - mrun[u]);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float mx = wave_max(mrun[u]);
        const float part = (mrun[u] == -INFINITY) ? 0.f : lrun[u] * expf(mrun[u] - mx);
        const float sm = wave_sum(part);
        const int row = r0 + (u >> 2);
        if (lane == 0 && row < rows)
            lse[static_cast<size_t>(row) * hq + g * kGroup + w + 4 * (u & 3)] =
                (mx == -INFINITY) ? -INFINITY : mx + logf(sm);
    }
}

// ------------------------------------------------------------------ prefill, pass 2
template <typename Tq, typename Tck>
__global__ __launch_bounds__(256) void sel_pre_scores(
    const Tq* __restrict__ q, int rows, int64_t q_start, const Tck* __restrict__ ck,
    const int64_t* __restrict__ ck_off, int hq, int hkv, int m, int p, int s, float score_scale,
    int64_t nblk_max, const float* __restrict__ lse, uint32_t* __restrict__ keys) {
    __shared__ float qs[kRowsPre][kGroup][kHeadDim];
    __shared__ float cks[kTilePre][kHeadDim + 1];
    __shared__ float rs[kRowsPre][kTilePre];
    __shared__ float ls[kRowsPre][kGroup];
    const int g = blockIdx.y, t = threadIdx.x;
    const int r0 = blockIdx.x * kRowsPre;
    const int64_t ccap = ck_off[1] - ck_off[0];
    const Tck* ckh = ck + (ck_off[0] * hkv + static_cast<int64_t>(g) * ccap) * kHeadDim;
    const int w = t >> 6, lane = t & 63;       // wave w owns row r0 + w
    const int row = r0 + w;
    int64_t vmax = 0;
    for (int rr = 0; rr < kRowsPre; ++rr) {
        int64_t v = (r0 + rr) < rows ? num_kernels(q_start + r0 + rr + 1, p, s) : 0;
        v = v < ccap ? v : ccap;
        vmax = v > vmax ? v : vmax;
    }
    int64_t vis = row < rows ? num_kernels(q_start + row + 1, p, s) : 0;
    vis = vis < ccap ? vis : ccap;
    for (int e = t; e < kRowsPre * kGroup * kHeadDim; e += 256) {
        const int rr = e / (kGroup * kHeadDim), rem = e % (kGroup * kHeadDim);
        const int rw = r0 + rr;
        qs[rr][rem / kHeadDim][rem % kHeadDim] =
            rw < rows ? io<Tq>::load(q + (static_cast<size_t>(rw) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim + rem) : 0.f;
    }
    if (t < kRowsPre * kGroup) {
        const int rw = r0 + t / kGroup;
        ls[t / kGroup][t % kGroup] = rw < rows ? lse[static_cast<size_t>(rw) * hq + g * kGroup + t % kGroup] : 0.f;
    }
    uint32_t* kb = keys + (static_cast<size_t>(row < rows ? row : 0) * hkv + g) * nblk_max;
    for (int64_t j0 = 0; j0 < vmax; j0 += kTilePre) {
        __syncthreads();
        load_ck_tile<Tq, Tck>(cks, ckh, j0, vmax);
        __syncthreads();
        const int64_t j = j0 + lane;
        float acc[kGroup];
#pragma unroll
        for (int h = 0; h < kGroup; ++h) acc[h] = 0.f;
        for (int d = 0; d < kHeadDim; ++d) {
            const float kd = cks[lane][d];
#pragma unroll
            for (int h = 0; h < kGroup; ++h) acc[h] = fmaf(qs[w][h][d], kd, acc[h]);
        }
        float R = -INFINITY;
        if (j < vis) {
            float sum = 0.f;
#pragma unroll
            for (int h = 0; h < kGroup; ++h) sum += expf(score_scale * acc[h] - ls[w][h]);
            R = sum * (1.0f / kGroup);
        }
        rs[w][lane] = R;
        __syncthreads();
        const int64_t jhi = (j0 + kTilePre < vis ? j0 + kTilePre : vis) - 1;
        if (row < rows && j0 <= jhi) {
            const int64_t blo = (j0 * s) / m, bhi = (jhi * s + p - 1) / m;
            for (int64_t blk = blo + lane; blk <= bhi; blk += 64) {
                int64_t k0 = first_kernel_of_block(blk, m, p, s), k1 = last_kernel_of_block(blk, m, s);
                k0 = k0 > j0 ? k0 : j0;
                k1 = k1 < jhi ? k1 : jhi;
                if (k0 > k1) continue;
                float mx = rs[w][k0 - j0];
                for (int64_t kk = k0 + 1; kk <= k1; ++kk) mx = fmaxf(mx, rs[w][kk - j0]);
                atomicMax(&kb[blk], score_to_key(mx));
            }
        }
    }
}

// ------------------------------------------------------------------ prefill passes on the matrix cores
// Thread block = 16 query rows of one KV head (8 waves, wave w: rows w, w + 8),
// streaming the compressed keys in tiles of 64 kernels through two LDS stages
// by direct global->LDS loads (bf16 keys as stored; fp32 keys as the hi + lo
// bf16 rows ck_split_hilo writes once per call).  Z[head][kernel] = Q . CK^T with Q
// as the A operand (lane: head lc, 8 consecutive d) and the CK tile as B, so
// each lane holds 4 heads (4 lg + r) of one kernel column (lc) per 16x16 tile.
//   pass 1: per-lane online (max, sum) of 2^(log2e z) per head, folded over
//           the 16 kernel columns at the end -> LSE[row][head]
//   pass 2: R = mean_h 2^(log2e z - LSE2_h): 4 heads in-lane + two cross-lane
//           adds; block max of R over the tile, atomicMax into the row's keys
constexpr int kPreRowsG = 16;
static_assert(kPreRowsG == 16, "the launch tables count groups of 16 rows");
constexpr int kPreTileK = 64;
constexpr int kPreWaves = 8;                          // wave w: rows w + 8 i
constexpr int kPreRW = kPreRowsG / kPreWaves;         // query rows per wave
constexpr int kPreThreads = kPreWaves * 64;
constexpr int kPreLoads = kPreTileK * 16 / kPreThreads;   // 16-byte loads per thread, tile and part
constexpr float kPreMrInit = -1e30f;                  // pass 1 reference before any visible logit

// fp32 compressed keys -> the bf16 pair the scoring products use, for x = the
// key times zs = score_scale log2 e (one fp32 rounding): hi = x rounded to
// bf16, lo = (x - hi) rounded to bf16, so that hi . q + lo . q carries x to
// about 16 significant bits and the products give the logit in log2 units.  Written once per call as [part][KV head][ld][d]
// (part 0 hi, 1 lo) for kernels 0 .. nk - 1 (those the call's rows see), instead
// of by every thread block that stages a tile.  Thread -> one 8-value chunk.
__global__ __launch_bounds__(256) void ck_split_hilo(const PrefillSeqs seqs, const float* __restrict__ ck,
                                                     const int64_t* __restrict__ ck_off_all, int hkv,
                                                     int p, int s, int64_t ld, float zs,
                                                     bf16_t* __restrict__ hl_all) {
    const int g = blockIdx.y, si = blockIdx.z;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t* ck_off = ck_off_all + seqs.seq[si];
    const int64_t ccap = ck_off[1] - ck_off[0];
    const int64_t nk = num_kernels(seqs.q_start[si] + seqs.rows[si], p, s);   // kernels its rows see
    bf16_t* hl = hl_all + static_cast<int64_t>(si) * 2 * hkv * ld * kHeadDim;
    const int64_t r = e >> 4;
    const int c = static_cast<int>(e & 15);
    if (r >= nk || r >= ccap || r >= ld) return;
    const float* src = ck + (ck_off[0] * hkv + static_cast<int64_t>(g) * ccap + r) * kHeadDim + 8 * c;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    const float x[8] = {a.x * zs, a.y * zs, a.z * zs, a.w * zs, b.x * zs, b.y * zs, b.z * zs, b.w * zs};
    float hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = bf16_to_f32(f32_to_bf16(x[i]));
        lo[i] = x[i] - hi[i];
    }
    const int64_t o = (static_cast<int64_t>(g) * ld + r) * kHeadDim + 8 * c;
    *reinterpret_cast<uint4*>(hl + o) =
        make_uint4(pack_exact(hi[0], hi[1]), pack_exact(hi[2], hi[3]), pack_exact(hi[4], hi[5]), pack_exact(hi[6], hi[7]));
    *reinterpret_cast<uint4*>(hl + static_cast<int64_t>(hkv) * ld * kHeadDim + o) =
        make_uint4(pack_rne(lo[0], lo[1]), pack_rne(lo[2], lo[3]), pack_rne(lo[4], lo[5]), pack_rne(lo[6], lo[7]));
}

template <int kPass, bool kCkBf16>
__global__ __launch_bounds__(kPreThreads, 4) void sel_pre_mfma(
    const PrefillSeqs seqs, const bf16_t* __restrict__ q_all, const void* __restrict__ ck,
    const int64_t* __restrict__ ck_off_all, const bf16_t* __restrict__ hl_all, int64_t ld, int hq,
    int hkv, int m, int p, int s, float score_scale, int64_t nblk_max, float* __restrict__ lse_all,
    uint32_t* __restrict__ keys_all) {
    // two stages of 64-kernel tiles: bf16 keys, or the hi and lo parts of fp32 keys
    __shared__ __attribute__((aligned(16))) bf16_t ck_hi[2][kPreTileK * kHeadDim];
    __shared__ __attribute__((aligned(16))) bf16_t ck_lo[kCkBf16 ? 1 : 2][kCkBf16 ? 8 : kPreTileK * kHeadDim];
    __shared__ float rs[kPreRowsG][kPreTileK + 1];   // +1: column reads across rows conflict-free
    __shared__ int32_t vrow[kPreRowsG];              // kernels visible to each row
    __shared__ int32_t bk[kPreThreads][2];                   // pass 2: tile-relative kernel range per block
    const int g = blockIdx.y, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    // this block's sequence and its row group
    const int grp = static_cast<int>(blockIdx.x);
    const int si = seq_of_group(seqs, grp);
    const int r0 = (grp - (si > 0 ? seqs.grp_end[si - 1] : 0)) * kPreRowsG;
    const int rows = seqs.rows[si];
    const int64_t q_start = seqs.q_start[si];
    const size_t row0 = static_cast<size_t>(seqs.row0[si]);
    const bf16_t* q = q_all + row0 * hq * kHeadDim;
    float* lse = lse_all + row0 * hq;
    uint32_t* keys = keys_all + row0 * hkv * nblk_max;
    const int64_t* ck_off = ck_off_all + seqs.seq[si];
    const bf16_t* hl = kCkBf16 ? nullptr : hl_all + static_cast<int64_t>(si) * 2 * hkv * ld * kHeadDim;
    const int64_t ccap = ck_off[1] - ck_off[0];
    // kernel rows of this KV head: the bf16 keys as stored, or the hi / lo rows
    // that ck_split_hilo wrote for fp32 keys ([part][KV head][ld][d])
    const bf16_t* src_hi = kCkBf16 ? static_cast<const bf16_t*>(ck) + (ck_off[0] * hkv + static_cast<int64_t>(g) * ccap) * kHeadDim
                                   : hl + static_cast<int64_t>(g) * ld * kHeadDim;
    const bf16_t* src_lo = kCkBf16 ? nullptr : hl + (static_cast<int64_t>(hkv) + g) * ld * kHeadDim;
    constexpr float kLog2e = 1.4426950408889634f;
    const float zscale = score_scale * kLog2e;

    int32_t vis[kPreRW];              // kernels visible to the row (counts < 2^31)
    bf16x8_t qf[kPreRW][4];
    int64_t vmax = 0;                     // the group's last valid row sees the most kernels
    int64_t vmin = 0;                     // and its first row the fewest
    {
        const int64_t v0 = num_kernels(q_start + r0 + 1, p, s);
        vmin = v0 < ccap ? v0 : ccap;
        const int last = (r0 + kPreRowsG - 1 < rows ? r0 + kPreRowsG - 1 : rows - 1);
        if (last >= r0) {
            const int64_t v = num_kernels(q_start + last + 1, p, s);
            vmax = v < ccap ? v : ccap;
        }
    }
#pragma unroll
    for (int i = 0; i < kPreRW; ++i) {
        const int row = r0 + w + kPreWaves * i;
        int64_t v = row < rows ? num_kernels(q_start + row + 1, p, s) : 0;
        vis[i] = static_cast<int32_t>(v < ccap ? v : ccap);
        const int rr = row < rows ? row : rows - 1;
        const bf16_t* qrow = q + (static_cast<size_t>(rr) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[i][ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
    }
    if (t < kPreRowsG) {
        const int row = r0 + t;
        int64_t v = row < rows ? num_kernels(q_start + row + 1, p, s) : 0;
        vrow[t] = static_cast<int32_t>(v < ccap ? v : ccap);
    }
    if (kPass == 1) {
        // pass 1 owns clearing the block-score keys of its rows
        for (int rr = 0; rr < kPreRowsG; ++rr) {
            const int row = r0 + rr;
            if (row >= rows) break;
            uint32_t* kb = keys + (static_cast<size_t>(row) * hkv + g) * nblk_max;
            for (int64_t jb = t; jb < nblk_max; jb += kPreThreads) kb[jb] = 0u;
        }
    }
    // pass 1 state: running (max, sum) for heads 4 lg + r; pass 2: LSE2 of those
    // heads.  The reference is held negated, nm = -reference, as the 4-vector
    // that seeds a column tile's products: with fp32 keys (stored pre-scaled by
    // score_scale log2 e) the products then end at the exponent itself.
    f32x4_t nm[kPreRW];
    float lr[kPreRW][4];
#pragma unroll
    for (int i = 0; i < kPreRW; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) { nm[i][r] = -kPreMrInit; lr[i][r] = 0.f; }
    }
    if (kPass == 2) {
#pragma unroll
        for (int i = 0; i < kPreRW; ++i) {
            const int row = r0 + w + kPreWaves * i;
            const int rr = row < rows ? row : rows - 1;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                nm[i][r] = -(lse[static_cast<size_t>(rr) * hq + g * kGroup + 4 * lg + r] * kLog2e);
        }
    }

    // Tiles stream through LDS with direct global->LDS loads, one tile ahead.
    // Load x of wave w fills 1 KB: tile rows 4 (kPreLoads w + x) .. + 3, lane l
    // writing stored chunk l % 16 of its row, which holds source chunk
    // (l % 16) ^ (row % 16) (chunk c of kernel r sits at c ^ (r & 15)).
    int dr[kPreLoads], dc[kPreLoads];
#pragma unroll
    for (int x = 0; x < kPreLoads; ++x) {
        const int e = (kPreLoads * w + x) * 64 + l;
        dr[x] = e >> 4;
        dc[x] = (e & 15) ^ (dr[x] & 15);
    }
    auto issue = [&](int64_t jt, int stg) {
#pragma unroll
        for (int x = 0; x < kPreLoads; ++x) {
            int64_t r = jt + dr[x];
            r = r < vmax ? r : vmax - 1;         // rows past the last visible kernel are never read
            const int64_t so = r * kHeadDim + 8 * dc[x];
            const int dst = (kPreLoads * w + x) * 512;          // bf16 elements (1 KB)
            dma16(src_hi + so, lds_offset(&ck_hi[stg][dst]));
            if (!kCkBf16) dma16(src_lo + so, lds_offset(&ck_lo[stg][dst]));
        }
    };
    // make the compiler wait for the q fragments and pass 2's normalisers here,
    // where it sees a use: otherwise it keeps them pending into the tile loop and
    // waits there for every outstanding load, the next tile's included
#pragma unroll
    for (int i = 0; i < kPreRW; ++i) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" :: "v"(qf[i][ks]));
        asm volatile("" :: "v"(nm[i]));
    }
    // pass 2: a tile's block-max update (at most one per thread with the usual
    // sizes) is issued after the next tile's loads, so that the wait for those
    // loads at the top of the tile after does not also wait for fresh atomics
    uint32_t* pend = nullptr;
    uint32_t pend_key = 0u;
    if (vmax > 0) issue(0, 0);
    // one 64-kernel tile; kFull (full_tag): every kernel of the tile is visible
    // to every row of the group (all tiles but the last few), so the visibility
    // mask drops out of the column loop
    // kFirst (pass 1, tile 0, masked): the products start from zero
    // Pass 2 passes the stage as a compile-time constant, so that its LDS
    // fragment addresses are lane offsets plus immediates (in pass 1 the second
    // copy of the tile code costs more registers than it saves instructions).
    auto tile = [&](const int64_t j0, auto stg_v, auto full_tag, auto first_tag) {
        const int stg = static_cast<int>(stg_v);
        constexpr bool kFull = decltype(full_tag)::value;
        constexpr bool kFirst = decltype(first_tag)::value;
        // tile j0 landed (with the previous tile's deferred updates, both issued
        // a tile ago) and every wave is done with the previous tile, whose stage
        // now takes the next one
        dma_wait_barrier();
        if (j0 + kPreTileK < vmax) issue(j0 + kPreTileK, stg ^ 1);
        if (kPass == 2 && pend) {
            atomicMax(pend, pend_key);
            pend = nullptr;
        }
        // pass 2: the tile's blocks and their kernel ranges (relative to the tile;
        // 32-bit arithmetic: kernel and block counts are below 2^31), the first
        // kPreThreads blocks here, where the barrier after the products covers them
        const int j0i = static_cast<int>(j0);
        const int jhi_t = static_cast<int>((j0 + kPreTileK < vmax ? j0 + kPreTileK : vmax) - 1);
        const int blo = (j0i * s) / m, bhi = (jhi_t * s + p - 1) / m;
        auto block_ranges = [&](int b0) {
            const int nb = (bhi - b0 + 1) < kPreThreads ? (bhi - b0 + 1) : kPreThreads;
            if (t < nb) {
                const int blk = b0 + t;
                int k0 = blk * m - p;                          // first kernel: floor((blk m - p) / s) + 1, >= 0
                k0 = (k0 >= 0 ? k0 / s : -((-k0 + s - 1) / s)) + 1;
                k0 = k0 > j0i ? k0 : j0i;
                int k1 = ((blk + 1) * m - 1) / s;              // last kernel
                k1 = k1 < jhi_t ? k1 : jhi_t;
                bk[t][0] = k0 - j0i;
                bk[t][1] = k1 - j0i;
            }
        };
        if (kPass == 2) block_ranges(blo);
        // B fragments of a 16-kernel column tile: lane holds CK[kernel 16 nt + lc]
        // [32 ks + 8 lg ..], hi and lo parts, all eight LDS reads issued together
        uint4 fh[1][4], fl[1][4];
        auto frags = [&](int nt, int buf) {
            const int kr = 16 * nt + lc;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = kr * kHeadDim + 8 * ((4 * ks + lg) ^ (kr & 15));
                fh[buf][ks] = *reinterpret_cast<const uint4*>(&ck_hi[stg][off]);
                if (!kCkBf16) fl[buf][ks] = *reinterpret_cast<const uint4*>(&ck_lo[stg][off]);
            }
        };
        // the 16-kernel column tiles of this tile
        {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int cur = 0;
                frags(nt, cur);
                // bf16 keys: raw logits; fp32 keys: the scaled logits minus the
                // reference (the products start from nm), except in pass 1's first
                // tile, whose reference is still the -1e30 placeholder
                f32x4_t z[kPreRW];
#pragma unroll
                for (int i = 0; i < kPreRW; ++i) z[i] = (kCkBf16 || kFirst) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : nm[i];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int i = 0; i < kPreRW; ++i) z[i] = mfma32(qf[i][ks], as_bf16x8(fh[cur][ks]), z[i]);
                    if (!kCkBf16) {
#pragma unroll
                        for (int i = 0; i < kPreRW; ++i) z[i] = mfma32(qf[i][ks], as_bf16x8(fl[cur][ks]), z[i]);
                    }
                }
                const int kr = 16 * nt + lc;
                const int32_t jk = static_cast<int32_t>(j0) + kr;   // this lane's kernel column
#pragma unroll
                for (int i = 0; i < kPreRW; ++i) {
                    const bool ok = kFull || jk < vis[i];
                    if (kPass == 1) {
                        // running (max, sum) with a lazy max: the reference of a head
                        // (shared by its 16 kernel-column lanes) moves only when some
                        // logit exceeds it by more than 2^8, so the common path is one
                        // FMA, one exp and one add per logit and no divergence.
                        // d = logit - reference; masked logits are -inf
                        float d[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            d[r] = !ok ? -INFINITY : kCkBf16 ? fmaf(z[i][r], zscale, nm[i][r])
                                                       : kFirst ? z[i][r] + nm[i][r] : z[i][r];
                        if (__builtin_amdgcn_ballot_w64(d[0] > 8.f || d[1] > 8.f || d[2] > 8.f || d[3] > 8.f) != 0) {
                            // raise the references to the max over the head's 16 columns
                            // (x: the scaled logit; fp32 keys after the first tile:
                            // the products minus the old reference's seed)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float x = !ok ? -INFINITY : kCkBf16 ? z[i][r] * zscale
                                                                : kFirst ? z[i][r] : z[i][r] - nm[i][r];
                                const float cm = max16(x);
                                const float mo = -nm[i][r];
                                const float mn = fmaxf(mo, cm);
                                lr[i][r] = lr[i][r] * fast_exp2(mo - mn);   // finite reference: no NaN
                                nm[i][r] = -mn;
                                d[r] = x - mn;
                            }
                        }
                        // the reference is finite (kPreMrInit at first), so masked logits
                        // (-inf) give 2^-inf = 0 without a test
#pragma unroll
                        for (int r = 0; r < 4; ++r) lr[i][r] += fast_exp2(d[r]);
                    } else {
                        float acc = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc += fast_exp2(kCkBf16 ? fmaf(z[i][r], zscale, nm[i][r]) : z[i][r]);
                        acc = add_xor32(add_xor16(acc));
                        if (lg == 0) rs[w + kPreWaves * i][kr] = ok ? acc * (1.0f / kGroup) : -INFINITY;
                    }
                }
            }
        }
        if (kPass == 2) {
            __syncthreads();
            // block max over this tile's kernels: one (row, block) per thread,
            // rows fastest
            for (int b0 = blo; b0 <= bhi; b0 += kPreThreads) {
                const int nb = (bhi - b0 + 1) < kPreThreads ? (bhi - b0 + 1) : kPreThreads;
                if (b0 != blo) {                  // more blocks than threads: the next ranges
                    block_ranges(b0);
                    __syncthreads();
                }
                for (int e = t; e < kPreRowsG * nb; e += kPreThreads) {
                    const int rr = e & (kPreRowsG - 1), b = e / kPreRowsG, row = r0 + rr;
                    if (row >= rows) continue;
                    const int k0 = bk[b][0];
                    int k1 = bk[b][1];
                    const int kv = vrow[rr] - 1 - j0i;            // last kernel the row sees
                    k1 = k1 < kv ? k1 : kv;
                    if (k0 > k1) continue;
                    float mx = rs[rr][k0];
                    for (int kk = k0 + 1; kk <= k1; ++kk) mx = fmaxf(mx, rs[rr][kk]);
                    uint32_t* dst = &keys[(static_cast<size_t>(row) * hkv + g) * nblk_max + b0 + b];
                    if (!pend) {              // the thread's first update waits for the next tile
                        pend = dst;
                        pend_key = score_to_key(mx);
                    } else {
                        atomicMax(dst, score_to_key(mx));
                    }
                }
                if (b0 + kPreThreads <= bhi) __syncthreads();   // ranges read before they are replaced
            }
        }
    };
    int64_t j0 = 0;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    int stg = 0;
    if (kPass == 1 && vmax > 0) {
        tile(j0, S0{}, std::false_type{}, std::true_type{});
        j0 += kPreTileK;
        stg = 1;
    }
    for (; j0 + kPreTileK <= vmin; j0 += kPreTileK, stg ^= 1) {
        if (kPass == 1) tile(j0, stg, std::true_type{}, std::false_type{});
        else if (stg) tile(j0, S1{}, std::true_type{}, std::false_type{});
        else tile(j0, S0{}, std::true_type{}, std::false_type{});
    }
    for (; j0 < vmax; j0 += kPreTileK, stg ^= 1) {
        if (kPass == 1) tile(j0, stg, std::false_type{}, std::false_type{});
        else if (stg) tile(j0, S1{}, std::false_type{}, std::false_type{});
        else tile(j0, S0{}, std::false_type{}, std::false_type{});
    }
    if (kPass == 2 && pend) atomicMax(pend, pend_key);
    if (kPass == 1) {
        // fold the 16 kernel columns: lanes with equal lg hold the same heads
#pragma unroll
        for (int i = 0; i < kPreRW; ++i) {
            const int row = r0 + w + kPreWaves * i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mo = -nm[i][r];
                float mx = mo;
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
                float sm = lr[i][r] * fast_exp2(mo - mx);   // lanes still at kPreMrInit hold 0
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o, 64);
                if (lc == 0 && row < rows)
                    lse[static_cast<size_t>(row) * hq + g * kGroup + 4 * lg + r] =
                        (mx == kPreMrInit) ? -INFINITY : (mx + __log2f(sm)) * 0.6931471805599453f;
            }
        }
    }
}

// ------------------------------------------------------------------ prefill, top-k
// kThreads = 64 (one wave per row: no cross-wave barriers, every (row, KV head)
// block resident at once) unless a row has too many blocks for 16 per lane.
template <int kThreads, int kPer>
__global__ __launch_bounds__(kThreads) void sel_pre_topk(const PrefillSeqs seqs, int hkv, int m, int topk,
                                                         int init, int local, int64_t nblk_max,
                                                         int per, const uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ score) {
    __shared__ TopkSmem<kThreads> sm;
    const int row = blockIdx.x, g = blockIdx.y;      // packed row (relative to the table's row 0)
    const int si = seq_of_row(seqs, row);
    const size_t rg = static_cast<size_t>(row) * hkv + g;
    int64_t c = (seqs.q_start[si] + (row - seqs.row0[si])) / m;
    c = c < nblk_max - 1 ? c : nblk_max - 1;
    const int jb = static_cast<int>(threadIdx.x) * per;
    int cnt = static_cast<int>(c + 1) - jb;
    cnt = cnt < 0 ? 0 : (cnt > per ? per : cnt);
    const uint32_t* gk = keys + rg * nblk_max;
    uint32_t key[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) key[u] = u < cnt ? gk[jb + u] : 0u;
    block_topk_regs<kThreads>(key, jb, cnt, static_cast<int>(c), topk, init, local, idx + rg * topk,
                              score ? score + rg * topk : nullptr, sm);
}

// ------------------------------------------------------------------ dense rows
// Every row shorter than k*m selects all its blocks ("Initial and local tokens
// always selected": below k*m tokens the method is exactly dense attention).
// When no block scores are requested, the ids need no scoring at all: one
// thread per (row, KV head, slot).  Decode row b ends at kv_lens[b] - 1;
// prefill row r sits at q_start + r.
__global__ __launch_bounds__(256) void sel_dense_ids(int mode_decode, int rows, int64_t q_start,
                                                     const int64_t* __restrict__ kv_off,
                                                     const int64_t* __restrict__ kv_lens, int hkv,
                                                     int m, int topk, int64_t nblk_max,
                                                     int32_t* __restrict__ idx) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(rows) * hkv * topk;
    if (e >= total) return;
    const int slot = static_cast<int>(e % topk);
    const int row = static_cast<int>(e / (static_cast<int64_t>(hkv) * topk));
    int64_t c;
    if (mode_decode) {
        const int64_t cap = kv_off[row + 1] - kv_off[row];
        int64_t n = kv_lens ? kv_lens[row] : cap;
        n = n < cap ? n : cap;
        c = n > 0 ? (n - 1) / m : -1;
    } else {
        c = (q_start + row) / m;
    }
    c = c < nblk_max - 1 ? c : nblk_max - 1;
    idx[e] = slot <= c ? slot : -1;
}

static void launch_dense_ids(const Shape& sh, int mode_decode, int rows, int64_t q_start,
                             const int64_t* kv_off, const int64_t* kv_lens, int64_t nblk_max,
                             int32_t* idx, hipStream_t st) {
    const int64_t total = static_cast<int64_t>(rows) * sh.hkv * sh.topk;
    KernelTimer kt(INFV2_KERNEL_SELECT_TOPK, st);
    sel_dense_ids<<<dim3(static_cast<unsigned>((total + 255) / 256)), 256, 0, st>>>(
        mode_decode, rows, q_start, kv_off, kv_lens, sh.hkv, sh.m, sh.topk, nblk_max, idx);
}

// ------------------------------------------------------------------ launchers
// keys per thread: the smallest register-array size that covers nblk_max / 256
#define INFV2_TOPK_DISPATCH(per, LAUNCH) \
    do {                                  \
        if ((per) <= 2) LAUNCH(2);        \
        else if ((per) <= 8) LAUNCH(8);   \
        else if ((per) <= 16) LAUNCH(16); \
        else LAUNCH(64);                  \
    } while (0)

static void launch_topk_dec(const Shape& sh, int batch, int64_t nblk_max, int64_t kld,
                            const int64_t* kv_off, const int64_t* lens, int lens_end,
                            const uint32_t* keys, int32_t* idx, float* score, hipStream_t st) {
    const int per = topk_per(nblk_max, 256);
#define INFV2_L(P) sel_dec_topk<P><<<dim3(sh.hkv, batch), 256, 0, st>>>( \
        kv_off, lens, lens_end, sh.hkv, sh.m, sh.topk, sh.init, sh.local, nblk_max, kld, keys, idx, score)
    INFV2_TOPK_DISPATCH(per, INFV2_L);
#undef INFV2_L
}

static void launch_topk_pre(const Shape& sh, const PrefillSeqs& seqs, int rows, int64_t nblk_max,
                            const uint32_t* keys, int32_t* idx, float* score, hipStream_t st) {
    const int per64 = topk_per(nblk_max, 64);
    if (per64 <= 16) {
#define INFV2_L(P) sel_pre_topk<64, P><<<dim3(rows, sh.hkv), 64, 0, st>>>( \
        seqs, sh.hkv, sh.m, sh.topk, sh.init, sh.local, nblk_max, per64, keys, idx, score)
        if (per64 <= 2) INFV2_L(2);
        else if (per64 <= 8) INFV2_L(8);
        else INFV2_L(16);
#undef INFV2_L
        return;
    }
    const int per = topk_per(nblk_max, 256);
#define INFV2_L(P) sel_pre_topk<256, P><<<dim3(rows, sh.hkv), 256, 0, st>>>( \
        seqs, sh.hkv, sh.m, sh.topk, sh.init, sh.local, nblk_max, per, keys, idx, score)
    INFV2_TOPK_DISPATCH(per, INFV2_L);
#undef INFV2_L
}

template <typename Tq, typename Tck>
static void dec_launch(const Shape& sh, const void* q, const void* ck, const int64_t* ck_off,
                       const int64_t* kv_off, const int64_t* kv_lens, int batch, int64_t max_len,
                       const SelectDecodeWs& w, char* ws, int32_t* idx, float* score,
                       const CoarseSel* cs, const void* fuse_k, bool skip_topk, hipStream_t st,
                       const DecAppend* app) {
    dim3 ga(w.nchunk_a, sh.hkv, batch), gb(w.nchunk_b, sh.hkv, batch);
    const int64_t ncm = w.nc_max > 0 ? w.nc_max : 1;
    const int64_t* lens = kv_lens ? kv_lens : kv_off + 1;
    const int lens_end = kv_lens ? (sh.lens_plus_one ? 2 : 0) : 1;
    const bf16_t* knew = app ? static_cast<const bf16_t*>(app->k_new) : nullptr;
    const bf16_t* vnew = app ? static_cast<const bf16_t*>(app->v_new) : nullptr;
    bf16_t* kapp = app ? static_cast<bf16_t*>(app->k) : nullptr;
    bf16_t* vapp = app ? static_cast<bf16_t*>(app->v) : nullptr;
    float* logits = reinterpret_cast<float*>(ws + w.logits);
    float2* partial = reinterpret_cast<float2*>(ws + w.partial);
    uint32_t* keys = reinterpret_cast<uint32_t*>(ws + w.keys);
    float* lse_c = nullptr;
    int nch_c = 1;
    float2* partial_c = nullptr;
    if (cs) {
        // pass 1 over the coarse kernels: their logits and per-chunk partials
        const int c = cs->coarse;
        const int64_t ncm_c = max_len < c ? 1 : (max_len - c) / c + 1;
        const int64_t ld_c = (ncm_c + 3) & ~int64_t(3);
        nch_c = static_cast<int>((ncm_c + kChunkA - 1) / kChunkA);
        float* logits_c = reinterpret_cast<float*>(ws + w.logits_c);
        partial_c = reinterpret_cast<float2*>(ws + w.partial_c);
        lse_c = reinterpret_cast<float*>(ws + w.lse_c);
        dim3 gc(nch_c, sh.hkv, batch);
        if (sizeof(Tq) == 2)
            launch_timed(INFV2_KERNEL_SELECT_LOGITS, sel_dec_logits_mfma<sizeof(Tck) == 2, false, true>, gc,
                         dim3(kLogWaves * 64), 0, st,
                static_cast<const bf16_t*>(q), cs->ckc, cs->ckc_off, kv_off, lens, lens_end, sh.hq,
                sh.hkv, c, c, sh.score_scale, ncm_c, ld_c, nch_c, w.nblk_max, w.keys_ld, logits_c,
                partial_c, keys, static_cast<const bf16_t*>(nullptr), static_cast<void*>(nullptr),
                static_cast<const bf16_t*>(nullptr), static_cast<const bf16_t*>(nullptr),
                static_cast<bf16_t*>(nullptr), static_cast<bf16_t*>(nullptr));
        else
            launch_timed(INFV2_KERNEL_SELECT_LOGITS, sel_dec_logits<Tq, Tck>, gc, dim3(256), 0, st,
                static_cast<const Tq*>(q), static_cast<const Tck*>(cs->ckc), cs->ckc_off, kv_off,
                kv_lens, sh.hq, sh.hkv, c, c, sh.score_scale, ncm_c, ld_c, nch_c, w.nblk_max,
                w.keys_ld, logits_c, partial_c, keys);
    }
    {
        if (sizeof(Tq) == 2)
        {
            const bool nt = static_cast<int64_t>(ga.x) * ga.y * ga.z <= kLogitsNtMaxBlocks;
#define INFV2_L(F, N) launch_timed(INFV2_KERNEL_SELECT_LOGITS, sel_dec_logits_mfma<sizeof(Tck) == 2, F, N>, \
                    ga, dim3(kLogWaves * 64), 0, st, \
                    static_cast<const bf16_t*>(q), ck, ck_off, kv_off, lens, lens_end, sh.hq, sh.hkv, \
                    sh.p, sh.s, sh.score_scale, ncm, w.nc_ld, w.nchunk_a, w.nblk_max, w.keys_ld, logits, \
                    partial, keys, static_cast<const bf16_t*>(fuse_k), const_cast<void*>(ck), \
                    knew, vnew, kapp, vapp)
            if (fuse_k) { if (nt) INFV2_L(true, true); else INFV2_L(true, false); }
            else { if (nt) INFV2_L(false, true); else INFV2_L(false, false); }
#undef INFV2_L
        }
        else
            launch_timed(INFV2_KERNEL_SELECT_LOGITS, sel_dec_logits<Tq, Tck>, ga, dim3(256), 0, st,
                static_cast<const Tq*>(q), static_cast<const Tck*>(ck), ck_off, kv_off, kv_lens,
                sh.hq, sh.hkv, sh.p, sh.s, sh.score_scale, ncm, w.nc_ld, w.nchunk_a, w.nblk_max,
                w.keys_ld, logits, partial, keys);
    }
    if (cs) {
        launch_timed(INFV2_KERNEL_SELECT_SCORES, sel_dec_lse_coarse, dim3(sh.hkv, batch), dim3(256),
                     0, st,
            kv_off, kv_lens, cs->ckc_off, sh.hkv, cs->coarse, nch_c, w.nchunk_a, partial_c, partial,
            lse_c);
    }
    {
        // large grids: 1024 kernels per block
        const bool two = static_cast<int64_t>(gb.x) * gb.y * gb.z > kScoresTwoMinBlocks;
        const dim3 gs(two ? (gb.x + 3) / 4 : gb.x, sh.hkv, batch);
        if (two)
            launch_timed(INFV2_KERNEL_SELECT_SCORES, sel_dec_scores<4>, gs, dim3(256), 0, st, kv_off,
                         lens, lens_end, ck_off, sh.hkv, sh.m, sh.p, sh.s, ncm, w.nc_ld, w.nchunk_a,
                         w.keys_ld, logits, partial, lse_c, keys);
        else
            launch_timed(INFV2_KERNEL_SELECT_SCORES, sel_dec_scores<1>, gs, dim3(256), 0, st, kv_off,
                         lens, lens_end, ck_off, sh.hkv, sh.m, sh.p, sh.s, ncm, w.nc_ld, w.nchunk_a,
                         w.keys_ld, logits, partial, lse_c, keys);
    }
    if (skip_topk) return;
    KernelTimer kt(INFV2_KERNEL_SELECT_TOPK, st);
    launch_topk_dec(sh, batch, w.nblk_max, w.keys_ld, kv_off, lens, lens_end, keys, idx, score, st);
}


hipError_t launch_select_decode(const Shape& sh, const void* q, const void* ck,
                                const int64_t* ck_off, const int64_t* kv_off,
                                const int64_t* kv_lens, int batch, int64_t max_len,
                                int32_t* idx, float* score, void* ws, const CoarseSel* cs,
                                hipStream_t st, const void* fuse_k, bool skip_topk,
                                const DecAppend* app) {
    const SelectDecodeWs w = select_decode_ws(sh, batch, max_len);
    if (!score && !fuse_k && !skip_topk && max_len <= static_cast<int64_t>(sh.topk) * sh.m) {   // every row dense
        launch_dense_ids(sh, 1, batch, 0, kv_off, kv_lens, w.nblk_max, idx, st);
        return hipGetLastError();
    }
    char* base = static_cast<char*>(ws);
    if (sh.io_bf16) {
        if (sh.ck_bf16) dec_launch<bf16_t, bf16_t>(sh, q, ck, ck_off, kv_off, kv_lens, batch, max_len, w, base, idx, score, cs, fuse_k, skip_topk, st, app);
        else dec_launch<bf16_t, float>(sh, q, ck, ck_off, kv_off, kv_lens, batch, max_len, w, base, idx, score, cs, fuse_k, skip_topk, st, app);
    } else {
        if (sh.ck_bf16) dec_launch<float, bf16_t>(sh, q, ck, ck_off, kv_off, kv_lens, batch, max_len, w, base, idx, score, cs, nullptr, skip_topk, st, nullptr);
        else dec_launch<float, float>(sh, q, ck, ck_off, kv_off, kv_lens, batch, max_len, w, base, idx, score, cs, nullptr, skip_topk, st, nullptr);
    }
    return hipGetLastError();
}

// Pass 1 (per-head LogSumExp and clearing the rows' block keys) for rows
// [r0, r0 + nr) of the call, over compressed keys `ck` of kernel size p, stride s.
// fp32 keys -> their hi / lo rows (ck_split_hilo), for the kernels each
// sequence's rows see, up to ld per sequence
static void split_hilo(const Shape& sh, const PrefillSeqs& seqs, const void* ck, const int64_t* ck_off,
                       int p, int s, int64_t ld, bf16_t* hl, hipStream_t st) {
    if (ld <= 0) return;
    const dim3 grid(static_cast<unsigned>((ld * 16 + 255) / 256), sh.hkv, seqs.n);
    launch_timed(INFV2_KERNEL_SELECT_PREFILL, ck_split_hilo, grid, dim3(256), 0, st, seqs,
                 static_cast<const float*>(ck), ck_off, sh.hkv, p, s, ld,
                 sh.score_scale * 1.4426950408889634f, hl);
}

// rows [r0, r0 + nr) of a one-sequence launch whose first row sits at q_start
static PrefillSeqs sub_seq(int r0, int nr, int64_t q_start) {
    PrefillSeqs t = one_seq(nr, q_start + r0);
    t.row0[0] = r0;                       // relative to the launch's row 0
    return t;
}

// Pass 1 (per-head LogSumExp and clearing the rows' block keys) over the rows of
// table t, with compressed keys `ck` of kernel size p, stride s.  The vector-ALU
// kernels (fp32 queries) take one sequence.
template <typename Tq, typename Tck>
static void pre_pass1(const Shape& sh, const PrefillSeqs& t, const void* q, const void* ck,
                      const int64_t* ck_off, int p, int s, const bf16_t* hl, int64_t ld,
                      const SelectPrefillWs& w, float* lse, uint32_t* keys, hipStream_t st) {
    const int groups = t.grp_end[t.n - 1];
    if (groups <= 0) return;
    if (sizeof(Tq) == 2) {
        launch_timed(INFV2_KERNEL_SELECT_PREFILL, sel_pre_mfma<1, sizeof(Tck) == 2>,
                     dim3(groups, sh.hkv), dim3(kPreThreads), 0, st, t,
            static_cast<const bf16_t*>(q), ck, ck_off, hl, ld, sh.hq, sh.hkv, sh.m, p, s,
            sh.score_scale, w.nblk_max, lse, keys);
    } else {
        const size_t r0 = static_cast<size_t>(t.row0[0]);
        const int nr = t.rows[0];
        const size_t qrow = static_cast<size_t>(sh.hq) * kHeadDim;
        dim3 g1((nr + kRowsPre - 1) / kRowsPre, sh.hkv);
        launch_timed(INFV2_KERNEL_SELECT_PREFILL, sel_pre_lse<Tq, Tck>, g1, dim3(256), 0, st,
                     static_cast<const Tq*>(q) + r0 * qrow, nr, t.q_start[0],
                     static_cast<const Tck*>(ck), ck_off + t.seq[0], sh.hq, sh.hkv, p, s,
                     sh.score_scale, w.nblk_max, lse + r0 * sh.hq, keys + r0 * sh.hkv * w.nblk_max);
    }
}

// The selection of the rows of table t (bf16 queries: any number of sequences;
// fp32 queries and the coarse-kernel LSE: one).
template <typename Tq, typename Tck>
static void pre_launch(const Shape& sh, const PrefillSeqs& t, const void* q, const void* ck,
                       const int64_t* ck_off, const SelectPrefillWs& w, char* ws, int32_t* idx,
                       float* score, const CoarseSel* cs, hipStream_t st) {
    const int rows_all = static_cast<int>(t.row0[t.n - 1] + t.rows[t.n - 1]);
    float* lse = reinterpret_cast<float*>(ws + w.lse);
    uint32_t* keys = reinterpret_cast<uint32_t*>(ws + w.keys);
    // matrix-core passes over fp32 keys read their hi / lo rows, made once here
    constexpr bool kSplit = sizeof(Tq) == 2 && sizeof(Tck) == 4;
    bf16_t* hl = kSplit ? reinterpret_cast<bf16_t*>(ws + w.hl) : nullptr;
    bf16_t* hlc = kSplit && cs ? reinterpret_cast<bf16_t*>(ws + w.hlc) : nullptr;
    if (kSplit) split_hilo(sh, t, ck, ck_off, sh.p, sh.s, w.ld, hl, st);
    if (cs) {
        // rows that see a coarse kernel take pass 1 over the coarse kernels; the
        // few before the first one (dense rows) keep the exact normaliser
        const int rows = t.rows[0];
        const int64_t q_start = t.q_start[0];
        int64_t nf = static_cast<int64_t>(cs->coarse) - 1 - q_start;
        nf = nf < 0 ? 0 : (nf > rows ? rows : nf);
        if (kSplit) split_hilo(sh, t, cs->ckc, cs->ckc_off, cs->coarse, cs->coarse, w.ldc, hlc, st);
        if (nf > 0)
            pre_pass1<Tq, Tck>(sh, sub_seq(0, static_cast<int>(nf), q_start), q, ck, ck_off, sh.p,
                               sh.s, hl, w.ld, w, lse, keys, st);
        if (rows - nf > 0)
            pre_pass1<Tq, Tck>(sh, sub_seq(static_cast<int>(nf), rows - static_cast<int>(nf), q_start),
                               q, cs->ckc, cs->ckc_off, cs->coarse, cs->coarse, hlc, w.ldc, w, lse,
                               keys, st);
    } else {
        pre_pass1<Tq, Tck>(sh, t, q, ck, ck_off, sh.p, sh.s, hl, w.ld, w, lse, keys, st);
    }
    if (sizeof(Tq) == 2) {
        constexpr bool kB = sizeof(Tck) == 2;
        launch_timed(INFV2_KERNEL_SELECT_PREFILL, sel_pre_mfma<2, kB>, dim3(t.grp_end[t.n - 1], sh.hkv),
                     dim3(kPreThreads), 0, st, t, static_cast<const bf16_t*>(q), ck, ck_off, hl,
                     w.ld, sh.hq, sh.hkv, sh.m, sh.p, sh.s, sh.score_scale, w.nblk_max, lse, keys);
    } else {
        const int rows = t.rows[0];
        dim3 g1((rows + kRowsPre - 1) / kRowsPre, sh.hkv);
        launch_timed(INFV2_KERNEL_SELECT_PREFILL, sel_pre_scores<Tq, Tck>, g1, dim3(256), 0, st,
                     static_cast<const Tq*>(q), rows, t.q_start[0], static_cast<const Tck*>(ck),
                     ck_off + t.seq[0], sh.hq, sh.hkv, sh.m, sh.p, sh.s, sh.score_scale, w.nblk_max,
                     lse, keys);
    }
    KernelTimer kt(INFV2_KERNEL_SELECT_TOPK, st);
    launch_topk_pre(sh, t, rows_all, w.nblk_max, keys, idx, score, st);
}

hipError_t launch_select_prefill(const Shape& sh, const void* q, int rows, int64_t q_start,
                                 const void* ck, const int64_t* ck_off, int64_t max_len,
                                 int32_t* idx, float* score, void* ws, const CoarseSel* cs,
                                 hipStream_t st) {
    const SelectPrefillWs w = select_prefill_ws(sh, rows, max_len);
    if (!score && q_start + rows <= static_cast<int64_t>(sh.topk) * sh.m) {   // every row dense
        launch_dense_ids(sh, 0, rows, q_start, nullptr, nullptr, w.nblk_max, idx, st);
        return hipGetLastError();
    }
    char* base = static_cast<char*>(ws);
    const PrefillSeqs t = one_seq(rows, q_start);
    if (sh.io_bf16) {
        if (sh.ck_bf16) pre_launch<bf16_t, bf16_t>(sh, t, q, ck, ck_off, w, base, idx, score, cs, st);
        else pre_launch<bf16_t, float>(sh, t, q, ck, ck_off, w, base, idx, score, cs, st);
    } else {
        if (sh.ck_bf16) pre_launch<float, bf16_t>(sh, t, q, ck, ck_off, w, base, idx, score, cs, st);
        else pre_launch<float, float>(sh, t, q, ck, ck_off, w, base, idx, score, cs, st);
    }
    return hipGetLastError();
}

hipError_t launch_select_prefill_seqs(const Shape& sh, const PrefillSeqs& seqs, const void* q,
                                      const void* ck, const int64_t* ck_off, int64_t max_len,
                                      int32_t* idx, float* score, void* ws, hipStream_t st) {
    if (!sh.io_bf16 || seqs.n < 1 || seqs.n > kVarlenMax) return hipErrorInvalidValue;
    const int rows_all = static_cast<int>(seqs.row0[seqs.n - 1] + seqs.rows[seqs.n - 1]);
    const SelectPrefillWs w = select_prefill_ws(sh, rows_all, max_len, seqs.n);
    char* base = static_cast<char*>(ws);
    if (sh.ck_bf16) pre_launch<bf16_t, bf16_t>(sh, seqs, q, ck, ck_off, w, base, idx, score, nullptr, st);
    else pre_launch<bf16_t, float>(sh, seqs, q, ck, ck_off, w, base, idx, score, nullptr, st);
    return hipGetLastError();
}

}  // namespace infv2
