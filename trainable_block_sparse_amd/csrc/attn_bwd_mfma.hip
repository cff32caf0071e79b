// Matrix-core kernels of the attention backward (bf16, KV block 64).
// MiniCPM4 summary page, "InfLLM v2" section, "Training-time considerations":
// gradients reach q, K and V only through the attention over the selected
// blocks; the selection is held fixed.  The arithmetic is the one stated in
// attn_bwd.hip; here it runs on 16x16x32 bf16 MFMA with fp32 accumulation.
//
// Row pass (bwd_row_mfma): like the forward prefill kernel (and placed like it),
// a thread block owns 16 consecutive rows of one KV head (one row per wave) and
// streams the union
// of their selected blocks through LDS (K and V as stored; the K^T operand comes
// from the K tile by transpose reads), two blocks per barrier interval with the
// next interval's loads in flight.  Per (row, block):
//   S^T  = K . Q^T          16 MFMA     dP^T = V . dO^T       16 MFMA
//   dA^T = P^T (dP^T - D), P against a lazily raised reference max
//   dQ^T += K^T . dA^T      16 MFMA (dA in bf16)
// and the row's LogSumExp (log2 units of the scaled logits) and D = dO . O go
// to the workspace for the column pass.
//
// Column pass (bwd_col_mfma): a thread block owns (KV head, block) and a segment
// of at most kSeg rows of the block's row list (from the inverse index); wave w
// owns keys 16 w .. 16 w + 15 and keeps their K and V fragments in registers.
// Rows go in pairs, the 32-wide contraction of the dk / dv products being
// (2 rows x 16 heads).  Per pair:
//   S = Q . K^T, dP = dO . V^T          4 x 4 MFMA (two rows, Q and dO)
//   P = 2^(S scale - lse), dA = P (dP - D)
//   dV^T += dO^T . P,  dK^T += Q^T . dA 16 MFMA
// The Q^T and dO^T operands (heads along the contraction) come from the same
// LDS tiles through transpose reads (ds_read_b64_tr_b16).  The pairs' Q, dO,
// lse and D go through a three-slot LDS ring with direct global->LDS loads,
// two pairs in flight (three thread blocks per CU).
// A block whose list is longer than kSeg rows is split into segments whose
// fp32 partials are summed in segment order by bwd_col_finish, so results do
// not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"
#include "prefill_tiles.hpp"

namespace infv2 {

constexpr int kRWaves = kUWaves;       // row pass: one row per wave
constexpr int kRThreads = kUThreads;
constexpr int kCThreads = 256;         // column pass: 4 waves x 16 keys
constexpr int kRSlots = 4;             // row pass: two LDS stages of two blocks (32 KB each)
constexpr int kSeg = 512;              // rows per column segment
constexpr int kXcdsB = 8;
constexpr float kSlackB = 8.f;         // log2 units, as in the forward

bool bwd_mfma_ok(const Shape& sh) {
    return sh.io_bf16 && sh.m == kPB && kURows * sh.topk <= kUnionCap;
}

// work items of the column pass: one per (column, segment); upper bound used for
// the grid and the partial buffers
static int64_t max_col_items(const Shape& sh, const BwdWs& w) {
    return static_cast<int64_t>(sh.hkv) * w.nblk + (static_cast<int64_t>(sh.hkv) * w.list_ld) / kSeg + 1;
}

size_t bwd_mfma_extra_bytes(const Shape& sh, const BwdWs& w) {
    const int64_t items = max_col_items(sh, w);
    const int64_t ncol = static_cast<int64_t>(sh.hkv) * w.nblk;
    return align256(static_cast<size_t>(ncol + 1) * sizeof(int32_t)) +          // item_start
           align256(static_cast<size_t>(items) * 2 * kPB * kHeadDim * sizeof(float));  // partials
}

// XCD-aware placement: thread block b runs on XCD b % 8; hand each XCD a
// contiguous range of work items
__device__ __forceinline__ int xcd_remap(int b, int nwg) {
    const int xcd = b % kXcdsB, kx = b / kXcdsB;
    const int qx = nwg / kXcdsB, rx = nwg % kXcdsB;
    return xcd * qx + (xcd < rx ? xcd : rx) + kx;
}

__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b) {
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), s);
        s = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), s);
    }
    return s;
}

// ---------------------------------------------------------------- row pass
__global__ __launch_bounds__(kRThreads, 1) void bwd_row_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ out, const bf16_t* __restrict__ dout,
    int rows, int64_t q_start, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ idx, bf16_t* __restrict__ dq, float* __restrict__ lse2,
    float* __restrict__ delta, int hq, int hkv, int topk, int64_t nblk, int nrg, float scale_log2,
    float scale) {
    __shared__ __attribute__((aligned(16))) BlockTile kst[kRSlots], vst[kRSlots];   // stage x: slots 2 x, 2 x + 1
    __shared__ UnionSmem sm;
    // placement as in the forward: each KV head's XCDs take its row groups in
    // turn, from the last (largest union) down; one call spans the whole
    // sequence, so contiguous ranges in row order would leave the XCD with the
    // last rows several times the work of the one with the first
    int g, grp;
    {
        const int xcd = static_cast<int>(blockIdx.x) % kXcdsB, kx = static_cast<int>(blockIdx.x) / kXcdsB;
        if (kXcdsB % hkv == 0) {
            const int xh = kXcdsB / hkv;
            g = xcd / xh;
            const int rank = kx * xh + xcd % xh;
            if (rank >= nrg) return;                       // grid padding (whole block)
            grp = nrg - 1 - rank;
        } else {
            const int lid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
            g = lid / nrg;
            grp = lid % nrg;
        }
    }
    const int r0 = grp * kURows;
    const int t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const int64_t cap = kv_off[1] - kv_off[0];
    const size_t hoff = (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const bf16_t* kh = k + hoff;
    const bf16_t* vh = v + hoff;
    const int64_t nlim = q_start + rows;

    const int n_u = build_union(sm, idx, rows, r0, hkv, g, topk, nblk);
    balance_union(sm, n_u);                   // intervals spread their work over the SIMDs
    refine_pairs(sm, n_u);                    // and exchanges between intervals even it out further

    // ---- row state: wave w owns row r0 + w; lane holds head lc, d = 32 ks + 8 lg ..
    const int row = r0 + w;
    const int rr = row < rows ? row : rows - 1;
    const int32_t qpos = static_cast<int32_t>(q_start + row);
    const size_t roff = (static_cast<size_t>(rr) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
    bf16x8_t qf[4], dof[4];
    float dd = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint4 qv = ldg16(q + roff + 32 * ks + 8 * lg);
        const uint4 dv = ldg16(dout + roff + 32 * ks + 8 * lg);
        const uint4 ov = ldg16(out + roff + 32 * ks + 8 * lg);
        qf[ks] = as_bf16x8(qv);
        dof[ks] = as_bf16x8(dv);
        dd += dot8_bf16(dv, ov);
    }
    dd = add_xor32(add_xor16(dd));              // D of head lc
    f32x4_t acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mref = -INFINITY, lsum = 0.f;
    // the compiler waits for q and dO here, where it sees their use, and not
    // for every outstanding load (the next block's tiles) inside the products
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" :: "v"(qf[ks]), "v"(dof[ks]));

    // ---- tile loads: each wave fills 1 KB of each tile (one 16-byte load per lane)
    const int key_l = 4 * w + (l >> 4);                          // keys 4 w .. 4 w + 3
    const int koff_l = key_l * kHeadDim + 8 * ((l & 15) ^ (key_l & 15));
    auto issue = [&](BlockTile& kt_, BlockTile& vt_, int u) {
        const int32_t blk = sm.list[u];
        const int64_t k0 = static_cast<int64_t>(blk) * kPB;
        int64_t off = k0 * kHeadDim + koff_l;
        if (k0 + kPB > nlim) {                                   // clamp: later keys are masked
            int64_t gk = k0 + key_l;
            gk = gk < nlim ? gk : nlim - 1;
            off = gk * kHeadDim + 8 * ((l & 15) ^ (key_l & 15));
        }
        dma16(kh + off, lds_offset(&kt_[w * 512]));
        dma16(vh + off, lds_offset(&vt_[w * 512]));
    };
    // K^T operands of dQ^T = K^T dA^T come from the K tile by transpose reads:
    // for d-tile dt and keys 32 kk + 16 a + 4 lg + 0..3 this lane reads the 4
    // values d = 16 dt + 4 (lc % 4) .. + 3 of key 32 kk + 16 a + kq, which hands
    // lane lc element e = K[key 32 kk + 16 a + 4 lg + e][d = 16 dt + lc] -- the
    // key order of the dA^T operand (the accumulator layout of S^T)
    const int kq = 4 * lg + (lc >> 2), kqb = (lc >> 1) & 1;
    const uint32_t kq0 = static_cast<uint32_t>(kq * kHeadDim * 2 + 8 * (lc & 1));
    auto compute = [&](const BlockTile& kt_, const BlockTile& vt_, int u) {
        const int32_t blk = sm.list[u];
        const int cntr = qpos + 1 - blk * kPB;                   // keys of the block at or before the row
        const bool act = ((sm.mask[u] >> w) & 1u) && row < rows && cntr > 0;
        if (!__builtin_amdgcn_readfirstlane(static_cast<int>(act))) return;
        f32x4_t s[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                s[mt] = mfma32(as_bf16x8(k_frag(kt_, 16 * mt + lc, 4 * ks + lg)), qf[ks], s[mt]);
        }
        // lane holds S^T[key 16 mt + 4 lg + r][head lc]
        float lm = -INFINITY;
        if (__builtin_amdgcn_readfirstlane(cntr) >= kPB) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) lm = fmaxf(lm, s[mt][r]);
        } else {
            const int lim_l = cntr - 4 * lg;                     // key 16 mt + 4 lg + r visible iff 16 mt + r < lim_l
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = (16 * mt + r) < lim_l ? s[mt][r] : -INFINITY;
                    s[mt][r] = x;
                    lm = fmaxf(lm, x);
                }
        }
        lm *= scale_log2;
        if (__any(lm > mref + kSlackB)) {
            const float mx = max_xor32(max_xor16(lm));
            const float mnew = fmaxf(mref, mx);
            const float alpha = (mref == -INFINITY) ? 0.f : fast_exp2(mref - mnew);
            lsum *= alpha;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][r] *= alpha;
            mref = mnew;
        }
        // dP^T one 16-key tile at a time (keeps few registers live), then dA^T
        float ls = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4_t dp = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                dp = mfma32(as_bf16x8(k_frag(vt_, 16 * mt + lc, 4 * ks + lg)), dof[ks], dp);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(fmaf(s[mt][r], scale_log2, -mref));   // masked: 0
                ls += p;
                s[mt][r] = p * (dp[r] - dd);
            }
        }
        lsum += ls;
        bf16x8_t af[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint4 pu;
            pu.x = pack_rne(s[2 * kk][0], s[2 * kk][1]);
            pu.y = pack_rne(s[2 * kk][2], s[2 * kk][3]);
            pu.z = pack_rne(s[2 * kk + 1][0], s[2 * kk + 1][1]);
            pu.w = pack_rne(s[2 * kk + 1][2], s[2 * kk + 1][3]);
            af[kk] = as_bf16x8(pu);
        }
        const uint32_t kb0 = lds_offset(&kt_[0]) + kq0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            // chunk 2 dt + kqb of key 32 kk + 16 a + kq sits at chunk (2 dt + kqb) ^ kq
            const uint32_t o = kb0 + 16u * static_cast<uint32_t>((2 * dt + kqb) ^ kq);
            const uint2 a0 = lds_read_tr16(o), a1 = lds_read_tr16(o + 16u * kHeadDim * 2);
            const uint2 b0 = lds_read_tr16(o + 32u * kHeadDim * 2), b1 = lds_read_tr16(o + 48u * kHeadDim * 2);
            acc[dt] = mfma32(as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y)), af[0], acc[dt]);
            acc[dt] = mfma32(as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y)), af[1], acc[dt]);
        }
    };
    // two-block barrier intervals, double-buffered: one block of the next
    // interval's loads is issued before each block of products
    const int n_iv = (n_u + 1) / 2;
    for (int x = 0; x < 2 && x < n_u; ++x) issue(kst[x], vst[x], x);
    for (int iv = 0; iv < n_iv; ++iv) {
        dma_wait_barrier();
        const int sx = ((iv + 1) & 1) * 2, sc = (iv & 1) * 2;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int xn = 2 * (iv + 1) + b, u = 2 * iv + b;
            if (xn < n_u) issue(kst[sx + b], vst[sx + b], xn);
            if (u < n_u) compute(kst[sc + b], vst[sc + b], u);
        }
    }

    // ---- epilogue: lane holds dQ^T[d = 16 mt + 4 lg + r][head lc]
    const float lt = add_xor32(add_xor16(lsum));
    if (row >= rows) return;
    const float inv = lt > 0.f ? scale / lt : 0.f;
    bf16_t* dst = dq + (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        uint2 pk;
        pk.x = pack_rne(acc[mt][0] * inv, acc[mt][1] * inv);
        pk.y = pack_rne(acc[mt][2] * inv, acc[mt][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * mt) = pk;
    }
    if (lg == 0) {
        const size_t o = static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup + lc;
        lse2[o] = lt > 0.f ? mref + log2f(lt) : INFINITY;    // +inf: nothing visible, P = 0
        delta[o] = dd;
    }
}

// ---------------------------------------------------------------- column pass
// items per column (1 + one per further kSeg rows) and their exclusive scan
__global__ __launch_bounds__(1024) void bwd_items_kernel(const int32_t* __restrict__ col_start,
                                                         int nblk, int ncol,
                                                         int32_t* __restrict__ item_start) {
    __shared__ uint32_t tmp[17];
    __shared__ uint32_t tile_total;
    const int t = threadIdx.x;
    uint32_t carry = 0;
    for (int base = 0; base < ncol; base += 1024) {
        const int c = base + t;
        uint32_t n = 0;
        if (c < ncol) {
            const int g = c / nblk, j = c % nblk;
            const int32_t* cs = col_start + static_cast<size_t>(g) * (nblk + 1);
            const int32_t len = cs[j + 1] - cs[j];
            n = len > kSeg ? static_cast<uint32_t>((len + kSeg - 1) / kSeg) : 1u;
        }
        const uint32_t incl = block_incl_scan<16>(n, tmp);
        if (c < ncol) item_start[c] = static_cast<int32_t>(carry + incl - n);
        if (t == 1023) tile_total = incl;
        __syncthreads();
        carry += tile_total;
        __syncthreads();
    }
    if (t == 0) item_start[ncol] = static_cast<int32_t>(carry);
}

typedef bf16_t RowTiles[4][kGroup * kHeadDim];   // Q_A, Q_B, dO_A, dO_B (4 KB each)
constexpr int kCStages = 3;                       // LDS ring of the column pass: 2 pairs in flight
constexpr int kCLoads = 5;                        // global->LDS loads per wave and pair

// Direct global->LDS load of 4 B per lane (lane i writes bytes 4 i .. 4 i + 3
// from the wave-uniform `lds`), issued by hand like dma16.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" :: "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}


// wait until this wave's loads of the current pair have landed (at most `later`
// further pairs' loads outstanding; loads complete in order), then a barrier
// makes every wave's share visible and frees the slot read one pair earlier
__device__ __forceinline__ void ring_wait(int later) {
    static_assert(kCStages == 3 && kCLoads == 5, "vmcnt immediates below");
    if (later >= 1) asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(kCThreads, 3) void bwd_col_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, int rows, int64_t q_start,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ list, int64_t list_ld,
    const int32_t* __restrict__ item_start, const float* __restrict__ lse2,
    const float* __restrict__ delta, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
    float* __restrict__ partial, int hq, int hkv, int nblk, float scale_log2, float scale) {
    __shared__ __attribute__((aligned(16))) RowTiles ring[kCStages];
    __shared__ __attribute__((aligned(16))) float lsd[kCStages][kCThreads / 64][64];  // per wave
    __shared__ __attribute__((aligned(16))) int32_t seg_rows[kSeg + 2];  // the segment's row ids
    const int ncol = hkv * nblk;
    // items in block order, dealt round the XCDs: the blocks resident at any
    // time work on neighbouring columns of one head, whose row lists overlap
    // (the local window, popular blocks), so the Q and dO rows they gather are
    // shared in the last-level cache; giving each XCD a contiguous range spreads
    // them over the whole sequence instead (measured 18 % slower)
    const int item = static_cast<int>(blockIdx.x);
    if (item >= item_start[ncol]) return;      // the grid is sized for the most items there can be
    // column of this item: last c with item_start[c] <= item
    int lo = 0, hi = ncol - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (item_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int col = lo, g = col / nblk, j = col % nblk;
    const int seg = item - item_start[col];
    const int nseg = item_start[col + 1] - item_start[col];
    const int32_t* cs = col_start + static_cast<size_t>(g) * (nblk + 1);
    const int32_t* lst = list + static_cast<size_t>(g) * list_ld;
    const int32_t beg = cs[j] + seg * kSeg;
    const int32_t end = (cs[j + 1] < beg + kSeg) ? cs[j + 1] : beg + kSeg;
    const int n = end - beg;

    const int t = threadIdx.x, w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const int64_t lim = q_start + rows;
    const int64_t cap = kv_off[1] - kv_off[0];
    const size_t hoff = (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const int64_t key = static_cast<int64_t>(j) * kPB + 16 * w + lc;      // this lane's key
    const int64_t keyc = key < lim ? key : lim - 1;
    bf16x8_t kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = as_bf16x8(ldg16(k + hoff + keyc * kHeadDim + 32 * ks + 8 * lg));
        vf[ks] = as_bf16x8(ldg16(v + hoff + keyc * kHeadDim + 32 * ks + 8 * lg));
    }
    {
        int32_t r[kSeg / kCThreads];         // all loads first, then the LDS writes
#pragma unroll
        for (int i = 0; i < kSeg / kCThreads; ++i) r[i] = (t + i * kCThreads < n) ? lst[beg + t + i * kCThreads] : 0;
#pragma unroll
        for (int i = 0; i < kSeg / kCThreads; ++i) seg_rows[t + i * kCThreads] = r[i];
    }
    f32x4_t av[8], ak[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) { av[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; ak[dt] = av[dt]; }
    // the compiler waits for K and V here, where it sees their use, and not for
    // every outstanding load (the ring's) inside the products
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" :: "v"(kf[ks]), "v"(vf[ks]));
    __syncthreads();                         // row ids in LDS

    // stage slot t of each tile: head h = t / 16 holds chunk (t % 16) ^ h there
    // (row bases are wave-uniform: SGPR addresses with a fixed lane offset)
    const int sh_h = t >> 4, sh_c = (t & 15) ^ (t >> 4);
    const uint32_t tile_off = static_cast<uint32_t>(((g * kGroup + sh_h) * kHeadDim + 8 * sh_c) * 2);
    auto row_base = [&](const bf16_t* base, int r) {
        return base + static_cast<size_t>(r) * hq * kHeadDim;
    };
    // lse / D slot of this wave: lane l loads quantity l / 16 (lse A, lse B, D A,
    // D B) of head l % 16
    const float* ld_src = (l < 32 ? lse2 : delta) + static_cast<size_t>(g) * kGroup + (l & 15);
    const bool ld_b = (l & 16) != 0;
    // The ring is filled by hand-issued loads (the compiler does not see them, so
    // it does not wait for all of them before each LDS read); ring_wait orders
    // them against the reads.
    auto issue = [&](int p) {
        const int s = p % kCStages;
        const int ra = __builtin_amdgcn_readfirstlane(seg_rows[2 * p]);
        const int rb = __builtin_amdgcn_readfirstlane((2 * p + 1 < n) ? seg_rows[2 * p + 1] : ra);
        dma16s(row_base(q, ra), tile_off, lds_offset(&ring[s][0][w * 512]));
        dma16s(row_base(q, rb), tile_off, lds_offset(&ring[s][1][w * 512]));
        dma16s(row_base(dout, ra), tile_off, lds_offset(&ring[s][2][w * 512]));
        dma16s(row_base(dout, rb), tile_off, lds_offset(&ring[s][3][w * 512]));
        dma4(ld_src + static_cast<size_t>(ld_b ? rb : ra) * hq, lds_offset(&lsd[s][w][0]));
    };
    // Transposed operands (d along M, (row, head) along K) come straight from
    // the tiles by transpose reads: for d-tile dt this lane reads the 4 values
    // d = 16 dt + 4 (lc % 4) .. + 3 of head 4 lg + lc / 4, which hands lane lc
    // element e = X[head 4 lg + e][d = 16 dt + lc].
    const int th = 4 * lg + (lc >> 2), tb = (lc >> 1) & 1;
    const uint32_t tr0 = 2u * static_cast<uint32_t>(th * kHeadDim + 4 * (lc & 1));

    auto compute = [&](int p) {
        const int sl = p % kCStages;
        const RowTiles& rt = ring[sl];
        const int ra = seg_rows[2 * p], rb = seg_rows[2 * p + 1];
        const bool has_b = 2 * p + 1 < n;
        // lse of rows A, B and D of rows A, B, heads 4 lg .. 4 lg + 3
        const f32x4_t la = *reinterpret_cast<const f32x4_t*>(&lsd[sl][w][4 * lg]);
        const f32x4_t lb = *reinterpret_cast<const f32x4_t*>(&lsd[sl][w][16 + 4 * lg]);
        const f32x4_t da = *reinterpret_cast<const f32x4_t*>(&lsd[sl][w][32 + 4 * lg]);
        const f32x4_t db = *reinterpret_cast<const f32x4_t*>(&lsd[sl][w][48 + 4 * lg]);
        f32x4_t s[2], dp[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) { s[x] = f32x4_t{0.f, 0.f, 0.f, 0.f}; dp[x] = s[x]; }
        // A fragments of tile x (Q_A, Q_B, dO_A, dO_B), one K-step at a time
        // (three waves per SIMD need the registers): lane holds
        // X[head lc][d = 32 ks + 8 lg ..] (chunks XOR-swizzled by head)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8_t fr[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                fr[x] = as_bf16x8(*reinterpret_cast<const uint4*>(&rt[x][lc * kHeadDim + 8 * ((4 * ks + lg) ^ lc)]));
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                s[x] = mfma32(fr[x], kf[ks], s[x]);
                dp[x] = mfma32(fr[2 + x], vf[ks], dp[x]);
            }
        }
        // lane holds S[head 4 lg + r][key 16 w + lc] of rows A (x = 0) and B (x = 1)
        float pv[2][4], av_[2][4];
        const int64_t pa = q_start + ra, pb = q_start + rb;
        const bool visa = key < lim && key <= pa;
        const bool visb = has_b && key < lim && key <= pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pv[0][r] = visa ? fast_exp2(fmaf(s[0][r], scale_log2, -la[r])) : 0.f;
            pv[1][r] = visb ? fast_exp2(fmaf(s[1][r], scale_log2, -lb[r])) : 0.f;
            av_[0][r] = pv[0][r] * (dp[0][r] - da[r]);
            av_[1][r] = pv[1][r] * (dp[1][r] - db[r]);
        }
        // B operands: k = 8 lg + e <-> (row e / 4, head 4 lg + e % 4), n = key lc
        uint4 pu, du;
        pu.x = pack_rne(pv[0][0], pv[0][1]); pu.y = pack_rne(pv[0][2], pv[0][3]);
        pu.z = pack_rne(pv[1][0], pv[1][1]); pu.w = pack_rne(pv[1][2], pv[1][3]);
        du.x = pack_rne(av_[0][0], av_[0][1]); du.y = pack_rne(av_[0][2], av_[0][3]);
        du.z = pack_rne(av_[1][0], av_[1][1]); du.w = pack_rne(av_[1][2], av_[1][3]);
        const bf16x8_t pb_ = as_bf16x8(pu), db_ = as_bf16x8(du);
        const uint32_t rt0 = lds_offset(&rt[0][0]) + tr0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint32_t o = rt0 + 16u * static_cast<uint32_t>((2 * dt + tb) ^ th);
            const uint2 qa = lds_read_tr16(o), qb = lds_read_tr16(o + 4096u);
            const uint2 oa = lds_read_tr16(o + 8192u), ob = lds_read_tr16(o + 12288u);
            // K index 8 lg + e <-> (row e / 4, head 4 lg + e % 4), as in pb_ / db_
            av[dt] = mfma32(as_bf16x8(make_uint4(oa.x, oa.y, ob.x, ob.y)), pb_, av[dt]);
            ak[dt] = mfma32(as_bf16x8(make_uint4(qa.x, qa.y, qb.x, qb.y)), db_, ak[dt]);
        }
    };

    const int npairs = (n + 1) >> 1;
    for (int p = 0; p < kCStages - 1 && p < npairs; ++p) issue(p);
    for (int p = 0; p < npairs; ++p) {
        const int left = npairs - 1 - p;
        ring_wait(left < kCStages - 2 ? left : kCStages - 2);
        if (p + kCStages - 1 < npairs) issue(p + kCStages - 1);
        compute(p);
    }

    // ---- epilogue: lane holds dV^T / dK^T[d = 16 dt + 4 lg + r][key 16 w + lc]
    if (nseg == 1) {
        if (key >= lim) return;
        bf16_t* pk = dk + hoff + key * kHeadDim + 4 * lg;
        bf16_t* pv = dv + hoff + key * kHeadDim + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            uint2 a, b;
            a.x = pack_rne(ak[dt][0] * scale, ak[dt][1] * scale);
            a.y = pack_rne(ak[dt][2] * scale, ak[dt][3] * scale);
            b.x = pack_rne(av[dt][0], av[dt][1]);
            b.y = pack_rne(av[dt][2], av[dt][3]);
            *reinterpret_cast<uint2*>(pk + 16 * dt) = a;
            *reinterpret_cast<uint2*>(pv + 16 * dt) = b;
        }
    } else {
        // fp32 partial of this segment: [2][64 keys][128 d]
        float* pk = partial + static_cast<size_t>(item) * 2 * kPB * kHeadDim + (16 * w + lc) * kHeadDim + 4 * lg;
        float* pv = pk + kPB * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            *reinterpret_cast<float4*>(pk + 16 * dt) = make_float4(ak[dt][0], ak[dt][1], ak[dt][2], ak[dt][3]);
            *reinterpret_cast<float4*>(pv + 16 * dt) = make_float4(av[dt][0], av[dt][1], av[dt][2], av[dt][3]);
        }
    }
}

// sums the segments of split columns in segment order and writes bf16 dk / dv
__global__ __launch_bounds__(256) void bwd_col_finish(
    const int32_t* __restrict__ item_start, const float* __restrict__ partial, int64_t lim,
    const int64_t* __restrict__ kv_off, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
    int hkv, int nblk, float scale) {
    const int col = blockIdx.x, g = col / nblk, j = col % nblk, t = threadIdx.x;
    const int i0 = item_start[col], n = item_start[col + 1] - i0;
    if (n <= 1) return;
    const int64_t cap = kv_off[1] - kv_off[0];
    const size_t hoff = (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    // thread: 4 consecutive values of the [2][64][128] partial (block y takes
    // 1024 of them); four segments' loads in flight at a time, summed in
    // segment order
    constexpr size_t kStride = 2 * kPB * kHeadDim;
    const int e = (static_cast<int>(blockIdx.y) * 256 + t) * 4;
    const float* src = partial + static_cast<size_t>(i0) * kStride + e;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int x = 0;
    for (; x + 4 <= n; x += 4) {
        float4 p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = *reinterpret_cast<const float4*>(src + static_cast<size_t>(x + u) * kStride);
#pragma unroll
        for (int u = 0; u < 4; ++u) { s.x += p[u].x; s.y += p[u].y; s.z += p[u].z; s.w += p[u].w; }
    }
    for (; x < n; ++x) {
        const float4 p = *reinterpret_cast<const float4*>(src + static_cast<size_t>(x) * kStride);
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    const int which = e / (kPB * kHeadDim), rem = e % (kPB * kHeadDim);
    const int64_t key = static_cast<int64_t>(j) * kPB + rem / kHeadDim;
    if (key >= lim) return;
    const float f = which == 0 ? scale : 1.f;
    uint2 pk;
    pk.x = pack_rne(s.x * f, s.y * f);
    pk.y = pack_rne(s.z * f, s.w * f);
    bf16_t* dst = (which == 0 ? dk : dv) + hoff + key * kHeadDim + rem % kHeadDim;
    *reinterpret_cast<uint2*>(dst) = pk;
}

hipError_t launch_attn_prefill_bwd_mfma(const Shape& sh, const BwdWs& w, const void* q, int rows,
                                        int64_t q_start, const void* k, const void* v,
                                        const int64_t* kv_off, const int32_t* idx,
                                        const void* out, const void* dout, void* dq, void* dk,
                                        void* dv, char* base, hipStream_t st) {
    const int64_t n = q_start + rows;
    const int64_t nblk = w.nblk;
    float* lse2 = reinterpret_cast<float*>(base + w.lse);
    float* delta = reinterpret_cast<float*>(base + w.delta);
    int32_t* item_start = reinterpret_cast<int32_t*>(base + w.extra);
    const int ncol = sh.hkv * w.nblk;
    float* partial = reinterpret_cast<float*>(base + w.extra + align256(static_cast<size_t>(ncol + 1) * sizeof(int32_t)));
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    hipError_t e = hipSuccess;
    {
        const int nrg = (rows + kURows - 1) / kURows;
        const unsigned grid_r = kXcdsB % sh.hkv == 0
            ? static_cast<unsigned>(kXcdsB) * static_cast<unsigned>((nrg + kXcdsB / sh.hkv - 1) / (kXcdsB / sh.hkv))
            : static_cast<unsigned>(nrg) * static_cast<unsigned>(sh.hkv);
        launch_timed(INFV2_KERNEL_BWD_ROW, bwd_row_mfma,
                     dim3(grid_r), dim3(kRThreads), 0, st,
            static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(out),
            static_cast<const bf16_t*>(dout), rows, q_start, static_cast<const bf16_t*>(k),
            static_cast<const bf16_t*>(v), kv_off, idx, static_cast<bf16_t*>(dq), lse2, delta,
            sh.hq, sh.hkv, sh.topk, nblk, nrg, scale_log2, sh.attn_scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_inverse_index(sh, w, rows, idx, base, st)) != hipSuccess) return e;
    const int32_t* cstart = reinterpret_cast<const int32_t*>(base + w.col_start);
    const int32_t* list = reinterpret_cast<const int32_t*>(base + w.list);
    bwd_items_kernel<<<1, 1024, 0, st>>>(cstart, w.nblk, ncol, item_start);
    const int64_t items = max_col_items(sh, w);
    launch_timed(INFV2_KERNEL_BWD_COL, bwd_col_mfma, dim3(static_cast<unsigned>(items)),
                 dim3(kCThreads), 0, st,
        static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout), rows, q_start,
        static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kv_off, cstart, list,
        w.list_ld, item_start, lse2, delta, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv),
        partial, sh.hq, sh.hkv, w.nblk, scale_log2, sh.attn_scale);
    static_assert(2 * kPB * kHeadDim % 1024 == 0, "finish grid");
    bwd_col_finish<<<dim3(static_cast<unsigned>(ncol), 2 * kPB * kHeadDim / 1024), 256, 0, st>>>(
        item_start, partial, n, kv_off, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), sh.hkv,
        w.nblk, sh.attn_scale);
    return hipGetLastError();
}

}  // namespace infv2
