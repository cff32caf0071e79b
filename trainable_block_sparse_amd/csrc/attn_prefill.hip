// Prefill attention over the selected blocks on the matrix cores (bf16, KV block 64).
// MiniCPM4 summary page, "InfLLM v2" section: "Complexity analysis" (Stage 2,
// each query token attends the k*m tokens of its own selected blocks), "Design
// principles summary" (token-level queries, block-level keys/values) and "Query
// group sharing" (the group's 16 heads form the 16-wide matrix tile of a token).
//
// Every query row picks its own 64 blocks, so the matrix tile of a (row, block)
// pair is 16 heads x 64 keys.  A thread block owns 16 consecutive rows (4 per
// wave) of one KV head and streams the union of their selected blocks through
// LDS once: K as stored, V as V^T tiles built by vt_build.  For each block a
// wave runs each of its rows that selected the block, reading the V^T
// fragments from LDS once for all of them:
//   S^T[key][head] = K_blk . Q_row^T          16 MFMA 16x16x32
//   O^T[d][head]  += V^T_blk . P_row^T        16 MFMA 16x16x32
// with the online softmax kept per (row, head) in registers (one head per lane
// column, so rescaling is a per-lane scalar).  Keys after the row (t > i) are
// masked in the row's own block.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kPB = 64;          // KV block size served here
constexpr int kPRows = 16;       // query rows per thread block
constexpr int kPRowsW = 4;       // query rows per wave
constexpr int kKPad = 136;       // LDS row length of K tiles (128 + 8 bf16: 16-byte pad)
constexpr int kVPad = 72;        // LDS row length of V^T tiles (64 + 8 bf16)
constexpr int kMaxWords = 512;   // bitmap words: up to 16384 blocks
constexpr int kUnionCap = 2048;  // union entries: 16 rows x top-k, top-k <= 128

// V^T tiles store the 64 keys of a block in the order the P^T operand of the
// PV product uses: position 32 kk + 8 g + 4 a + r holds key 32 kk + 16 a + 4 g + r.
__device__ __forceinline__ int vt_key_of_pos(int pos) {
    const int kk = pos >> 5, w = pos & 31, g = w >> 3, a = (w >> 2) & 1, r = w & 3;
    return 32 * kk + 16 * a + 4 * g + r;
}

// vt[g][blk][d][pos] = V[g][blk*64 + key(pos)][d]; keys at or past n read as zero.
__global__ __launch_bounds__(256) void vt_build(const bf16_t* __restrict__ v,
                                                const int64_t* __restrict__ kv_off, int hkv,
                                                int64_t n, int64_t nblk, bf16_t* __restrict__ vt) {
    __shared__ bf16_t tile[kPB][kHeadDim + 8];
    const int blk = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    const int64_t cap = kv_off[1] - kv_off[0];
    const bf16_t* vh = v + (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = t + 256 * i, row = e >> 4, c = e & 15;
        const int64_t key = static_cast<int64_t>(blk) * kPB + row;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (key < n) val = ldg16(vh + key * kHeadDim + 8 * c);
        *reinterpret_cast<uint4*>(&tile[row][8 * c]) = val;
    }
    __syncthreads();
    bf16_t* dst = vt + ((static_cast<int64_t>(g) * nblk + blk) * kHeadDim) * kPB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = t + 256 * i, d = e >> 3, p0 = (e & 7) * 8;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = static_cast<uint32_t>(tile[vt_key_of_pos(p0 + 2 * j)][d]) |
                   (static_cast<uint32_t>(tile[vt_key_of_pos(p0 + 2 * j + 1)][d]) << 16);
        *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(d) * kPB + p0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

struct PreSmem {
    bf16_t k[2][kPB][kKPad];
    bf16_t vt[2][kHeadDim][kVPad];
    int32_t list[kUnionCap];          // union of the rows' blocks, ascending (<= 16 * topk)
    uint32_t mask[kUnionCap];         // which of the 16 rows selected each union block
    uint32_t bits[kMaxWords];
    uint32_t wbase[kMaxWords];
    uint32_t scan_tmp[8];
};

__global__ __launch_bounds__(256, 1) void attn_prefill_mfma(
    const bf16_t* __restrict__ q, int rows, int64_t q_start, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ vt, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ idx, bf16_t* __restrict__ out, int hq, int hkv, int topk,
    int64_t nblk, float scale_log2) {
    extern __shared__ unsigned char smem_raw[];
    PreSmem& sm = *reinterpret_cast<PreSmem*>(smem_raw);
    const int g = blockIdx.y, t = threadIdx.x;
    const int w = t >> 6, l = t & 63, lg = l >> 4, lc = l & 15;
    const int r0 = blockIdx.x * kPRows;
    const int64_t cap = kv_off[1] - kv_off[0];
    const bf16_t* kh = k + (kv_off[0] * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const bf16_t* vth = vt + static_cast<int64_t>(g) * nblk * kHeadDim * kPB;
    const int64_t nlim = q_start + rows;                     // keys needed are < nlim

    // ---- union of the 16 rows' selected blocks (bitmap -> ascending list + row masks)
    const int nwords = static_cast<int>((nblk + 31) / 32);
    for (int x = t; x < nwords; x += 256) sm.bits[x] = 0u;
    __syncthreads();
    const int nent = kPRows * topk;
    for (int e = t; e < nent; e += 256) {
        const int row = r0 + e / topk;
        if (row >= rows) continue;
        const int32_t blk = idx[(static_cast<size_t>(row) * hkv + g) * topk + e % topk];
        if (blk >= 0 && blk < nblk) atomicOr(&sm.bits[blk >> 5], 1u << (blk & 31));
    }
    __syncthreads();
    uint32_t cnt_t = 0;
    for (int x = 2 * t; x < 2 * t + 2 && x < nwords; ++x) cnt_t += __popc(sm.bits[x]);
    const uint32_t base_t = block_incl_scan256(cnt_t, sm.scan_tmp) - cnt_t;
    {
        uint32_t pos = base_t;
        for (int x = 2 * t; x < 2 * t + 2 && x < nwords; ++x) {
            sm.wbase[x] = pos;
            uint32_t bw = sm.bits[x];
            while (bw) {
                const int bit = __ffs(bw) - 1;
                bw &= bw - 1;
                sm.list[pos] = x * 32 + bit;
                sm.mask[pos] = 0u;
                ++pos;
            }
        }
        if (t == 255) sm.scan_tmp[4] = pos;
    }
    __syncthreads();
    const int n_u = static_cast<int>(sm.scan_tmp[4]);
    for (int e = t; e < nent; e += 256) {
        const int tok = e / topk, row = r0 + tok;
        if (row >= rows) continue;
        const int32_t blk = idx[(static_cast<size_t>(row) * hkv + g) * topk + e % topk];
        if (blk < 0 || blk >= nblk) continue;
        const uint32_t word = sm.bits[blk >> 5];
        const uint32_t pos = sm.wbase[blk >> 5] + __popc(word & ((1u << (blk & 31)) - 1u));
        atomicOr(&sm.mask[pos], 1u << tok);
    }

    // ---- per-wave row state
    bf16x8_t qf[kPRowsW][4];
    f32x4_t o[kPRowsW][8];
    float mrun[kPRowsW], lrun[kPRowsW];
    int64_t qpos[kPRowsW];
#pragma unroll
    for (int i = 0; i < kPRowsW; ++i) {
        const int row = r0 + kPRowsW * w + i;
        const int rr = row < rows ? row : rows - 1;
        qpos[i] = q_start + row;
        const bf16_t* qrow = q + (static_cast<size_t>(rr) * hq + static_cast<size_t>(g) * kGroup + lc) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[i][ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * lg));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[i][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mrun[i] = -INFINITY;
        lrun[i] = 0.f;
    }

    // ---- stream the union: registers -> LDS, double buffered
    uint4 kreg[4], vreg[4];
    auto fetch = [&](int u) {
        const int32_t blk = sm.list[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = t + 256 * i;
            const int row = e >> 4, c = e & 15;                // K: 64 rows x 16 chunks
            const int64_t key = static_cast<int64_t>(blk) * kPB + row;
            kreg[i] = key < nlim ? ldg16(kh + key * kHeadDim + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
            const int d = e >> 3, p0 = (e & 7) * 8;            // V^T: 128 rows x 8 chunks
            vreg[i] = ldg16(vth + (static_cast<int64_t>(blk) * kHeadDim + d) * kPB + p0);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = t + 256 * i;
            *reinterpret_cast<uint4*>(&sm.k[buf][e >> 4][8 * (e & 15)]) = kreg[i];
            *reinterpret_cast<uint4*>(&sm.vt[buf][e >> 3][8 * (e & 7)]) = vreg[i];
        }
    };
    __syncthreads();
    if (n_u > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    for (int u = 0; u < n_u; ++u) {
        const int buf = u & 1;
        if (u + 1 < n_u) fetch(u + 1);
        const int32_t blk = sm.list[u];
        const uint32_t act_all = (sm.mask[u] >> (kPRowsW * w)) & 0xFu;
        uint32_t act = 0;
        int cntr[kPRowsW];
#pragma unroll
        for (int i = 0; i < kPRowsW; ++i) {
            int64_t c = qpos[i] + 1 - static_cast<int64_t>(blk) * kPB;
            c = c < kPB ? c : kPB;
            cntr[i] = static_cast<int>(c);
            if (((act_all >> i) & 1u) && c > 0) act |= 1u << i;
        }
        if (act) {
            bf16x8_t pf[kPRowsW][2];
#pragma unroll
            for (int i = 0; i < kPRowsW; ++i) {
                if (!((act >> i) & 1u)) continue;
                // S^T for row i: lane holds S[head lc][key 16 mt + 4 lg + r]
                f32x4_t s[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        a = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(&sm.k[buf][16 * mt + lc][32 * ks + 8 * lg])),
                                   qf[i][ks], a);
                    s[mt] = a;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = (16 * mt + 4 * lg + r) < cntr[i] ? s[mt][r] * scale_log2 : -INFINITY;
                        s[mt][r] = x;
                        mx = fmaxf(mx, x);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mnew = fmaxf(mrun[i], mx);
                const float alpha = (mrun[i] == -INFINITY) ? 0.f : exp2f(mrun[i] - mnew);
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
                lrun[i] = lrun[i] * alpha + ls;
                mrun[i] = mnew;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[i][mt][r] *= alpha;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    uint4 pu;
                    pu.x = pack_rne(s[2 * kk][0], s[2 * kk][1]);
                    pu.y = pack_rne(s[2 * kk][2], s[2 * kk][3]);
                    pu.z = pack_rne(s[2 * kk + 1][0], s[2 * kk + 1][1]);
                    pu.w = pack_rne(s[2 * kk + 1][2], s[2 * kk + 1][3]);
                    pf[i][kk] = as_bf16x8(pu);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const bf16x8_t v0 = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.vt[buf][16 * mt + lc][8 * lg]));
                const bf16x8_t v1 = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.vt[buf][16 * mt + lc][32 + 8 * lg]));
#pragma unroll
                for (int i = 0; i < kPRowsW; ++i) {
                    if (!((act >> i) & 1u)) continue;
                    o[i][mt] = mfma32(v0, pf[i][0], o[i][mt]);
                    o[i][mt] = mfma32(v1, pf[i][1], o[i][mt]);
                }
            }
        }
        if (u + 1 < n_u) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds O[head lc][d = 16 mt + 4 lg + r]
#pragma unroll
    for (int i = 0; i < kPRowsW; ++i) {
        const int row = r0 + kPRowsW * w + i;
        if (row >= rows) continue;
        const float inv = lrun[i] > 0.f ? 1.f / lrun[i] : 0.f;
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

bool attn_prefill_mfma_ok(const Shape& sh) {
    return sh.io_bf16 && sh.m == kPB && kPRows * sh.topk <= kUnionCap;
}

size_t attn_prefill_ws_bytes(const Shape& sh, int64_t max_len) {
    if (!attn_prefill_mfma_ok(sh)) return 0;
    const int64_t nblk = (max_len + kPB - 1) / kPB;
    return align256(static_cast<size_t>(sh.hkv) * nblk * kHeadDim * kPB * sizeof(bf16_t));
}

hipError_t launch_attn_prefill_mfma(const Shape& sh, const void* q, int rows, int64_t q_start,
                                    const void* k, const void* v, const int64_t* kv_off,
                                    const int32_t* idx, void* out, void* ws, hipStream_t st) {
    const int64_t n = q_start + rows;
    const int64_t nblk = (n + kPB - 1) / kPB;
    bf16_t* vt = static_cast<bf16_t*>(ws);
    vt_build<<<dim3(static_cast<unsigned>(nblk), sh.hkv), 256, 0, st>>>(
        static_cast<const bf16_t*>(v), kv_off, sh.hkv, n, nblk, vt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t smem = sizeof(PreSmem);
    const float scale_log2 = sh.attn_scale * 1.4426950408889634f;
    attn_prefill_mfma<<<dim3((rows + kPRows - 1) / kPRows, sh.hkv), 256, smem, st>>>(
        static_cast<const bf16_t*>(q), rows, q_start, static_cast<const bf16_t*>(k), vt, kv_off,
        idx, static_cast<bf16_t*>(out), sh.hq, sh.hkv, sh.topk, nblk, scale_log2);
    return hipGetLastError();
}

}  // namespace infv2
