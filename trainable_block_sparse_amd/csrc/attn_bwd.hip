// Backward of the sparse attention over the selected blocks (training).
// MiniCPM4 summary page, "InfLLM v2" section, paragraphs "Training-time
// considerations" and "Why mean pooling": top-k is not differentiable, so the
// selection is a constant of the backward pass and the compressed keys (which
// only feed the selection) receive no gradient; K and V receive gradient only
// through the attention of stage 2.
//
// With a = attn_scale * q.k over the row's selected tokens, P = softmax(a),
// o = P V and the upstream gradient dO, per query head:
//   D = dO . o,   dP_t = dO . v_t,   dA_t = P_t (dP_t - D),
//   dq = attn_scale * sum_t dA_t k_t,   dk_t += attn_scale * dA_t q,   dv_t += P_t dO.
//
// Three phases, no atomics on the gradients:
//   1. row pass (grid: row x KV head): D from the forward output, an online
//      softmax over the selected blocks that also accumulates sum_t e^(a_t - m)
//      (dP_t - D) k_t with the usual rescaling, so dq needs one sweep; writes dq
//      and the row's LogSumExp and D for phase 3.
//   2. inverse index: for each (KV head, block) the rows that selected it, in
//      ascending row order (chunk histograms, a scan over chunks and blocks,
//      then an ordered scatter), so the result is deterministic.
//   3. column pass (grid: block x KV head): every token's dk and dv summed
//      over the rows of its block's list, written once.
//
// These vector-ALU kernels serve fp32 and the shapes the matrix-core kernels
// (attn_bwd_mfma.hip) do not take; the inverse index serves both.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kInvRows = 64;      // rows per chunk of the inverse index
constexpr int kBTok = 64;         // tokens per LDS tile

BwdWs bwd_ws(const Shape& sh, int rows, int64_t max_len) {
    BwdWs w{};
    w.nblk = static_cast<int>((max_len + sh.m - 1) / sh.m);
    w.nchunk = (rows + kInvRows - 1) / kInvRows;
    w.list_ld = static_cast<int64_t>(rows) * sh.topk;
    const size_t rh = static_cast<size_t>(rows) * sh.hq;
    size_t off = 0;
    w.lse = off;        off += align256(rh * sizeof(float));
    w.delta = off;      off += align256(rh * sizeof(float));
    w.counts = off;     off += align256(static_cast<size_t>(sh.hkv) * w.nblk * w.nchunk * sizeof(int32_t));
    w.totals = off;     off += align256(static_cast<size_t>(sh.hkv) * w.nblk * sizeof(int32_t));
    w.col_start = off;  off += align256(static_cast<size_t>(sh.hkv) * (w.nblk + 1) * sizeof(int32_t));
    w.list = off;       off += align256(static_cast<size_t>(sh.hkv) * w.list_ld * sizeof(int32_t));
    w.extra = off;
    if (bwd_mfma_ok(sh)) off += bwd_mfma_extra_bytes(sh, w);
    w.total = off;
    return w;
}

// ---------------------------------------------------------------- phase 1: rows (vector ALU)
struct BwdRowSmem {
    float qs[kGroup][kHeadDim];
    float dos[kGroup][kHeadDim];
    float ks[kBTok][kHeadDim + 1];
    float vs[kBTok][kHeadDim + 1];
    float ps[kGroup][kBTok];
    float dps[kGroup][kBTok];
};

// grid (rows, Hkv), 256 threads: thread t owns head t/16 and columns (t%16)*8 .. +8
template <typename T>
__global__ __launch_bounds__(256) void bwd_row_kernel(
    const T* __restrict__ q, const T* __restrict__ out, const T* __restrict__ dout,
    int64_t q_start, const T* __restrict__ k, const T* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ idx, T* __restrict__ dq,
    float* __restrict__ lse, float* __restrict__ delta, int hq, int hkv, int m, int topk,
    float scale) {
    __shared__ BwdRowSmem sm;
    const int row = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    const int h = t >> 4, c0 = (t & 15) * 8, w = t >> 6, lane = t & 63;
    const int64_t o0 = kv_off[0], cap = kv_off[1] - o0;
    const T* kh = k + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const T* vh = v + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const size_t qoff = (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim;
    for (int e = t; e < kGroup * kHeadDim; e += 256) {
        sm.qs[e / kHeadDim][e % kHeadDim] = io<T>::load(q + qoff + e);
        sm.dos[e / kHeadDim][e % kHeadDim] = io<T>::load(dout + qoff + e);
    }
    float dd = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const size_t o = qoff + static_cast<size_t>(h) * kHeadDim + c0 + x;
        dd = fmaf(io<T>::load(dout + o), io<T>::load(out + o), dd);
    }
    const float dh = sum16(dd);              // D of head h
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const int64_t i = q_start + row;
    const int64_t lim = (i + 1 < cap) ? i + 1 : cap;
    const int32_t* sel = idx + (static_cast<size_t>(row) * hkv + g) * topk;
    for (int e = 0; e < topk; ++e) {
        const int32_t blk = sel[e];
        if (blk < 0) continue;
        for (int sub = 0; sub < m; sub += kBTok) {
            const int64_t t0 = static_cast<int64_t>(blk) * m + sub;
            int64_t cnt = lim - t0;
            cnt = cnt < m - sub ? cnt : m - sub;
            cnt = cnt < kBTok ? cnt : kBTok;
            if (cnt <= 0) continue;
            __syncthreads();
            for (int x = t * 4; x < kBTok * kHeadDim; x += 256 * 4) {
                const int r = x / kHeadDim, col = x % kHeadDim;
                float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (r < cnt) {
                    load4(kh + (t0 + r) * kHeadDim + col, kv);
                    load4(vh + (t0 + r) * kHeadDim + col, vv);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) { sm.ks[r][col + u] = kv[u]; sm.vs[r][col + u] = vv[u]; }
            }
            __syncthreads();
            // logits and dP: thread -> key `lane`, heads w, w+4, w+8, w+12
            {
                float sa[4] = {0.f, 0.f, 0.f, 0.f}, pa[4] = {0.f, 0.f, 0.f, 0.f};
                for (int d = 0; d < kHeadDim; ++d) {
                    const float kd = sm.ks[lane][d], vd = sm.vs[lane][d];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        sa[u] = fmaf(sm.qs[w + 4 * u][d], kd, sa[u]);
                        pa[u] = fmaf(sm.dos[w + 4 * u][d], vd, pa[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sm.ps[w + 4 * u][lane] = lane < cnt ? scale * sa[u] : -INFINITY;
                    sm.dps[w + 4 * u][lane] = pa[u];
                }
            }
            __syncthreads();
            // online softmax of head h (16 threads x 4 keys); unnormalised dA
            float sv[4];
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; ++u) { sv[u] = sm.ps[h][(t & 15) * 4 + u]; mt = fmaxf(mt, sv[u]); }
            mt = max16(mt);
            const float mnew = fmaxf(mrun, mt);
            const float alpha = (mrun == -INFINITY) ? 0.f : expf(mrun - mnew);
            float ls = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float pe = (sv[u] == -INFINITY) ? 0.f : expf(sv[u] - mnew);
                ls += pe;
                sv[u] = pe * (sm.dps[h][(t & 15) * 4 + u] - dh);
            }
            ls = sum16(ls);
            lrun = lrun * alpha + ls;
            mrun = mnew;
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[x] *= alpha;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u) sm.ps[h][(t & 15) * 4 + u] = sv[u];
            __syncthreads();
            for (int r = 0; r < cnt; ++r) {
                const float da = sm.ps[h][r];
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[x] = fmaf(da, sm.ks[r][c0 + x], acc[x]);
            }
        }
    }
    const float inv = lrun > 0.f ? scale / lrun : 0.f;
    T* dst = dq + qoff + static_cast<size_t>(h) * kHeadDim + c0;
#pragma unroll
    for (int x = 0; x < 8; ++x) io<T>::store(dst + x, acc[x] * inv);
    if ((t & 15) == 0) {
        const size_t o = static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup + h;
        lse[o] = lrun > 0.f ? mrun + logf(lrun) : INFINITY;   // +inf: no visible token, P = 0
        delta[o] = dh;
    }
}

// ---------------------------------------------------------------- phase 2: inverse index
// counts[(g * nblk + j) * nchunk + c] = rows of chunk c (kInvRows rows) that selected block j
__global__ __launch_bounds__(256) void inv_count_kernel(const int32_t* __restrict__ idx, int rows,
                                                        int hkv, int topk, int nblk, int nchunk,
                                                        int32_t* __restrict__ counts) {
    extern __shared__ uint32_t hist[];
    const int c = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    for (int j = t; j < nblk; j += 256) hist[j] = 0u;
    __syncthreads();
    const int r0 = c * kInvRows;
    const int nr = (rows - r0 < kInvRows) ? rows - r0 : kInvRows;
    for (int e = t; e < nr * topk; e += 256) {
        const int r = r0 + e / topk, s = e % topk;
        const int32_t j = idx[(static_cast<size_t>(r) * hkv + g) * topk + s];
        if (j >= 0 && j < nblk) atomicAdd(&hist[j], 1u);
    }
    __syncthreads();
    for (int j = t; j < nblk; j += 256)
        counts[(static_cast<size_t>(g) * nblk + j) * nchunk + c] = static_cast<int32_t>(hist[j]);
}

// one wave per (KV head, block): exclusive scan of the chunk counts in place, and the total
__global__ __launch_bounds__(256) void inv_scan_chunks_kernel(int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ totals,
                                                              int ncol, int nchunk) {
    const int col = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (col >= ncol) return;
    int32_t* p = counts + static_cast<size_t>(col) * nchunk;
    int32_t carry = 0;
    for (int base = 0; base < nchunk; base += 64) {
        const int c = base + lane;
        const int32_t v = c < nchunk ? p[c] : 0;
        int32_t x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t u = __shfl_up(x, o, 64);
            if (lane >= o) x += u;
        }
        if (c < nchunk) p[c] = carry + x - v;
        carry += __shfl(x, 63, 64);
    }
    if (lane == 0) totals[col] = carry;
}

// one block of 1024 threads per KV head: col_start[g][j] = sum of totals before j
__global__ __launch_bounds__(1024) void inv_scan_blocks_kernel(const int32_t* __restrict__ totals,
                                                               int32_t* __restrict__ col_start,
                                                               int nblk) {
    __shared__ uint32_t tmp[17];
    __shared__ uint32_t tile_total;
    const int g = blockIdx.x, t = threadIdx.x;
    uint32_t carry = 0;
    for (int base = 0; base < nblk; base += 1024) {
        const int j = base + t;
        const uint32_t v = j < nblk ? static_cast<uint32_t>(totals[static_cast<size_t>(g) * nblk + j]) : 0u;
        const uint32_t incl = block_incl_scan<16>(v, tmp);
        if (j < nblk) col_start[static_cast<size_t>(g) * (nblk + 1) + j] = static_cast<int32_t>(carry + incl - v);
        if (t == 1023) tile_total = incl;
        __syncthreads();
        carry += tile_total;
        __syncthreads();
    }
    if (t == 0) col_start[static_cast<size_t>(g) * (nblk + 1) + nblk] = static_cast<int32_t>(carry);
}

// rows of chunk c in ascending order: list[g][pos] = row, pos from the block's start
// plus the chunk's prefix plus the rows of this chunk already placed
__global__ __launch_bounds__(256) void inv_scatter_kernel(
    const int32_t* __restrict__ idx, int rows, int hkv, int topk, int nblk, int nchunk,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ col_start,
    int32_t* __restrict__ list, int64_t list_ld) {
    extern __shared__ uint32_t cur[];
    const int c = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    for (int j = t; j < nblk; j += 256)
        cur[j] = static_cast<uint32_t>(col_start[static_cast<size_t>(g) * (nblk + 1) + j] +
                                       counts[(static_cast<size_t>(g) * nblk + j) * nchunk + c]);
    __syncthreads();
    const int r0 = c * kInvRows;
    const int r1 = (rows - r0 < kInvRows) ? rows : r0 + kInvRows;
    int32_t* dst = list + static_cast<size_t>(g) * list_ld;
    constexpr int kSlots = 4;                 // topk <= 1024 = 4 x 256
    int32_t jc[kSlots];
    auto fetch = [&](int r, int32_t (&jj)[kSlots]) {
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            const int s = t + 256 * u;
            jj[u] = (r < r1 && s < topk) ? idx[(static_cast<size_t>(r) * hkv + g) * topk + s] : -1;
        }
    };
    fetch(r0, jc);
    for (int r = r0; r < r1; ++r) {
        int32_t jn[kSlots];
        fetch(r + 1, jn);
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            const int32_t j = jc[u];
            if (j >= 0 && j < nblk) dst[atomicAdd(&cur[j], 1u)] = r;
        }
        __syncthreads();                      // this row placed before the next one
#pragma unroll
        for (int u = 0; u < kSlots; ++u) jc[u] = jn[u];
    }
}

// ---------------------------------------------------------------- phase 3: columns (vector ALU)
struct BwdColSmem {
    float qs[kGroup][kHeadDim];
    float dos[kGroup][kHeadDim];
    float lse[kGroup], delta[kGroup];
};

// grid (nblk * nsub, Hkv), 256 threads: thread t owns token t/4 of the 64-token
// tile and columns (t%4)*32 .. +32 of its dk and dv
template <typename T>
__global__ __launch_bounds__(256) void bwd_col_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, int64_t q_start, int rows,
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ list, int64_t list_ld,
    const float* __restrict__ lse, const float* __restrict__ delta, T* __restrict__ dk,
    T* __restrict__ dv, int hq, int hkv, int m, int nblk, int nsub, float scale) {
    __shared__ BwdColSmem sm;
    const int j = blockIdx.x / nsub, sub = blockIdx.x % nsub, g = blockIdx.y, t = threadIdx.x;
    const int64_t lim = q_start + rows;
    const int64_t t0 = static_cast<int64_t>(j) * m + sub * kBTok;
    int64_t cnt = lim - t0;
    cnt = cnt < m - sub * kBTok ? cnt : m - sub * kBTok;
    cnt = cnt < kBTok ? cnt : kBTok;
    if (cnt <= 0) return;
    const int tok = t >> 2, c0 = (t & 3) * 32;
    const int64_t o0 = kv_off[0], cap = kv_off[1] - o0;
    const size_t hoff = (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    float kr[32], vr[32], ak[32], av[32];
#pragma unroll
    for (int x = 0; x < 32; x += 4) {
        if (tok < cnt) {
            load4(k + hoff + (t0 + tok) * kHeadDim + c0 + x, kr + x);
            load4(v + hoff + (t0 + tok) * kHeadDim + c0 + x, vr + x);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) { kr[x + u] = 0.f; vr[x + u] = 0.f; }
        }
    }
#pragma unroll
    for (int x = 0; x < 32; ++x) { ak[x] = 0.f; av[x] = 0.f; }
    const int32_t* cs = col_start + static_cast<size_t>(g) * (nblk + 1);
    const int32_t* lst = list + static_cast<size_t>(g) * list_ld;
    const int32_t beg = cs[j], end = cs[j + 1];
    for (int32_t e = beg; e < end; ++e) {
        const int r = lst[e];
        const int64_t i = q_start + r;
        const size_t qoff = (static_cast<size_t>(r) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim;
        __syncthreads();
        for (int x = t; x < kGroup * kHeadDim; x += 256) {
            sm.qs[x / kHeadDim][x % kHeadDim] = io<T>::load(q + qoff + x);
            sm.dos[x / kHeadDim][x % kHeadDim] = io<T>::load(dout + qoff + x);
        }
        if (t < kGroup) {
            const size_t o = static_cast<size_t>(r) * hq + static_cast<size_t>(g) * kGroup + t;
            sm.lse[t] = lse[o];
            sm.delta[t] = delta[o];
        }
        __syncthreads();
        const bool vis = tok < cnt && t0 + tok <= i;
        for (int hh = 0; hh < kGroup; ++hh) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int x = 0; x < 32; ++x) {
                s = fmaf(sm.qs[hh][c0 + x], kr[x], s);
                dp = fmaf(sm.dos[hh][c0 + x], vr[x], dp);
            }
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            dp += __shfl_xor(dp, 1, 64);
            dp += __shfl_xor(dp, 2, 64);
            const float p = vis ? expf(scale * s - sm.lse[hh]) : 0.f;
            const float da = p * (dp - sm.delta[hh]);
#pragma unroll
            for (int x = 0; x < 32; ++x) {
                av[x] = fmaf(p, sm.dos[hh][c0 + x], av[x]);
                ak[x] = fmaf(da, sm.qs[hh][c0 + x], ak[x]);
            }
        }
    }
    if (tok < cnt) {
        T* pk = dk + hoff + (t0 + tok) * kHeadDim + c0;
        T* pv = dv + hoff + (t0 + tok) * kHeadDim + c0;
#pragma unroll
        for (int x = 0; x < 32; ++x) {
            io<T>::store(pk + x, scale * ak[x]);
            io<T>::store(pv + x, av[x]);
        }
    }
}

// ---------------------------------------------------------------- launcher
hipError_t launch_inverse_index(const Shape& sh, const BwdWs& w, int rows, const int32_t* idx,
                                char* base, hipStream_t st) {
    int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts);
    int32_t* totals = reinterpret_cast<int32_t*>(base + w.totals);
    int32_t* cstart = reinterpret_cast<int32_t*>(base + w.col_start);
    int32_t* list = reinterpret_cast<int32_t*>(base + w.list);
    const size_t lds = static_cast<size_t>(w.nblk) * sizeof(uint32_t);
    KernelTimer kt(INFV2_KERNEL_BWD_INDEX, st);
    inv_count_kernel<<<dim3(w.nchunk, sh.hkv), 256, lds, st>>>(idx, rows, sh.hkv, sh.topk, w.nblk, w.nchunk, counts);
    const int ncol = sh.hkv * w.nblk;
    inv_scan_chunks_kernel<<<(ncol + 3) / 4, 256, 0, st>>>(counts, totals, ncol, w.nchunk);
    inv_scan_blocks_kernel<<<sh.hkv, 1024, 0, st>>>(totals, cstart, w.nblk);
    inv_scatter_kernel<<<dim3(w.nchunk, sh.hkv), 256, lds, st>>>(idx, rows, sh.hkv, sh.topk, w.nblk, w.nchunk, counts, cstart, list, w.list_ld);
    return hipGetLastError();
}

hipError_t launch_attn_prefill_bwd(const Shape& sh, const void* q, int rows, int64_t q_start,
                                   const void* k, const void* v, const int64_t* kv_off,
                                   const int32_t* idx, const void* out, const void* dout,
                                   void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const BwdWs w = bwd_ws(sh, rows, q_start + rows);
    char* base = static_cast<char*>(ws);
    float* lse = reinterpret_cast<float*>(base + w.lse);
    float* delta = reinterpret_cast<float*>(base + w.delta);
    if (bwd_mfma_ok(sh))
        return launch_attn_prefill_bwd_mfma(sh, w, q, rows, q_start, k, v, kv_off, idx, out, dout, dq, dk, dv, base, st);
    hipError_t e;
    {
        if (sh.io_bf16)
            launch_timed(INFV2_KERNEL_BWD_ROW, bwd_row_kernel<bf16_t>, dim3(rows, sh.hkv), dim3(256), 0, st, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), q_start, static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kv_off, idx, static_cast<bf16_t*>(dq), lse, delta, sh.hq, sh.hkv, sh.m, sh.topk, sh.attn_scale);
        else
            launch_timed(INFV2_KERNEL_BWD_ROW, bwd_row_kernel<float>, dim3(rows, sh.hkv), dim3(256), 0, st, static_cast<const float*>(q), static_cast<const float*>(out), static_cast<const float*>(dout), q_start, static_cast<const float*>(k), static_cast<const float*>(v), kv_off, idx, static_cast<float*>(dq), lse, delta, sh.hq, sh.hkv, sh.m, sh.topk, sh.attn_scale);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if ((e = launch_inverse_index(sh, w, rows, idx, base, st)) != hipSuccess) return e;
    const int32_t* cstart = reinterpret_cast<const int32_t*>(base + w.col_start);
    const int32_t* list = reinterpret_cast<const int32_t*>(base + w.list);
    const int nsub = (sh.m + kBTok - 1) / kBTok;
    const dim3 grid(w.nblk * nsub, sh.hkv);
    if (sh.io_bf16)
        launch_timed(INFV2_KERNEL_BWD_COL, bwd_col_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout), q_start, rows, static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kv_off, cstart, list, w.list_ld, lse, delta, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), sh.hq, sh.hkv, sh.m, w.nblk, nsub, sh.attn_scale);
    else
        launch_timed(INFV2_KERNEL_BWD_COL, bwd_col_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(q), static_cast<const float*>(dout), q_start, rows, static_cast<const float*>(k), static_cast<const float*>(v), kv_off, cstart, list, w.list_ld, lse, delta, static_cast<float*>(dk), static_cast<float*>(dv), sh.hq, sh.hkv, sh.m, w.nblk, nsub, sh.attn_scale);
    return hipGetLastError();
}

}  // namespace infv2
