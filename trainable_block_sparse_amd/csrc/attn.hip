// Exact softmax attention over the selected blocks.  MiniCPM4 summary page,
// "InfLLM v2" section, "Complexity analysis" (Stage 2: each query token attends
// the k*m tokens of its selected blocks) and "Query group sharing" (the 16 heads
// of a group read the same blocks, so K/V of a block is loaded once per group).
//
// These vector-ALU kernels serve fp32 inputs and the shapes the matrix-core
// kernels do not take (attn_decode.hip, attn_prefill.hip).
// Both stage 64-token K/V tiles of a selected block in LDS and keep an online
// softmax (running max, running sum, unnormalised output) per head.
//   attn_decode_kernel   grid (split, KV head, sequence): each block handles
//                        the split's selected blocks (one or four, chosen with
//                        the workspace) and writes a partial (max, sum,
//                        output); attn_decode_merge combines them by their
//                        LogSumExp.
//   attn_prefill_kernel  grid (row, KV head): all selected blocks of one row,
//                        causal within the query's own block (t <= i).
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

// Scratch of infv2_sparse_attn_decode_noalloc: the decode attention's split
// partials live in this file-scope device array instead of a caller workspace.
// Every device the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): it uses the device address that hipGetSymbolAddress
// returns, fetched once per device on the first call made on that device.
static __device__ __align__(256) char scratch[INFV2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

constexpr int kTok = 64;             // tokens per LDS tile

// Tiles per wave of the matrix-core decode attention: one while the grid stays
// below kDecodeWaveTarget waves (small batches are latency-bound), longer runs
// beyond (fewer partials, loads pipelined); always a divisor of the block's
// tpb tiles (a run stays in one block) and long enough for the merge's split
// limit.
static int decode_tpw(int tpb, int64_t tiles, int64_t bg) {
    int64_t want = (bg * tiles + kDecodeWaveTarget - 1) / kDecodeWaveTarget;
    want = want < kDecodeMaxTpw ? want : kDecodeMaxTpw;
    const int64_t need = (tiles + 4 * kDecodeMaxSplit - 1) / (4 * kDecodeMaxSplit);
    if (want < need) want = need;
    int tpw = 1;
    for (int x = 1; x <= tpb; ++x)
        if (tpb % x == 0 && x <= want) tpw = x;
    if (tpw < need)                                 // the smallest divisor that meets the limit
        for (int x = tpb; x >= 1; --x)
            if (tpb % x == 0 && x >= need) tpw = x;
    return tpw;
}

AttnDecodeWs attn_decode_ws(const Shape& sh, int batch) {
    AttnDecodeWs w{};
    const int64_t bg = static_cast<int64_t>(batch) * sh.hkv;
    // vector-ALU path: four selected blocks per split, or one where four would
    // give fewer thread blocks than the chip has compute units (small batches)
    constexpr int kOneBlockMax = 256;
    const int64_t wide = bg * ((sh.topk + 3) / 4);
    w.bps = (wide < kDecodeFewBlocks && sh.topk <= kOneBlockMax) ? 1 : 4;
    w.nsplit = (sh.topk + w.bps - 1) / w.bps;
    const int64_t nalloc_v = sh.topk <= kOneBlockMax ? sh.topk : w.nsplit;
    // matrix-core path: four waves per split, each a run of tpw 16-key tiles:
    // one tile while the grid stays below kDecodeWaveTarget waves (small
    // batches are latency-bound), longer runs beyond (fewer partials, loads
    // pipelined), and long enough that the merge takes the splits
    const int tpb = sh.m / 16;
    const int64_t tiles = static_cast<int64_t>(sh.topk) * tpb;
    w.tpw = decode_tpw(tpb, tiles, bg);
    w.nsplit_m = static_cast<int>((tiles + 4 * w.tpw - 1) / (4 * w.tpw));
    // runs only grow with the batch: the smallest batch has the most splits
    const int tpw1 = decode_tpw(tpb, tiles, 1);
    const int64_t nalloc_m = (tiles + 4 * tpw1 - 1) / (4 * tpw1);
    // room for the largest split count of either path at any batch, so the size
    // never shrinks as the batch grows (a workspace sized for a batch serves
    // every smaller one)
    const size_t nalloc = static_cast<size_t>(nalloc_v > nalloc_m ? nalloc_v : nalloc_m);
    const size_t nbg = static_cast<size_t>(bg);
    size_t off = 0;
    w.part_o = off;   off += align256(nbg * nalloc * kGroup * kHeadDim * sizeof(float));
    w.part_ml = off;  off += align256(nbg * nalloc * kGroup * sizeof(float2));
    w.total = off;
    return w;
}

struct AttnSmem {
    float qs[kGroup][kHeadDim];
    float ks[kTok][kHeadDim + 1];
    float vs[kTok][kHeadDim];
    float ps[kGroup][kTok];
};

// Online-softmax accumulation of selected blocks idx[jb..je) for the group's
// 16 heads at query position i over keys [0, n).  Thread t owns head t/16 and
// output columns (t%16)*8 .. +8.
template <typename T>
__device__ void attend_blocks(AttnSmem& sm, const T* __restrict__ kh, const T* __restrict__ vh,
                              const int32_t* __restrict__ sel, int jb, int je, int64_t i,
                              int64_t n, int m, float scale, float (&o)[8], float& mrun,
                              float& lrun) {
    const int t = threadIdx.x;
    const int h = t >> 4, c0 = (t & 15) * 8;
    const int w = t >> 6, lane = t & 63;
    const int64_t lim = (i + 1 < n) ? i + 1 : n;   // keys t < min(i+1, n)
    for (int e = jb; e < je; ++e) {
        const int32_t blk = sel[e];
        if (blk < 0) continue;
        for (int sub = 0; sub < m; sub += kTok) {
            const int64_t t0 = static_cast<int64_t>(blk) * m + sub;
            int64_t cnt = lim - t0;
            const int64_t in_blk = m - sub;
            cnt = cnt < in_blk ? cnt : in_blk;
            cnt = cnt < kTok ? cnt : kTok;
            if (cnt <= 0) continue;
            __syncthreads();
            for (int x = t * 4; x < kTok * kHeadDim; x += 256 * 4) {
                const int r = x / kHeadDim, col = x % kHeadDim;
                float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (r < cnt) {
                    load4(kh + (t0 + r) * kHeadDim + col, kv);
                    load4(vh + (t0 + r) * kHeadDim + col, vv);
                }
                sm.ks[r][col] = kv[0]; sm.ks[r][col + 1] = kv[1];
                sm.ks[r][col + 2] = kv[2]; sm.ks[r][col + 3] = kv[3];
                *reinterpret_cast<float4*>(&sm.vs[r][col]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            }
            __syncthreads();
            // scores: thread -> key `lane`, heads w, w+4, w+8, w+12
            {
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
                for (int d = 0; d < kHeadDim; ++d) {
                    const float kd = sm.ks[lane][d];
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[u] = fmaf(sm.qs[w + 4 * u][d], kd, acc[u]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) sm.ps[w + 4 * u][lane] = lane < cnt ? scale * acc[u] : -INFINITY;
            }
            __syncthreads();
            // softmax update for head h (16 threads per head, 4 keys each)
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
                sv[u] = pe;
            }
            ls = sum16(ls);
            lrun = lrun * alpha + ls;
            mrun = mnew;
#pragma unroll
            for (int x = 0; x < 8; ++x) o[x] *= alpha;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u) sm.ps[h][(t & 15) * 4 + u] = sv[u];
            __syncthreads();
            for (int r = 0; r < cnt; ++r) {
                const float pr = sm.ps[h][r];
                const float4 v0 = *reinterpret_cast<const float4*>(&sm.vs[r][c0]);
                const float4 v1 = *reinterpret_cast<const float4*>(&sm.vs[r][c0 + 4]);
                o[0] = fmaf(pr, v0.x, o[0]); o[1] = fmaf(pr, v0.y, o[1]);
                o[2] = fmaf(pr, v0.z, o[2]); o[3] = fmaf(pr, v0.w, o[3]);
                o[4] = fmaf(pr, v1.x, o[4]); o[5] = fmaf(pr, v1.y, o[5]);
                o[6] = fmaf(pr, v1.z, o[6]); o[7] = fmaf(pr, v1.w, o[7]);
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ void load_q_group(AttnSmem& sm, const T* qg) {
    for (int e = threadIdx.x; e < kGroup * kHeadDim; e += 256) sm.qs[e / kHeadDim][e % kHeadDim] = io<T>::load(qg + e);
}

template <typename T>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ kv_lens,
    const int32_t* __restrict__ idx, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int hq, int hkv, int m, int topk, int nsplit, int bps, float scale) {
    __shared__ AttnSmem sm;
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x, t = threadIdx.x;
    const int64_t o0 = kv_off[b], cap = kv_off[b + 1] - o0;
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const size_t bg = static_cast<size_t>(b) * hkv + g;
    const T* kh = k + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const T* vh = v + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    load_q_group(sm, q + (static_cast<size_t>(b) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim);
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const int jb = sp * bps;
    const int je = (jb + bps < topk) ? jb + bps : topk;
    attend_blocks<T>(sm, kh, vh, idx + bg * topk, jb, je, n - 1, n, m, scale, o, mrun, lrun);

    const int h = t >> 4, c0 = (t & 15) * 8;
    float* po = part_o + ((bg * nsplit + sp) * kGroup + h) * kHeadDim + c0;
    *reinterpret_cast<float4*>(po) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(po + 4) = make_float4(o[4], o[5], o[6], o[7]);
    // max in log2 units, as the shared merge kernel expects
    if ((t & 15) == 0)
        part_ml[(bg * nsplit + sp) * kGroup + h] = make_float2(mrun * 1.4426950408889634f, lrun);

}

template <typename T>
__global__ __launch_bounds__(256) void attn_prefill_kernel(
    const T* __restrict__ q, int64_t q_start, const T* __restrict__ k, const T* __restrict__ v,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ idx, T* __restrict__ out,
    int hq, int hkv, int m, int topk, float scale) {
    __shared__ AttnSmem sm;
    const int row = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
    const int64_t o0 = kv_off[0], cap = kv_off[1] - o0;
    const T* kh = k + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    const T* vh = v + (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
    load_q_group(sm, q + (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup) * kHeadDim);
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const size_t rg = static_cast<size_t>(row) * hkv + g;
    attend_blocks<T>(sm, kh, vh, idx + rg * topk, 0, topk, q_start + row, cap, m, scale, o, mrun, lrun);
    const int h = t >> 4, c0 = (t & 15) * 8;
    const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
    T* dst = out + (static_cast<size_t>(row) * hq + static_cast<size_t>(g) * kGroup + h) * kHeadDim + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) io<T>::store(dst + e, o[e] * inv);
}

hipError_t launch_attn_decode(const Shape& sh, const void* q, const void* k, const void* v,
                              const int64_t* kv_off, const int64_t* kv_lens, int batch,
                              const int32_t* idx, void* out, void* ws, hipStream_t st) {
    const AttnDecodeWs w = attn_decode_ws(sh, batch);
    char* base = static_cast<char*>(ws);
    dim3 grid(w.nsplit, sh.hkv, batch);
    float* po = reinterpret_cast<float*>(base + w.part_o);
    float2* pml = reinterpret_cast<float2*>(base + w.part_ml);
    hipError_t e;
    if (sh.io_bf16) {
        e = launch_attn_decode_mfma(sh, q, k, v, kv_off, kv_lens, batch, idx, po, pml, w.nsplit_m,
                                    w.tpw, st);
        if (e != hipSuccess) return e;
        return launch_attn_decode_merge(sh, po, pml, out, batch, w.nsplit_m, st);
    } else {
        launch_timed(INFV2_KERNEL_ATTN_DECODE, attn_decode_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), kv_off, kv_lens, idx, po, pml, sh.hq, sh.hkv, sh.m, sh.topk, w.nsplit, w.bps, sh.attn_scale);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return launch_attn_decode_merge(sh, po, pml, out, batch, w.nsplit, st);
}

hipError_t launch_attn_prefill(const Shape& sh, const void* q, int rows, int64_t q_start,
                               const void* k, const void* v, const int64_t* kv_off,
                               const int32_t* idx, void* out, void* ws, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (attn_prefill_mfma_ok(sh))
        return launch_attn_prefill_mfma(sh, q, rows, q_start, k, v, kv_off, idx, out, ws, st);
    dim3 grid(rows, sh.hkv);
    if (sh.io_bf16)
        launch_timed(INFV2_KERNEL_ATTN_PREFILL, attn_prefill_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(q), q_start, static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kv_off, idx, static_cast<bf16_t*>(out), sh.hq, sh.hkv, sh.m, sh.topk, sh.attn_scale);
    else
        launch_timed(INFV2_KERNEL_ATTN_PREFILL, attn_prefill_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(q), q_start, static_cast<const float*>(k), static_cast<const float*>(v), kv_off, idx, static_cast<float*>(out), sh.hq, sh.hkv, sh.m, sh.topk, sh.attn_scale);
    return hipGetLastError();
}

}  // namespace infv2
