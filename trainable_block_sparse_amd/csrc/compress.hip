// Compressed keys: kbar_j = Mean(K[j*s : j*s + p]) for every complete kernel j.
// MiniCPM4 summary page, "InfLLM v2" section, paragraph "Semantic kernels for
// block relevance scoring" (eq. S, "What this computes", "Why mean pooling").
//
// HBM-streaming kernel: each 256-thread block owns 16 consecutive kernels of one
// (sequence, KV head); 32 threads cover one 128-wide key row with 4 lanes of
// d each.  The p keys of a kernel are summed in float64 (exact for bf16 keys and
// for p up to 2^21), divided by p, and rounded once to the storage type.  The
// overlapping tokens (p > s) are re-read from L1/L2, so HBM sees each key once.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kCompressKpb = 16;   // kernels per thread block
constexpr int kCompressFew = 4;    // up to this many new kernels: one block per kernel

template <typename Tin, bool kCkBf16>
__global__ __launch_bounds__(256) void compress_kernel(
    const Tin* __restrict__ k, const int64_t* __restrict__ kv_off,
    const int64_t* __restrict__ kv_lens, const int64_t* __restrict__ ck_off,
    const int64_t* __restrict__ ck_begin, void* __restrict__ ck_out, int hkv, int p, int s) {
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t o0 = kv_off[b], cap = kv_off[b + 1] - o0;
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const int64_t nc = num_kernels(n, p, s);
    const int64_t c0 = ck_off[b], ccap = ck_off[b + 1] - c0;
    const int64_t jb = ck_begin ? ck_begin[b] : 0;
    const int col = (threadIdx.x & 31) * 4;
    const Tin* kh = k + (o0 * hkv + static_cast<int64_t>(h) * cap) * kHeadDim + col;

    for (int r = threadIdx.x >> 5; r < kCompressKpb; r += 8) {
        const int64_t j = jb + static_cast<int64_t>(blockIdx.x) * kCompressKpb + r;
        if (j < 0 || j >= nc || j >= ccap) continue;
        double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
        const Tin* src = kh + j * s * kHeadDim;
        // batches of 8 independent loads keep the memory pipeline full; the sum
        // itself still runs over t in order
        int t = 0;
        for (; t + 8 <= p; t += 8) {
            float v[8][4];
#pragma unroll
            for (int u = 0; u < 8; ++u) load4(src + static_cast<int64_t>(t + u) * kHeadDim, v[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) { acc0 += v[u][0]; acc1 += v[u][1]; acc2 += v[u][2]; acc3 += v[u][3]; }
        }
        for (; t < p; ++t) {
            float v[4];
            load4(src + static_cast<int64_t>(t) * kHeadDim, v);
            acc0 += v[0]; acc1 += v[1]; acc2 += v[2]; acc3 += v[3];
        }
        const double pd = static_cast<double>(p);
        const double m0 = acc0 / pd, m1 = acc1 / pd, m2 = acc2 / pd, m3 = acc3 / pd;
        const int64_t dst = ((c0 * hkv + static_cast<int64_t>(h) * ccap) + j) * kHeadDim + col;
        if (kCkBf16) {
            bf16_t* o = static_cast<bf16_t*>(ck_out) + dst;
            uint2 w;
            w.x = static_cast<uint32_t>(f64_to_bf16(m0)) | (static_cast<uint32_t>(f64_to_bf16(m1)) << 16);
            w.y = static_cast<uint32_t>(f64_to_bf16(m2)) | (static_cast<uint32_t>(f64_to_bf16(m3)) << 16);
            *reinterpret_cast<uint2*>(o) = w;
        } else {
            float* o = static_cast<float*>(ck_out) + dst;
            *reinterpret_cast<float4*>(o) = make_float4(static_cast<float>(m0), static_cast<float>(m1),
                                                        static_cast<float>(m2), static_cast<float>(m3));
        }
    }
}

// Few new kernels per sequence (a decode step completes at most one): one block
// per kernel, the p rows split over 8 groups of 32 lanes so that every row is
// loaded in the same memory round trip, then the 8 float64 partial sums are
// added in LDS.
template <typename Tin, bool kCkBf16>
__global__ __launch_bounds__(256) void compress_few_kernel(
    const Tin* __restrict__ k, const int64_t* __restrict__ kv_off,
    const int64_t* __restrict__ kv_lens, const int64_t* __restrict__ ck_off,
    const int64_t* __restrict__ ck_begin, void* __restrict__ ck_out, int hkv, int p, int s,
    int last_only) {
    __shared__ double part[8][kHeadDim];
    const int b = blockIdx.z, h = blockIdx.y;
    const int64_t o0 = kv_off[b], cap = kv_off[b + 1] - o0;
    int64_t n = kv_lens ? kv_lens[b] : cap;
    n = n < cap ? n : cap;
    const int64_t nc = num_kernels(n, p, s);
    const int64_t c0 = ck_off[b], ccap = ck_off[b + 1] - c0;
    // last_only: the kernel that the newest token n - 1 completes, if it completes one
    const int64_t j = last_only ? ((n >= p && (n - p) % s == 0) ? (n - p) / s : -1)
                                : (ck_begin ? ck_begin[b] : 0) + blockIdx.x;
    if (j < 0 || j >= nc || j >= ccap) return;          // uniform over the block
    const int grp = threadIdx.x >> 5, col = (threadIdx.x & 31) * 4;
    const Tin* src = k + (o0 * hkv + static_cast<int64_t>(h) * cap + j * s) * kHeadDim + col;
    double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
    for (int t0 = grp; t0 < p; t0 += 64) {               // up to 8 rows per batch
        float v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = t0 + 8 * u;
            if (t < p) load4(src + static_cast<int64_t>(t) * kHeadDim, v[u]);
            else v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) { acc0 += v[u][0]; acc1 += v[u][1]; acc2 += v[u][2]; acc3 += v[u][3]; }
    }
    part[grp][col] = acc0; part[grp][col + 1] = acc1; part[grp][col + 2] = acc2; part[grp][col + 3] = acc3;
    __syncthreads();
    if (threadIdx.x >= kHeadDim) return;
    const int d = threadIdx.x;
    double sum = 0.0;
#pragma unroll
    for (int g2 = 0; g2 < 8; ++g2) sum += part[g2][d];
    const double mean = sum / static_cast<double>(p);
    const int64_t dst = ((c0 * hkv + static_cast<int64_t>(h) * ccap) + j) * kHeadDim + d;
    if (kCkBf16) static_cast<bf16_t*>(ck_out)[dst] = f64_to_bf16(mean);
    else static_cast<float*>(ck_out)[dst] = static_cast<float>(mean);
}

// One decode step's cache update: one block per sequence (all its KV heads, so
// the length is read by every thread before it is advanced).  Writes the new
// token's K and V rows at position n = kv_lens[b], then, if the token completes
// kernel j = (n + 1 - p) / s, its compressed key with the same float64 sum and
// single rounding as compress_kernel (the new row is taken from k_new, the
// p - 1 older rows from the cache), and finally kv_lens[b] = n + 1.  A full
// cache (n >= capacity) or a compressed-key region without room for kernel j
// leaves the sequence unchanged.
template <typename Tin, bool kCkBf16>
__global__ __launch_bounds__(256) void append_kv_kernel(
    const Tin* __restrict__ k_new, const Tin* __restrict__ v_new, Tin* __restrict__ k,
    Tin* __restrict__ v, const int64_t* __restrict__ kv_off, int64_t* __restrict__ kv_lens,
    const int64_t* __restrict__ ck_off, void* __restrict__ ck_out, int hkv, int p, int s) {
    __shared__ double part[8][kHeadDim];
    const int b = blockIdx.x, t = threadIdx.x;
    const int64_t o0 = kv_off[b], cap = kv_off[b + 1] - o0;
    const int64_t n = kv_lens[b];
    if (n < 0 || n >= cap) return;                       // uniform: full cache, no change
    const int64_t c0 = ck_off[b], ccap = ck_off[b + 1] - c0;
    const bool completes = n + 1 >= p && (n + 1 - p) % s == 0;
    const int64_t j = completes ? (n + 1 - p) / s : -1;
    const bool store_ck = completes && j < ccap;
    const int grp = t >> 5, col = (t & 31) * 4;
    for (int g = 0; g < hkv; ++g) {
        const Tin* kn = k_new + (static_cast<int64_t>(b) * hkv + g) * kHeadDim;
        const Tin* vn = v_new + (static_cast<int64_t>(b) * hkv + g) * kHeadDim;
        const int64_t row0 = (o0 * hkv + static_cast<int64_t>(g) * cap) * kHeadDim;
        if (t < kHeadDim) k[row0 + n * kHeadDim + t] = kn[t];
        else v[row0 + n * kHeadDim + (t - kHeadDim)] = vn[t - kHeadDim];
        if (!store_ck) continue;                         // uniform
        // rows j s .. j s + p - 1; the last one is the new token
        double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
        for (int r = grp; r < p; r += 8) {
            float x[4];
            if (r == p - 1) load4(kn + col, x);
            else load4(k + row0 + (j * s + r) * kHeadDim + col, x);
            acc0 += x[0]; acc1 += x[1]; acc2 += x[2]; acc3 += x[3];
        }
        part[grp][col] = acc0; part[grp][col + 1] = acc1; part[grp][col + 2] = acc2; part[grp][col + 3] = acc3;
        __syncthreads();
        if (t < kHeadDim) {
            double sum = 0.0;
#pragma unroll
            for (int g2 = 0; g2 < 8; ++g2) sum += part[g2][t];
            const double mean = sum / static_cast<double>(p);
            const int64_t dst = ((c0 * hkv + static_cast<int64_t>(g) * ccap) + j) * kHeadDim + t;
            if (kCkBf16) static_cast<bf16_t*>(ck_out)[dst] = f64_to_bf16(mean);
            else static_cast<float*>(ck_out)[dst] = static_cast<float>(mean);
        }
        __syncthreads();                                 // part reused by the next head
    }
    __syncthreads();                                     // every thread has read kv_lens[b]
    if (t == 0) kv_lens[b] = n + 1;
}

hipError_t launch_append_kv(const Shape& sh, const void* k_new, const void* v_new, void* k,
                            void* v, const int64_t* kv_off, int64_t* kv_lens,
                            const int64_t* ck_off, void* ck, int batch, hipStream_t st) {
#define INFV2_APPEND(TIN, CKB) launch_timed(INFV2_KERNEL_APPEND, append_kv_kernel<TIN, CKB>, \
        dim3(batch), dim3(256), 0, st, static_cast<const TIN*>(k_new), static_cast<const TIN*>(v_new), static_cast<TIN*>(k), \
        static_cast<TIN*>(v), kv_off, kv_lens, ck_off, ck, sh.hkv, sh.p, sh.s)
    if (sh.io_bf16) { if (sh.ck_bf16) INFV2_APPEND(bf16_t, true); else INFV2_APPEND(bf16_t, false); }
    else { if (sh.ck_bf16) INFV2_APPEND(float, true); else INFV2_APPEND(float, false); }
#undef INFV2_APPEND
    return hipGetLastError();
}

hipError_t launch_compress(const Shape& sh, const void* k, const int64_t* kv_off,
                           const int64_t* kv_lens, const int64_t* ck_off, const int64_t* ck_begin,
                           int batch, int64_t max_new, void* ck, hipStream_t st, bool last_only) {
    if (max_new <= 0) return hipSuccess;
    KernelTimer kt(INFV2_KERNEL_COMPRESS, st);
    if (max_new <= kCompressFew || last_only) {
        const dim3 g1(last_only ? 1u : static_cast<unsigned>(max_new), sh.hkv, batch);
        const int lo = last_only ? 1 : 0;
#define INFV2_FEW(TIN, CKB) compress_few_kernel<TIN, CKB><<<g1, 256, 0, st>>>(static_cast<const TIN*>(k), kv_off, kv_lens, ck_off, ck_begin, ck, sh.hkv, sh.p, sh.s, lo)
        if (sh.io_bf16) { if (sh.ck_bf16) INFV2_FEW(bf16_t, true); else INFV2_FEW(bf16_t, false); }
        else { if (sh.ck_bf16) INFV2_FEW(float, true); else INFV2_FEW(float, false); }
#undef INFV2_FEW
        return hipGetLastError();
    }
    dim3 grid(static_cast<unsigned>((max_new + kCompressKpb - 1) / kCompressKpb), sh.hkv, batch);
    if (sh.io_bf16) {
        if (sh.ck_bf16)
            compress_kernel<bf16_t, true><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(k), kv_off, kv_lens, ck_off, ck_begin, ck, sh.hkv, sh.p, sh.s);
        else
            compress_kernel<bf16_t, false><<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(k), kv_off, kv_lens, ck_off, ck_begin, ck, sh.hkv, sh.p, sh.s);
    } else {
        if (sh.ck_bf16)
            compress_kernel<float, true><<<grid, 256, 0, st>>>(static_cast<const float*>(k), kv_off, kv_lens, ck_off, ck_begin, ck, sh.hkv, sh.p, sh.s);
        else
            compress_kernel<float, false><<<grid, 256, 0, st>>>(static_cast<const float*>(k), kv_off, kv_lens, ck_off, ck_begin, ck, sh.hkv, sh.p, sh.s);
    }
    return hipGetLastError();
}

}  // namespace infv2
