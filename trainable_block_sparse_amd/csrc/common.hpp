// Device helpers shared by the InfLLM v2 HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.hpp"

namespace infv2 {

constexpr int kWave = 64;

typedef uint16_t bf16_t;          // bf16 carried as its bit pattern
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even (gfx950 has a hardware conversion for this)
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(bf16_t, h);
}

// float64 -> bf16, one rounding to nearest even (including the subnormal range)
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return f32_to_bf16(static_cast<float>(x));
    int e;
    frexp(x, &e);                         // |x| in [2^(e-1), 2^e)
    const int ulp_exp = max(e - 1, -126) - 7;
    const double y = ldexp(rint(ldexp(x, -ulp_exp)), ulp_exp);
    const float f = static_cast<float>(y);   // exact (8 significant bits), or inf on overflow
    return static_cast<bf16_t>(__float_as_uint(f) >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ static __forceinline__ float load(const float* p) { return *p; }
    __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct io<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// load 4 consecutive elements as floats (16-byte aligned for float, 8-byte for bf16)
__device__ __forceinline__ void load4(const float* p, float* o) {
    float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float* o) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// ---------------------------------------------------------------- scores as sortable keys
// Block scores are >= 0 or -inf ("no visible kernel").  key = bits + 1 keeps the
// order of non-negative floats and maps -inf to 0, the smallest key.
__device__ __forceinline__ uint32_t score_to_key(float s) {
    return (s == -INFINITY) ? 0u : (__float_as_uint(s) + 1u);
}
__device__ __forceinline__ float key_to_score(uint32_t k) {
    return k == 0u ? -INFINITY : __uint_as_float(k - 1u);
}

// ---------------------------------------------------------------- method arithmetic helpers
__host__ __device__ __forceinline__ int64_t num_kernels(int64_t n, int p, int s) {
    return n < p ? 0 : (n - p) / s + 1;
}

// ---------------------------------------------------------------- wave reductions
// Data-parallel-primitive (DPP) lane moves of gfx9: within each row of 16 lanes
// row_shr:n reads lane i - n (0 or `old` where that leaves the row), and
// row_bcast:15 / row_bcast:31 hand lane 15 / lane 31 to the rows above.  A
// wave-wide inclusive scan or reduction is then four row shifts and two
// broadcasts: six register moves instead of six LDS permutes.
template <int kCtrl, int kRowMask = 0xf, bool kBoundZero = true>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t old, uint32_t src) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(src),
                                                             kCtrl, kRowMask, 0xf, kBoundZero));
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// inclusive prefix sum over the 64 lanes (lane 63 holds the total)
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v += dpp_mov<kDppShr1>(0u, v);
    v += dpp_mov<kDppShr2>(0u, v);
    v += dpp_mov<kDppShr4>(0u, v);
    v += dpp_mov<kDppShr8>(0u, v);
    v += dpp_mov<kDppBcast15, 0xa>(0u, v);
    v += dpp_mov<kDppBcast31, 0xc>(0u, v);
    return v;
}
// maximum / minimum over the 64 lanes, in every lane
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = max(v, dpp_mov<kDppShr1>(0u, v));
    v = max(v, dpp_mov<kDppShr2>(0u, v));
    v = max(v, dpp_mov<kDppShr4>(0u, v));
    v = max(v, dpp_mov<kDppShr8>(0u, v));
    v = max(v, dpp_mov<kDppBcast15, 0xa>(0u, v));
    v = max(v, dpp_mov<kDppBcast31, 0xc>(0u, v));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
    constexpr uint32_t kId = 0xffffffffu;
    v = min(v, dpp_mov<kDppShr1, 0xf, false>(kId, v));
    v = min(v, dpp_mov<kDppShr2, 0xf, false>(kId, v));
    v = min(v, dpp_mov<kDppShr4, 0xf, false>(kId, v));
    v = min(v, dpp_mov<kDppShr8, 0xf, false>(kId, v));
    v = min(v, dpp_mov<kDppBcast15, 0xa, false>(kId, v));
    v = min(v, dpp_mov<kDppBcast31, 0xc, false>(kId, v));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
    const uint32_t kId = __float_as_uint(-INFINITY);
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppShr1, 0xf, false>(kId, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppShr2, 0xf, false>(kId, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppShr4, 0xf, false>(kId, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppShr8, 0xf, false>(kId, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppBcast15, 0xa, false>(kId, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppBcast31, 0xc, false>(kId, __float_as_uint(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += __uint_as_float(dpp_mov<kDppShr1>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppShr2>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppShr4>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppShr8>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppBcast15, 0xa>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppBcast31, 0xc>(0u, __float_as_uint(v)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// reductions over aligned groups of 16 lanes (DPP rows): rotations by 8 and 4
// inside the row, then the two quad butterflies; every lane gets its row's result
constexpr int kDppRor8 = 0x128, kDppRor4 = 0x124, kDppQuadSwap2 = 0x4e, kDppQuadSwap1 = 0xb1;
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppRor8>(0u, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppRor4>(0u, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppQuadSwap2>(0u, __float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mov<kDppQuadSwap1>(0u, __float_as_uint(v))));
    return v;
}
__device__ __forceinline__ float sum16(float v) {
    v += __uint_as_float(dpp_mov<kDppRor8>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppRor4>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppQuadSwap2>(0u, __float_as_uint(v)));
    v += __uint_as_float(dpp_mov<kDppQuadSwap1>(0u, __float_as_uint(v)));
    return v;
}
// Across rows: lane l combined with lane l ^ 16 (l ^ 32) by one lane-swap
// instruction of gfx950 (v_permlane16_swap: odd rows of the first operand trade
// places with even rows of the second; v_permlane32_swap: the upper half of the
// first with the lower half of the second).  With both operands v, each lane
// ends up holding its own value in one result and its partner's in the other,
// so a sum or max of the two is exactly own (op) partner, with no LDS permute.
__device__ __forceinline__ float add_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace infv2

namespace infv2 {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

// D = A(16x32) * B(32x16) + C; lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16],
// C/D[4(l/16)+r][l%16]  (layout checked on gfx950)
__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D = A(16x16) * B(16x16) + C; lane l holds A[l%16][4(l/16)+e], B[4(l/16)+e][l%16]
__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// 16-byte load of data read once (selected K/V rows, compressed keys): the
// nontemporal hint streams it past the caches (+12 % read bandwidth measured)
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

// Valid length of sequence b from its offsets and the caller's lengths.  The
// launchers pass `lens` = kv_lens, or kv_offsets + 1 with lens_end = 1 when
// kv_lens is NULL, so the length is loaded unconditionally, together with the
// offsets (one memory round trip instead of two).  lens_end = 2: a decode step
// that appends the new token first, so the length is kv_lens[b] + 1.
__device__ __forceinline__ int64_t seq_len(int64_t o0, int64_t o1, int64_t lv, int lens_end) {
    const int64_t cap = o1 - o0;
    const int64_t n = lens_end == 1 ? cap : lv + (lens_end >> 1);
    return n < cap ? n : cap;
}

// two floats that hold bf16 values exactly -> packed bf16 pair (no rounding needed)
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
    // one byte permute: bytes 2, 3 of lo, then bytes 2, 3 of hi
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
// LDS byte offset of a __shared__ object: the low half of its generic address
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
// Direct global->LDS load of 16 B per lane (lane i writes bytes 16 i .. 16 i + 15
// from `lds`, which is wave-uniform).  Issued by hand: the compiler then knows
// nothing of the LDS write and does not wait for every outstanding load before
// each LDS read (it cannot tell the stages of a ring apart).  The caller waits
// for the load (s_waitcnt vmcnt) and synchronises before reading the data.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
// The same with a wave-uniform base address (held in SGPRs) and a 32-bit byte
// offset per lane: no 64-bit address arithmetic or registers per load.
__device__ __forceinline__ void dma16s(const void* base, uint32_t byte_off, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(byte_off), "s"(base),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
// wait for every outstanding global access of this wave, then a block barrier
__device__ __forceinline__ void dma_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}
// two floats -> packed bf16 pair, round to nearest even (one paired conversion)
__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const f32x2_v x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_v));
}

}  // namespace infv2

namespace infv2 {

// inclusive prefix sum over the threads of a block of kWaves waves; `tmp` holds kWaves words
template <int kWaves>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    v = wave_incl_sum(v);
    if (lane == 63) tmp[wid] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int w = 0; w < wid; ++w) add += tmp[w];
    __syncthreads();
    return v + add;
}

// the same with one barrier: `tmp` must not be written again before a barrier
// that follows this call; `total` receives the block's sum
template <int kWaves>
__device__ __forceinline__ uint32_t block_incl_scan_1b(uint32_t v, uint32_t* tmp, uint32_t& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    v = wave_incl_sum(v);
    if (lane == 63) tmp[wid] = v;
    __syncthreads();
    uint32_t add = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = tmp[w];
        add += (w < wid) ? x : 0u;
        tot += x;
    }
    total = tot;
    return v + add;
}

// 2^x on the transcendental unit (no denormal range handling: exp2(-inf) = 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace infv2
