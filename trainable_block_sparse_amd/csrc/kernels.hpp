// Host-side launchers of the HIP kernels (defined in the .hip files).
// Arguments are already validated by the entry points in infv2_api.cpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/infv2.h"

namespace infv2 {

constexpr int kHeadDim = 128;     // d supported by the kernels
constexpr int kGroup = 16;        // query heads per KV head supported by the kernels

// Brackets the launches made in its scope with HIP events recorded on the
// stream while a timing session for the family (an infv2_kernel id) is open;
// does nothing otherwise (timing.cpp).  Used for families of several kernels.
class KernelTimer {
  public:
    KernelTimer(int kernel, hipStream_t st);
    ~KernelTimer();
    KernelTimer(const KernelTimer&) = delete;
    KernelTimer& operator=(const KernelTimer&) = delete;

  private:
    hipStream_t st_;
    void* stop_ = nullptr;
};

// Start and stop events for one launch of a kernel of family `kernel` on `st`
// while a timing session for that family is open and `st` is not capturing;
// both null otherwise (timing.cpp).
void launch_events(int kernel, hipStream_t st, hipEvent_t* start, hipEvent_t* stop);

// Launches f<<<grid, block, shmem, st>>>(args...) (arguments converted to the
// kernel's parameter types).  While a session for `kernel` is open the launch
// itself stamps the two events with the dispatch's begin and end, so the
// session sees the kernel's own duration, without the gaps that events recorded
// between launches add.
template <typename F, typename... Args>
inline void launch_timed(int kernel, F f, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                         Args... args) {
    hipEvent_t a = nullptr, b = nullptr;
    launch_events(kernel, st, &a, &b);
    hipExtLaunchKernelGGL(f, grid, block, shmem, st, a, b, 0u, args...);
}

struct Shape {
    int hq, hkv, d, m, p, s, topk, init, local;
    int io_bf16, ck_bf16;
    float score_scale, attn_scale;
    // decode step with the cache append folded in: every kernel of the step
    // takes a sequence's length as kv_lens[b] + 1 (capped at its capacity),
    // and the last kernel stores that length
    int lens_plus_one = 0;
};

// the new token of each sequence for a decode step that also appends it:
// k_new / v_new [batch][Hkv][d] (bf16), written into the caches k / v at
// position kv_lens[b] when it is below the capacity
struct DecAppend {
    const void* k_new;
    const void* v_new;
    void* k;
    void* v;
};

// workspace carving (all offsets 256-byte aligned)
struct SelectDecodeWs {
    size_t logits, partial, keys, total;
    size_t logits_c, partial_c, lse_c, total_coarse;   // coarse-kernel LSE variant
    int nchunk_a, nchunk_b;
    int64_t nc_max, nc_ld, nblk_max;   // nc_ld: logits row stride (multiple of 4)
    int64_t keys_ld;                   // block-key row stride (padded for the top-k)
};
SelectDecodeWs select_decode_ws(const Shape& sh, int batch, int64_t max_len);

// Sequences of one prefill launch (varlen calls: several; single-sequence calls:
// one), passed by value as kernel arguments.  Rows are packed sequence after
// sequence; group = 16 consecutive rows of one sequence.
constexpr int kVarlenMax = 64;          // sequences per launch
constexpr int kVarlenMaxGroups = 1 << 24;   // row groups per launch (grid of groups x KV heads)
struct PrefillSeqs {
    int n;                              // sequences in this launch (1 .. kVarlenMax)
    int grp_end[kVarlenMax];            // row groups of sequences 0 .. i together
    int seq[kVarlenMax];                // index into kv_offsets / ck_offsets
    int64_t row0[kVarlenMax];           // first packed row
    int rows[kVarlenMax];
    int64_t q_start[kVarlenMax];
};

struct SelectPrefillWs {
    size_t lse, keys, total;
    int64_t nblk_max;
    // fp32 compressed keys: their hi / lo bf16 rows, [seq][2][Hkv][ld][d], for
    // the fine kernels (hl, ld) and, in the coarse-LSE call, the coarse ones
    // (hlc, ldc; one sequence)
    size_t hl, hlc, total_coarse;
    int64_t ld, ldc;
};
// rows: all rows of the launch; nseq: its sequences (at most kVarlenMax)
SelectPrefillWs select_prefill_ws(const Shape& sh, int rows, int64_t max_len, int nseq = 1);

// Decode attention: each split gives one partial (max, sum, output) per head.
// Vector-ALU path (fp32): a split is bps selected blocks (1 or 4).  Matrix-core
// path (bf16): a split is four waves, each a run of tpw 16-key tiles.
constexpr int kDecodeFewBlocks = 256;   // vector-ALU: below this many 4-block splits, 1-block splits
constexpr int kDecodeWaveTarget = 2048; // matrix cores: waves in flight before runs grow past one tile
constexpr int kDecodeMaxTpw = 8;        // matrix cores: longest tile run of a wave
constexpr int kDecodeMaxSplit = 1024;   // splits the merge kernel takes
struct AttnDecodeWs {
    size_t part_o, part_ml, total;
    int nsplit, bps;              // vector-ALU path
    int nsplit_m, tpw;            // matrix-core path
};
AttnDecodeWs attn_decode_ws(const Shape& sh, int batch);

// last_only: for every sequence, only the kernel its newest token completes
// (if any); ck_begin is then ignored
hipError_t launch_compress(const Shape& sh, const void* k, const int64_t* kv_off,
                           const int64_t* kv_lens, const int64_t* ck_off, const int64_t* ck_begin,
                           int batch, int64_t max_new, void* ck, hipStream_t st,
                           bool last_only = false);

hipError_t launch_append_kv(const Shape& sh, const void* k_new, const void* v_new, void* k,
                            void* v, const int64_t* kv_off, int64_t* kv_lens,
                            const int64_t* ck_off, void* ck, int batch, hipStream_t st);

// pass 1 over coarse kernels (size = stride = coarse) with their compressed keys
struct CoarseSel {
    int coarse;
    const void* ckc;
    const int64_t* ckc_off;
};

// cs == nullptr: the exact selection.  fuse_k != nullptr (bf16 queries only):
// the cached keys, from which the first kernel also computes and stores the
// compressed key of the kernel each sequence's newest token completes.
// skip_topk: stop after the block-score keys (the workspace's `keys` rows), for
// launch_attn_decode_topk, which makes the selection itself.
hipError_t launch_select_decode(const Shape& sh, const void* q, const void* ck,
                                const int64_t* ck_off, const int64_t* kv_off,
                                const int64_t* kv_lens, int batch, int64_t max_len,
                                int32_t* idx, float* score, void* ws, const CoarseSel* cs,
                                hipStream_t st, const void* fuse_k = nullptr,
                                bool skip_topk = false, const DecAppend* app = nullptr);

hipError_t launch_select_prefill(const Shape& sh, const void* q, int rows, int64_t q_start,
                                 const void* ck, const int64_t* ck_off, int64_t max_len,
                                 int32_t* idx, float* score, void* ws, const CoarseSel* cs,
                                 hipStream_t st);
// bf16 queries: the sequences of `seqs` in one launch per kernel; q, idx, score
// point at the table's row 0 (row0 relative to it), ck_off at the offsets of
// sequence 0 of the call; ws sized by select_prefill_ws(rows of the table,
// max_len, seqs.n)
hipError_t launch_select_prefill_seqs(const Shape& sh, const PrefillSeqs& seqs, const void* q,
                                      const void* ck, const int64_t* ck_off, int64_t max_len,
                                      int32_t* idx, float* score, void* ws, hipStream_t st);

// Device address of this device's static decode scratch (INFV2_NOALLOC_SCRATCH_BYTES,
// looked up once per device); the no-allocation decode entry point passes it as
// the workspace.
hipError_t decode_scratch(void** ptr);

hipError_t launch_attn_decode(const Shape& sh, const void* q, const void* k, const void* v,
                              const int64_t* kv_off, const int64_t* kv_lens, int batch,
                              const int32_t* idx, void* out, void* ws, hipStream_t st);

hipError_t launch_attn_decode_mfma(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int tpw, hipStream_t st);
// lens_adv != nullptr: also advance lens_adv[b] by one where it is below the
// capacity (the step's append; no other kernel of the step is running then)
hipError_t launch_attn_decode_merge(const Shape& sh, const float* part_o, const float2* part_ml,
                                    void* out, int batch, int nsplit, hipStream_t st,
                                    int64_t* lens_adv = nullptr, const int64_t* kv_off = nullptr);
// Decode attention that first makes the top-k selection from the block-score
// keys (rows of kld, one per (sequence, KV head)) in every thread block, with
// the matrix-core path's splits (nsplit, tpw); split 0 stores the selection in
// idx.  attn_decode_topk_ok: shapes it takes.
bool attn_decode_topk_ok(const Shape& sh, int64_t nblk_max);
hipError_t launch_attn_decode_topk(const Shape& sh, const void* q, const void* k, const void* v,
                                   const int64_t* kv_off, const int64_t* kv_lens, int batch,
                                   const uint32_t* keys, int64_t kld, int64_t nblk_max,
                                   int32_t* idx, float* part_o, float2* part_ml, int nsplit,
                                   int tpw, hipStream_t st);

// the launch's sequence holding row group grp / packed row r (relative to row0[0])
__device__ __forceinline__ int seq_of_group(const PrefillSeqs& t, int grp) {
    int i = 0;
    while (i + 1 < t.n && grp >= t.grp_end[i]) ++i;
    return i;
}
__device__ __forceinline__ int seq_of_row(const PrefillSeqs& t, int64_t r) {
    int i = 0;
    while (i + 1 < t.n && r >= t.row0[i + 1]) ++i;
    return i;
}
// one-sequence table: rows at q_start, offsets kv/ck_off + 0
PrefillSeqs one_seq(int rows, int64_t q_start);

bool attn_prefill_mfma_ok(const Shape& sh);
// transposed 64-key tiles of K or V for the matrix-core prefill kernels
size_t attn_prefill_ws_bytes(const Shape& sh, int64_t max_len);
hipError_t launch_attn_prefill_mfma(const Shape& sh, const void* q, int rows, int64_t q_start,
                                    const void* k, const void* v, const int64_t* kv_off,
                                    const int32_t* idx, void* out, void* ws, hipStream_t st);
// the sequences of `seqs` in one launch; q, idx, out point at packed row 0 and
// kv_off at the offsets of sequence 0 of the call
hipError_t launch_attn_prefill_mfma_seqs(const Shape& sh, const PrefillSeqs& seqs, const void* q,
                                         const void* k, const void* v, const int64_t* kv_off,
                                         const int32_t* idx, void* out, hipStream_t st);

hipError_t launch_attn_prefill(const Shape& sh, const void* q, int rows, int64_t q_start,
                               const void* k, const void* v, const int64_t* kv_off,
                               const int32_t* idx, void* out, void* ws, hipStream_t st);

// backward of the prefill attention (attn_bwd.hip, attn_bwd_mfma.hip)
struct BwdWs {
    size_t lse, delta, counts, totals, col_start, list, extra, total;
    int nblk, nchunk;
    int64_t list_ld;
};
BwdWs bwd_ws(const Shape& sh, int rows, int64_t max_len);
bool bwd_mfma_ok(const Shape& sh);
size_t bwd_mfma_extra_bytes(const Shape& sh, const BwdWs& w);
hipError_t launch_inverse_index(const Shape& sh, const BwdWs& w, int rows, const int32_t* idx,
                                char* base, hipStream_t st);
hipError_t launch_attn_prefill_bwd(const Shape& sh, const void* q, int rows, int64_t q_start,
                                   const void* k, const void* v, const int64_t* kv_off,
                                   const int32_t* idx, const void* out, const void* dout,
                                   void* dq, void* dk, void* dv, void* ws, hipStream_t st);
hipError_t launch_attn_prefill_bwd_mfma(const Shape& sh, const BwdWs& w, const void* q, int rows,
                                        int64_t q_start, const void* k, const void* v,
                                        const int64_t* kv_off, const int32_t* idx,
                                        const void* out, const void* dout, void* dq, void* dk,
                                        void* dv, char* ws, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace infv2
