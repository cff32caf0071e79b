// extern "C" entry points of libinfv2: host-side validation, workspace sizing
// and dispatch to the HIP launchers.  Every check runs before the first HIP
// call, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/infv2.h"
#include "kernels.hpp"

using infv2::Shape;

namespace {

constexpr int64_t kMaxBlocks = 16384;   // per sequence (top-k keys per row)
constexpr int kMaxTopk = 1024;

bool dtype_ok(int32_t d) { return d == INFV2_FP32 || d == INFV2_BF16; }

int32_t check_config(const infv2_config* c) {
    if (!c) return INFV2_ERR_NULL;
    if (c->head_dim <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 ||
        c->kernel_size <= 0 || c->kernel_stride <= 0 || c->topk <= 0 || c->init_blocks < 0 ||
        c->local_blocks < 0)
        return INFV2_ERR_SHAPE;
    if (c->num_q_heads % c->num_kv_heads != 0) return INFV2_ERR_SHAPE;
    if (c->kernel_size < c->kernel_stride) return INFV2_ERR_SHAPE;
    if (c->topk < static_cast<int64_t>(c->init_blocks) + c->local_blocks) return INFV2_ERR_SHAPE;
    if (!dtype_ok(c->io_dtype) || !dtype_ok(c->ck_dtype)) return INFV2_ERR_SHAPE;
    // scales: 0 selects the default (make_shape), negative values are rejected
    if (!isfinite(c->score_scale) || !isfinite(c->attn_scale)) return INFV2_ERR_SHAPE;
    if (c->score_scale < 0.f || c->attn_scale < 0.f) return INFV2_ERR_SHAPE;
    // implemented subset
    if (c->head_dim != infv2::kHeadDim) return INFV2_ERR_UNSUPPORTED;
    if (c->num_q_heads / c->num_kv_heads != infv2::kGroup) return INFV2_ERR_UNSUPPORTED;
    if (c->block_size % 16 != 0 || c->block_size > 256) return INFV2_ERR_UNSUPPORTED;
    if (c->kernel_size > 256) return INFV2_ERR_UNSUPPORTED;
    if (c->topk > kMaxTopk) return INFV2_ERR_UNSUPPORTED;
    return INFV2_OK;
}

int32_t check_len(const infv2_config* c, int64_t max_len) {
    if (max_len < 0) return INFV2_ERR_SHAPE;
    if ((max_len + c->block_size - 1) / c->block_size > kMaxBlocks) return INFV2_ERR_UNSUPPORTED;
    return INFV2_OK;
}

Shape make_shape(const infv2_config* c) {
    Shape s;
    s.hq = c->num_q_heads; s.hkv = c->num_kv_heads; s.d = c->head_dim;
    s.m = c->block_size; s.p = c->kernel_size; s.s = c->kernel_stride;
    s.topk = c->topk; s.init = c->init_blocks; s.local = c->local_blocks;
    s.io_bf16 = c->io_dtype == INFV2_BF16; s.ck_bf16 = c->ck_dtype == INFV2_BF16;
    // defaults: selection logits unscaled, as printed in "Semantic kernels";
    // attention scaled by 1/sqrt(d), standard scaled dot-product attention
    s.score_scale = c->score_scale == 0.f ? 1.f : c->score_scale;
    s.attn_scale = c->attn_scale == 0.f ? static_cast<float>(1.0 / sqrt(static_cast<double>(c->head_dim)))
                                        : c->attn_scale;
    return s;
}

int32_t status_of(hipError_t e) { return e == hipSuccess ? INFV2_OK : INFV2_ERR_DEVICE; }

size_t ws_bytes_for(const infv2_config* c, int32_t op, int32_t rows, int32_t batch, int64_t max_len) {
    const Shape sh = make_shape(c);
    switch (op) {
        case INFV2_OP_SELECT_DECODE: return infv2::select_decode_ws(sh, batch, max_len).total;
        case INFV2_OP_SELECT_PREFILL:      // batch > 1: a varlen call's rows in one launch
            return infv2::select_prefill_ws(sh, rows, max_len,
                                            batch < 1 ? 1 : (batch < infv2::kVarlenMax ? batch : infv2::kVarlenMax)).total;
        case INFV2_OP_ATTN_DECODE: return infv2::attn_decode_ws(sh, batch).total;
        case INFV2_OP_ATTN_PREFILL: return infv2::attn_prefill_ws_bytes(sh, max_len);
        case INFV2_OP_ATTN_PREFILL_BWD: return rows > 0 ? infv2::bwd_ws(sh, rows, max_len).total : 0;
        case INFV2_OP_SELECT_COARSE_DECODE: return infv2::select_decode_ws(sh, batch, max_len).total_coarse;
        case INFV2_OP_SELECT_COARSE_PREFILL: return infv2::select_prefill_ws(sh, rows, max_len).total_coarse;
        case INFV2_OP_DECODE_STEP:
            return infv2::align256(infv2::select_decode_ws(sh, batch, max_len).total) +
                   infv2::attn_decode_ws(sh, batch).total;
        default: return 0;
    }
}

}  // namespace

extern "C" {

int32_t infv2_abi_version(void) { return INFV2_ABI_VERSION; }

const char* infv2_status_str(int32_t s) {
    switch (s) {
        case INFV2_OK: return "INFV2_OK";
        case INFV2_ERR_NULL: return "INFV2_ERR_NULL: a required pointer is NULL";
        case INFV2_ERR_SHAPE: return "INFV2_ERR_SHAPE: inconsistent sizes or parameters";
        case INFV2_ERR_UNSUPPORTED: return "INFV2_ERR_UNSUPPORTED: valid but not implemented on this path";
        case INFV2_ERR_WORKSPACE: return "INFV2_ERR_WORKSPACE: workspace missing or too small";
        case INFV2_ERR_DEVICE: return "INFV2_ERR_DEVICE: a HIP launch failed";
        case INFV2_ERR_SCRATCH: return "INFV2_ERR_SCRATCH: the call needs more than the library's static scratch";
        default: return "INFV2: unknown status";
    }
}

int64_t infv2_num_kernels(const infv2_config* c, int64_t n) {
    if (!c || c->kernel_size <= 0 || c->kernel_stride <= 0 || n < c->kernel_size) return 0;
    return (n - c->kernel_size) / c->kernel_stride + 1;
}

int32_t infv2_workspace_bytes(const infv2_config* c, int32_t op, int32_t rows, int32_t batch,
                              int64_t max_len, size_t* bytes) {
    if (!bytes) return INFV2_ERR_NULL;
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    if (op < INFV2_OP_COMPRESS || op > INFV2_OP_DECODE_STEP || rows < 0 || batch < 0) return INFV2_ERR_SHAPE;
    *bytes = ws_bytes_for(c, op, rows, batch, max_len);
    return INFV2_OK;
}

int32_t infv2_compress_keys(const infv2_config* c, const void* k, const int64_t* kv_offsets,
                            const int64_t* kv_lens, const int64_t* ck_offsets,
                            const int64_t* ck_begin, int32_t batch, int64_t max_len,
                            int64_t max_new, void* ck, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!k || !kv_offsets || !ck_offsets || !ck) return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const int64_t nc = infv2_num_kernels(c, max_len);
    if (max_new < 0 || max_new > nc) max_new = nc;
    return status_of(infv2::launch_compress(make_shape(c), k, kv_offsets, kv_lens, ck_offsets,
                                            ck_begin, batch, max_new, ck,
                                            static_cast<hipStream_t>(stream)));
}

int32_t infv2_append_kv(const infv2_config* c, const void* k_new, const void* v_new, void* k,
                        void* v, const int64_t* kv_offsets, int64_t* kv_lens,
                        const int64_t* ck_offsets, void* ck, int32_t batch, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!k_new || !v_new || !k || !v || !kv_offsets || !kv_lens || !ck_offsets || !ck)
        return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    return status_of(infv2::launch_append_kv(make_shape(c), k_new, v_new, k, v, kv_offsets,
                                             kv_lens, ck_offsets, ck, batch,
                                             static_cast<hipStream_t>(stream)));
}

int32_t infv2_select_blocks(const infv2_config* c, int32_t mode, const void* q, int32_t rows,
                            int64_t q_start, const void* ck, const int64_t* ck_offsets,
                            const int64_t* kv_offsets, const int64_t* kv_lens, int32_t batch,
                            int64_t max_len, int32_t* block_idx, float* block_score, void* ws,
                            size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !ck || !ck_offsets || !block_idx) return INFV2_ERR_NULL;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == INFV2_MODE_DECODE) {
        if (!kv_offsets) return INFV2_ERR_NULL;
        if (batch < 1 || rows != batch) return INFV2_ERR_SHAPE;
        const size_t need = ws_bytes_for(c, INFV2_OP_SELECT_DECODE, rows, batch, max_len);
        if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
        return status_of(infv2::launch_select_decode(make_shape(c), q, ck, ck_offsets, kv_offsets,
                                                     kv_lens, batch, max_len, block_idx,
                                                     block_score, ws, nullptr, s));
    }
    if (mode == INFV2_MODE_PREFILL) {
        if (batch != 1 || rows < 0 || q_start < 0) return INFV2_ERR_SHAPE;
        if (q_start + rows > max_len) return INFV2_ERR_SHAPE;
        if (rows == 0) return INFV2_OK;
        const size_t need = ws_bytes_for(c, INFV2_OP_SELECT_PREFILL, rows, batch, max_len);
        if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
        return status_of(infv2::launch_select_prefill(make_shape(c), q, rows, q_start, ck,
                                                      ck_offsets, max_len, block_idx, block_score,
                                                      ws, nullptr, s));
    }
    return INFV2_ERR_SHAPE;
}

int32_t infv2_select_blocks_coarse(const infv2_config* c, int32_t coarse, int32_t mode,
                                   const void* q, int32_t rows, int64_t q_start, const void* ck,
                                   const int64_t* ck_offsets, const void* ck_coarse,
                                   const int64_t* ckc_offsets, const int64_t* kv_offsets,
                                   const int64_t* kv_lens, int32_t batch, int64_t max_len,
                                   int32_t* block_idx, float* block_score, void* ws,
                                   size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !ck || !ck_offsets || !ck_coarse || !ckc_offsets || !block_idx) return INFV2_ERR_NULL;
    if (coarse < c->kernel_size || coarse > 256 ||
        static_cast<int64_t>(coarse) > static_cast<int64_t>(c->topk) * c->block_size)
        return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const infv2::CoarseSel cs{coarse, ck_coarse, ckc_offsets};
    if (mode == INFV2_MODE_DECODE) {
        if (!kv_offsets) return INFV2_ERR_NULL;
        if (batch < 1 || rows != batch) return INFV2_ERR_SHAPE;
        const size_t need = ws_bytes_for(c, INFV2_OP_SELECT_COARSE_DECODE, rows, batch, max_len);
        if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
        return status_of(infv2::launch_select_decode(make_shape(c), q, ck, ck_offsets, kv_offsets,
                                                     kv_lens, batch, max_len, block_idx,
                                                     block_score, ws, &cs, s));
    }
    if (mode == INFV2_MODE_PREFILL) {
        if (batch != 1 || rows < 0 || q_start < 0) return INFV2_ERR_SHAPE;
        if (q_start + rows > max_len) return INFV2_ERR_SHAPE;
        if (rows == 0) return INFV2_OK;
        const size_t need = ws_bytes_for(c, INFV2_OP_SELECT_COARSE_PREFILL, rows, batch, max_len);
        if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
        return status_of(infv2::launch_select_prefill(make_shape(c), q, rows, q_start, ck,
                                                      ck_offsets, max_len, block_idx, block_score,
                                                      ws, &cs, s));
    }
    return INFV2_ERR_SHAPE;
}

int32_t infv2_sparse_attn_decode(const infv2_config* c, const void* q, const void* k,
                                 const void* v, const int64_t* kv_offsets, const int64_t* kv_lens,
                                 int32_t batch, int64_t max_len, const int32_t* block_idx,
                                 void* out, void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !block_idx || !out) return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const size_t need = ws_bytes_for(c, INFV2_OP_ATTN_DECODE, batch, batch, max_len);
    if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
    return status_of(infv2::launch_attn_decode(make_shape(c), q, k, v, kv_offsets, kv_lens, batch,
                                               block_idx, out, ws,
                                               static_cast<hipStream_t>(stream)));
}

int32_t infv2_sparse_attn_decode_noalloc(const infv2_config* c, const void* q, const void* k,
                                         const void* v, const int64_t* kv_offsets,
                                         const int64_t* kv_lens, int32_t batch, int64_t max_len,
                                         const int32_t* block_idx, void* out, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !block_idx || !out) return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const size_t need = ws_bytes_for(c, INFV2_OP_ATTN_DECODE, batch, batch, max_len);
    if (need > INFV2_NOALLOC_SCRATCH_BYTES) return INFV2_ERR_SCRATCH;
    void* scratch = nullptr;
    if (infv2::decode_scratch(&scratch) != hipSuccess) return INFV2_ERR_DEVICE;
    return status_of(infv2::launch_attn_decode(make_shape(c), q, k, v, kv_offsets, kv_lens, batch,
                                               block_idx, out, scratch,
                                               static_cast<hipStream_t>(stream)));
}

int32_t infv2_decode_step(const infv2_config* c, const void* q, const void* k, const void* v,
                          const int64_t* kv_offsets, const int64_t* kv_lens,
                          const int64_t* ck_offsets, void* ck, int32_t batch, int64_t max_len,
                          int32_t* block_idx, void* out, void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !ck_offsets || !ck || !block_idx || !out)
        return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const size_t need = ws_bytes_for(c, INFV2_OP_DECODE_STEP, batch, batch, max_len);
    if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
    const Shape sh = make_shape(c);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const infv2::SelectDecodeWs sw = infv2::select_decode_ws(sh, batch, max_len);
    char* ws_attn = static_cast<char*>(ws) + infv2::align256(sw.total);
    hipError_t e;
    if (sh.io_bf16) {
        // the selection's first kernel also builds the newest token's compressed
        // key, and the attention makes the top-k selection itself from the
        // block-score keys
        const infv2::AttnDecodeWs aw = infv2::attn_decode_ws(sh, batch);
        const bool fused = infv2::attn_decode_topk_ok(sh, sw.nblk_max);
        e = infv2::launch_select_decode(sh, q, ck, ck_offsets, kv_offsets, kv_lens, batch, max_len,
                                        block_idx, nullptr, ws, nullptr, s, k, fused);
        if (e != hipSuccess) return INFV2_ERR_DEVICE;
        if (fused) {
            const uint32_t* keys = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + sw.keys);
            float* po = reinterpret_cast<float*>(ws_attn + aw.part_o);
            float2* pml = reinterpret_cast<float2*>(ws_attn + aw.part_ml);
            e = infv2::launch_attn_decode_topk(sh, q, k, v, kv_offsets, kv_lens, batch, keys,
                                               sw.keys_ld, sw.nblk_max, block_idx, po, pml,
                                               aw.nsplit_m, aw.tpw, s);
            if (e != hipSuccess) return status_of(e);
            return status_of(infv2::launch_attn_decode_merge(sh, po, pml, out, batch, aw.nsplit_m, s));
        }
    } else {
        e = infv2::launch_compress(sh, k, kv_offsets, kv_lens, ck_offsets, nullptr, batch, 1, ck, s,
                                   true);
        if (e == hipSuccess)
            e = infv2::launch_select_decode(sh, q, ck, ck_offsets, kv_offsets, kv_lens, batch,
                                            max_len, block_idx, nullptr, ws, nullptr, s);
    }
    if (e != hipSuccess) return INFV2_ERR_DEVICE;
    return status_of(infv2::launch_attn_decode(sh, q, k, v, kv_offsets, kv_lens, batch, block_idx,
                                               out, ws_attn, s));
}

int32_t infv2_decode_step_append(const infv2_config* c, const void* q, const void* k_new,
                                 const void* v_new, void* k, void* v, const int64_t* kv_offsets,
                                 int64_t* kv_lens, const int64_t* ck_offsets, void* ck,
                                 int32_t batch, int64_t max_len, int32_t* block_idx, void* out,
                                 void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k_new || !v_new || !k || !v || !kv_offsets || !kv_lens || !ck_offsets || !ck ||
        !block_idx || !out)
        return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, max_len)) != INFV2_OK) return st;
    const size_t need = ws_bytes_for(c, INFV2_OP_DECODE_STEP, batch, batch, max_len);
    if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
    Shape sh = make_shape(c);
    const infv2::SelectDecodeWs sw = infv2::select_decode_ws(sh, batch, max_len);
    if (!sh.io_bf16 || !infv2::attn_decode_topk_ok(sh, sw.nblk_max)) {
        // the two calls it stands for
        if ((st = infv2_append_kv(c, k_new, v_new, k, v, kv_offsets, kv_lens, ck_offsets, ck, batch,
                                  stream)) != INFV2_OK)
            return st;
        return infv2_decode_step(c, q, k, v, kv_offsets, kv_lens, ck_offsets, ck, batch, max_len,
                                 block_idx, out, ws, ws_bytes, stream);
    }
    // the step's kernels see kv_lens[b] + 1; the logits kernel writes the new
    // token into the caches (and builds the kernel it completes from it), the
    // merge kernel stores the new lengths
    sh.lens_plus_one = 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws_attn = static_cast<char*>(ws) + infv2::align256(sw.total);
    const infv2::AttnDecodeWs aw = infv2::attn_decode_ws(sh, batch);
    const infv2::DecAppend app{k_new, v_new, k, v};
    hipError_t e = infv2::launch_select_decode(sh, q, ck, ck_offsets, kv_offsets, kv_lens, batch,
                                               max_len, block_idx, nullptr, ws, nullptr, s, k, true,
                                               &app);
    if (e != hipSuccess) return INFV2_ERR_DEVICE;
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + sw.keys);
    float* po = reinterpret_cast<float*>(ws_attn + aw.part_o);
    float2* pml = reinterpret_cast<float2*>(ws_attn + aw.part_ml);
    e = infv2::launch_attn_decode_topk(sh, q, k, v, kv_offsets, kv_lens, batch, keys, sw.keys_ld,
                                       sw.nblk_max, block_idx, po, pml, aw.nsplit_m, aw.tpw, s);
    if (e != hipSuccess) return status_of(e);
    return status_of(infv2::launch_attn_decode_merge(sh, po, pml, out, batch, aw.nsplit_m, s, kv_lens,
                                                     kv_offsets));
}

int32_t infv2_sparse_attn_prefill(const infv2_config* c, const void* q, int32_t rows,
                                  int64_t q_start, const void* k, const void* v,
                                  const int64_t* kv_offsets, const int32_t* block_idx, void* out,
                                  void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !block_idx || !out) return INFV2_ERR_NULL;
    if (rows < 0 || q_start < 0) return INFV2_ERR_SHAPE;
    if ((st = check_len(c, q_start + rows)) != INFV2_OK) return st;
    if (rows == 0) return INFV2_OK;
    const size_t need = ws_bytes_for(c, INFV2_OP_ATTN_PREFILL, rows, 1, q_start + rows);
    if (need > 0 && (!ws || ws_bytes < need)) return INFV2_ERR_WORKSPACE;
    return status_of(infv2::launch_attn_prefill(make_shape(c), q, rows, q_start, k, v, kv_offsets,
                                                block_idx, out, ws,
                                                static_cast<hipStream_t>(stream)));
}

int32_t infv2_sparse_attn_prefill_bwd(const infv2_config* c, const void* q, int32_t rows,
                                      int64_t q_start, const void* k, const void* v,
                                      const int64_t* kv_offsets, const int32_t* block_idx,
                                      const void* out, const void* dout, void* dq, void* dk,
                                      void* dv, void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !block_idx || !out || !dout || !dq || !dk || !dv)
        return INFV2_ERR_NULL;
    if (rows < 0 || q_start < 0) return INFV2_ERR_SHAPE;
    if (static_cast<int64_t>(rows) * c->topk > (int64_t(1) << 30)) return INFV2_ERR_UNSUPPORTED;
    if ((st = check_len(c, q_start + rows)) != INFV2_OK) return st;
    if (rows == 0) return INFV2_OK;
    const size_t need = ws_bytes_for(c, INFV2_OP_ATTN_PREFILL_BWD, rows, 1, q_start + rows);
    if (!ws || ws_bytes < need) return INFV2_ERR_WORKSPACE;
    return status_of(infv2::launch_attn_prefill_bwd(make_shape(c), q, rows, q_start, k, v,
                                                    kv_offsets, block_idx, out, dout, dq, dk, dv,
                                                    ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------- varlen prefill
// Several sequences per call (serving-style prefill).  Each sequence's rows run
// through the single-sequence path with its offsets advanced: kv_offsets + b
// and ck_offsets + b describe sequence b alone.  Every host array is checked
// before the first launch.

namespace {

int32_t check_varlen(const infv2_config* c, int32_t batch, const int32_t* rows,
                     const int64_t* q_start, int32_t op, size_t ws_bytes, const void* ws) {
    if (!rows || !q_start) return INFV2_ERR_NULL;
    if (batch < 1) return INFV2_ERR_SHAPE;
    size_t need = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (rows[b] < 0 || q_start[b] < 0) return INFV2_ERR_SHAPE;
        const int32_t st = check_len(c, q_start[b] + rows[b]);
        if (st != INFV2_OK) return st;
        if (rows[b] == 0) continue;
        const size_t nb = ws_bytes_for(c, op, rows[b], 1, q_start[b] + rows[b]);
        need = nb > need ? nb : need;
    }
    if (need > 0 && (!ws || ws_bytes < need)) return INFV2_ERR_WORKSPACE;
    return INFV2_OK;
}

}  // namespace

extern "C" {

int32_t infv2_select_blocks_varlen(const infv2_config* c, const void* q, int32_t batch,
                                   const int32_t* rows_per_seq, const int64_t* q_start_per_seq,
                                   const void* ck, const int64_t* ck_offsets,
                                   const int64_t* kv_offsets, int32_t* block_idx,
                                   float* block_score, void* ws, size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !ck || !ck_offsets || !kv_offsets || !block_idx) return INFV2_ERR_NULL;
    if ((st = check_varlen(c, batch, rows_per_seq, q_start_per_seq, INFV2_OP_SELECT_PREFILL,
                           ws_bytes, ws)) != INFV2_OK)
        return st;
    const Shape sh = make_shape(c);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t qrow = static_cast<size_t>(c->num_q_heads) * c->head_dim *
                        (c->io_dtype == INFV2_BF16 ? 2 : 4);
    const size_t irow = static_cast<size_t>(c->num_kv_heads) * c->topk;
    if (sh.io_bf16) {
        // one launch per kernel for up to kVarlenMax sequences, when the workspace
        // holds all of their rows (else sequence after sequence, below)
        int64_t total = 0, max_len = 0;
        int nseq = 0;
        for (int32_t b = 0; b < batch; ++b) {
            if (rows_per_seq[b] <= 0) continue;
            total += rows_per_seq[b];
            ++nseq;
            const int64_t e = q_start_per_seq[b] + rows_per_seq[b];
            max_len = e > max_len ? e : max_len;
        }
        if (nseq > 0 && total <= INT32_MAX &&
            ws_bytes >= ws_bytes_for(c, INFV2_OP_SELECT_PREFILL, static_cast<int32_t>(total), nseq, max_len)) {
            infv2::PrefillSeqs seqs{};
            int grp = 0;
            int64_t base = 0;                  // packed row of the table's row 0
            auto flush = [&]() -> bool {
                const bool ok = seqs.n == 0 ||
                    infv2::launch_select_prefill_seqs(
                        sh, seqs, static_cast<const char*>(q) + base * qrow, ck, ck_offsets, max_len,
                        block_idx + base * irow, block_score ? block_score + base * irow : nullptr,
                        ws, s) == hipSuccess;
                seqs = infv2::PrefillSeqs{};
                grp = 0;
                return ok;
            };
            int64_t r0 = 0;
            for (int32_t b = 0; b < batch; ++b) {
                const int32_t rows = rows_per_seq[b];
                const int ng = (rows + 15) / 16;
                if (rows > 0) {
                    if (seqs.n == infv2::kVarlenMax || grp + ng > infv2::kVarlenMaxGroups) {
                        if (!flush()) return INFV2_ERR_DEVICE;
                    }
                    if (seqs.n == 0) base = r0;
                    const int i = seqs.n++;
                    grp += ng;
                    seqs.grp_end[i] = grp;
                    seqs.seq[i] = b;
                    seqs.row0[i] = r0 - base;
                    seqs.rows[i] = rows;
                    seqs.q_start[i] = q_start_per_seq[b];
                }
                r0 += rows;
            }
            return flush() ? INFV2_OK : INFV2_ERR_DEVICE;
        }
    }
    int64_t r0 = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t rows = rows_per_seq[b];
        if (rows > 0) {
            const hipError_t e = infv2::launch_select_prefill(
                sh, static_cast<const char*>(q) + r0 * qrow, rows, q_start_per_seq[b], ck,
                ck_offsets + b, q_start_per_seq[b] + rows, block_idx + r0 * irow,
                block_score ? block_score + r0 * irow : nullptr, ws, nullptr, s);
            if (e != hipSuccess) return INFV2_ERR_DEVICE;
        }
        r0 += rows;
    }
    return INFV2_OK;
}

int32_t infv2_sparse_attn_prefill_varlen(const infv2_config* c, const void* q, int32_t batch,
                                         const int32_t* rows_per_seq,
                                         const int64_t* q_start_per_seq, const void* k,
                                         const void* v, const int64_t* kv_offsets,
                                         const int32_t* block_idx, void* out, void* ws,
                                         size_t ws_bytes, void* stream) {
    int32_t st = check_config(c);
    if (st != INFV2_OK) return st;
    if (!q || !k || !v || !kv_offsets || !block_idx || !out) return INFV2_ERR_NULL;
    if ((st = check_varlen(c, batch, rows_per_seq, q_start_per_seq, INFV2_OP_ATTN_PREFILL,
                           ws_bytes, ws)) != INFV2_OK)
        return st;
    const Shape sh = make_shape(c);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (infv2::attn_prefill_mfma_ok(sh)) {
        // one launch per kVarlenMax sequences (with rows) of the call
        infv2::PrefillSeqs seqs{};
        int grp = 0;
        auto flush = [&]() -> bool {
            const bool ok = seqs.n == 0 ||
                infv2::launch_attn_prefill_mfma_seqs(sh, seqs, q, k, v, kv_offsets, block_idx, out,
                                                     s) == hipSuccess;
            seqs = infv2::PrefillSeqs{};
            grp = 0;
            return ok;
        };
        int64_t r0 = 0;
        for (int32_t b = 0; b < batch; ++b) {
            const int32_t rows = rows_per_seq[b];
            const int ng = (rows + 15) / 16;
            if (rows > 0) {
                if ((seqs.n == infv2::kVarlenMax || grp + ng > infv2::kVarlenMaxGroups) && !flush())
                    return INFV2_ERR_DEVICE;
                const int i = seqs.n++;
                grp += ng;
                seqs.grp_end[i] = grp;
                seqs.seq[i] = b;
                seqs.row0[i] = r0;
                seqs.rows[i] = rows;
                seqs.q_start[i] = q_start_per_seq[b];
            }
            r0 += rows;
        }
        return flush() ? INFV2_OK : INFV2_ERR_DEVICE;
    }
    const size_t qrow = static_cast<size_t>(c->num_q_heads) * c->head_dim *
                        (c->io_dtype == INFV2_BF16 ? 2 : 4);
    const size_t irow = static_cast<size_t>(c->num_kv_heads) * c->topk;
    int64_t r0 = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t rows = rows_per_seq[b];
        if (rows > 0) {
            const hipError_t e = infv2::launch_attn_prefill(
                sh, static_cast<const char*>(q) + r0 * qrow, rows, q_start_per_seq[b], k, v,
                kv_offsets + b, block_idx + r0 * irow, static_cast<char*>(out) + r0 * qrow, ws, s);
            if (e != hipSuccess) return INFV2_ERR_DEVICE;
        }
        r0 += rows;
    }
    return INFV2_OK;
}

}  // extern "C"

