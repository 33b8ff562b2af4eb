// attn_abi.cpp -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every entry point validates its host-side arguments first and returns a
// status without touching the HIP runtime when they are invalid; only then
// does it configure and launch the kernels on the caller's stream.  Nothing
// here allocates, synchronises or keeps state between calls.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/attn.h"
#include "launch.h"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_size(int dt) { return dt == ATTN_F32 ? 4 : ((dt == ATTN_BF16 || dt == ATTN_F16) ? 2 : 0); }

bool is16(int dt) { return dt == ATTN_BF16 || dt == ATTN_F16; }

// softmax_scale must be finite and positive, and large enough that s * log2(e)
// is a normal float: the kernels form masked weights as 2^(-inf * c - m), which
// is 0 only for c > 0 (c = 0 would give NaN, c < 0 would turn the mask around).
bool scale_ok(float s) {
    return std::isfinite(s) && (double)s * 1.4426950408889634 >= (double)FLT_MIN;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Keys per decode item: the caller's (a positive multiple of 32), or, for
// 0, 32 -- one wavefront chunk, the finest grain the runs can be cut at.
int resolve_split(int split) {
    if (split < 0 || split % 32 != 0) return -1;
    return split > 0 ? split : 32;
}

// Decode workspace: partial slots (runs + batch) x hq of d fp32 values; then
// (256-aligned) 2 fp32 words per slot and head (m, d'); then (256-aligned)
// two int32 per sequence (its first and last run).  runs is kDecodeMaxRuns
// for a caller's workspace (a size that holds on every device), the current
// device's run count for the built-in scratch.
struct DecodeLayout {
    int split;
    size_t ml_off;
    size_t runs_off;
    size_t total;
};

bool decode_layout(int batch, int hq, int hkv, int d, int mbs, int bs, int split_req, int runs,
                   DecodeLayout *L) {
    if (batch <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || mbs <= 0 || bs <= 0) return false;
    const int split = resolve_split(split_req);
    if (split <= 0) return false;
    if (runs <= 0 || runs > attn::kDecodeMaxRuns) return false;
    const size_t rows = ((size_t)runs + (size_t)batch) * (size_t)hq;
    L->split = split;
    L->ml_off = (rows * (size_t)d * sizeof(float) + 255) / 256 * 256;
    L->runs_off = (L->ml_off + rows * 2 * sizeof(float) + 255) / 256 * 256;
    L->total = L->runs_off + (size_t)batch * 2 * sizeof(int32_t);
    return true;
}

}  // namespace

ATTN_API const char *attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid or inconsistent sizes";
        case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, alignment or layout";
        case ATTN_ERR_WORKSPACE: return "workspace missing, too small or unaligned, or larger than the built-in decode scratch";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

ATTN_API int attn_version(void) { return kVersion; }

ATTN_API int kv_store_slots(const void *k, const void *v, void *k_cache, void *v_cache,
                            const int32_t *slot_mapping, int num_tokens, int num_kv_heads,
                            int head_dim, int num_blocks, int block_size, int dtype,
                            void *stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return ATTN_ERR_SHAPE;
    const int es = dtype_size(dtype);
    if (es == 0) return ATTN_ERR_UNSUPPORTED;
    if (num_tokens == 0) return ATTN_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping) return ATTN_ERR_NULL;
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * es;
    if (row_bytes % 16 != 0 || row_bytes > (1 << 30)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_UNSUPPORTED;
    const int64_t total_chunks = (int64_t)num_tokens * (row_bytes / 16);
    if ((total_chunks + 255) / 256 > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    return hip_status(attn::launch_kv_store(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                            (int)row_bytes, (int64_t)num_blocks * block_size,
                                            (hipStream_t)stream));
}

ATTN_API int attn_prefill_varlen(const void *q, const void *k, const void *v, void *o,
                                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                 int batch, int max_seqlen_q, int max_seqlen_k,
                                 int total_q, int total_k,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 float softmax_scale, int causal,
                                 const int32_t *block_table, int max_blocks_per_seq,
                                 int num_blocks, int block_size,
                                 int in_dtype, int out_dtype, void *stream) {
    // K and V may be NULL only when there is no key to read
    const bool no_keys = block_table == nullptr && total_k == 0;
    if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || (!no_keys && (!k || !v))) return ATTN_ERR_NULL;
    if (batch <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 ||
        num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (!scale_ok(softmax_scale)) return ATTN_ERR_SHAPE;
    const bool paged = block_table != nullptr;
    if (paged) {
        if (max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0) return ATTN_ERR_SHAPE;
        // the kernels form a cache slot (block * block_size + offset) in 32 bits
        if ((int64_t)num_blocks * block_size > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    } else if (total_k < 0) {
        return ATTN_ERR_SHAPE;
    }
    if (is16(in_dtype)) {
        if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
        if (paged && block_size % 64 != 0) return ATTN_ERR_UNSUPPORTED;
        if (out_dtype != ATTN_F32 && out_dtype != in_dtype) return ATTN_ERR_UNSUPPORTED;
    } else if (in_dtype == ATTN_F32) {
        if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
        if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    } else {
        return ATTN_ERR_UNSUPPORTED;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
    // grid bound: every launch shape derived below must fit a 32-bit grid
    const int64_t units = ((int64_t)max_seqlen_q + 31) / 32 * batch * num_q_heads;
    if (units > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (max_seqlen_q == 0 || total_q == 0) return ATTN_OK;

    attn::VarlenArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.block_table = block_table;
    a.batch = batch;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.total_q = total_q;
    a.total_k = paged ? 0 : total_k;
    a.hq = num_q_heads; a.hkv = num_kv_heads; a.d = head_dim;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a.causal = causal ? 1 : 0;
    a.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
    a.num_blocks = paged ? num_blocks : 0;
    a.block_size = paged ? block_size : 0;
    a.out_f32 = out_dtype == ATTN_F32;
    a.seqlens_q = nullptr;
    a.seqlens_k = nullptr;
    a.pad_q = 0;
    a.pad_k = 0;
    a.in_f16 = in_dtype == ATTN_F16;
    const hipError_t e = is16(in_dtype) ? attn::launch_prefill_mfma(a, (hipStream_t)stream)
                                        : attn::launch_prefill_f32(a, (hipStream_t)stream);
    return hip_status(e);
}

ATTN_API int attn_prefill_padded(const void *q, const void *k, const void *v, void *o,
                                 const int32_t *seqlens_q, const int32_t *seqlens_k,
                                 int batch, int max_seqlen_q, int max_seqlen_k,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 float softmax_scale, int causal, int in_dtype, int out_dtype,
                                 void *stream) {
    // K and V may be NULL only when there is no key to read
    if (!q || !o || !seqlens_q || !seqlens_k || (max_seqlen_k != 0 && (!k || !v))) return ATTN_ERR_NULL;
    if (batch <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (!scale_ok(softmax_scale)) return ATTN_ERR_SHAPE;
    if (is16(in_dtype)) {
        if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
        if (out_dtype != ATTN_F32 && out_dtype != in_dtype) return ATTN_ERR_UNSUPPORTED;
    } else if (in_dtype == ATTN_F32) {
        if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
        if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    } else {
        return ATTN_ERR_UNSUPPORTED;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
    const int64_t total_q = (int64_t)batch * max_seqlen_q, total_k = (int64_t)batch * max_seqlen_k;
    if (total_q > 0x7fffffffLL || total_k > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    const int64_t units = ((int64_t)max_seqlen_q + 31) / 32 * batch * num_q_heads;
    if (units > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (max_seqlen_q == 0) return ATTN_OK;

    attn::VarlenArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.cu_q = nullptr; a.cu_k = nullptr;
    a.block_table = nullptr;
    a.batch = batch;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.total_q = total_q;
    a.total_k = total_k;
    a.hq = num_q_heads; a.hkv = num_kv_heads; a.d = head_dim;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a.causal = causal ? 1 : 0;
    a.max_blocks_per_seq = 0;
    a.num_blocks = 0;
    a.block_size = 0;
    a.out_f32 = out_dtype == ATTN_F32;
    a.seqlens_q = seqlens_q;
    a.seqlens_k = seqlens_k;
    a.pad_q = max_seqlen_q;
    a.pad_k = max_seqlen_k;   // 0: every sequence has no key
    a.in_f16 = in_dtype == ATTN_F16;
    const hipError_t e = is16(in_dtype) ? attn::launch_prefill_mfma(a, (hipStream_t)stream)
                                        : attn::launch_prefill_f32(a, (hipStream_t)stream);
    return hip_status(e);
}

ATTN_API size_t attn_decode_workspace_bytes(int batch, int num_q_heads, int num_kv_heads,
                                            int head_dim, int max_blocks_per_seq,
                                            int block_size, int split_tokens) {
    DecodeLayout L;
    if (!decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                       split_tokens, attn::kDecodeMaxRuns, &L))
        return 0;
    return L.total;
}

namespace {

// Validation and argument set-up shared by the two decode entry points; the
// three workspace pointers are left for the caller to fill from L.
int decode_prepare(const void *q, const void *k_cache, const void *v_cache, void *o,
                   const int32_t *cache_seqlens, const int32_t *block_table, int batch,
                   int num_q_heads, int num_kv_heads, int head_dim, int max_blocks_per_seq,
                   int num_blocks, int block_size, float softmax_scale, int split_tokens,
                   int in_dtype, int out_dtype, attn::DecodeArgs *a, DecodeLayout *L) {
    if (!q || !k_cache || !v_cache || !o || !cache_seqlens || !block_table) return ATTN_ERR_NULL;
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (!scale_ok(softmax_scale)) return ATTN_ERR_SHAPE;
    if (!is16(in_dtype) || head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_F32 && out_dtype != in_dtype) return ATTN_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > 16) return ATTN_ERR_UNSUPPORTED;
    if (block_size % 64 != 0) return ATTN_ERR_UNSUPPORTED;
    if (split_tokens < 0 || split_tokens % 32 != 0) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return ATTN_ERR_UNSUPPORTED;
    if (!decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                       split_tokens, attn::kDecodeMaxRuns, L))
        return ATTN_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if ((int64_t)batch * num_q_heads * head_dim > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    a->q = q; a->k_cache = k_cache; a->v_cache = v_cache; a->o = o;
    a->cache_seqlens = cache_seqlens; a->block_table = block_table;
    a->batch = batch; a->hq = num_q_heads; a->hkv = num_kv_heads; a->d = head_dim;
    a->max_blocks_per_seq = max_blocks_per_seq; a->num_blocks = num_blocks; a->block_size = block_size;
    a->scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a->split_tokens = L->split;
    a->out_f32 = out_dtype == ATTN_F32;
    a->in_f16 = in_dtype == ATTN_F16;
    return ATTN_OK;
}

// Runs on the current device, then the launch on the workspace at ws.
int decode_launch(attn::DecodeArgs *a, const DecodeLayout &L, void *ws, void *stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return ATTN_ERR_HIP;
    a->n_runs = attn::decode_runs(a->hkv, cus);
    a->ws_o = reinterpret_cast<float *>(ws);
    a->ws_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.ml_off);
    a->ws_runs = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) + L.runs_off);
    return hip_status(attn::launch_decode(*a, (hipStream_t)stream));
}

}  // namespace

ATTN_API int attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                               void *o, const int32_t *cache_seqlens,
                               const int32_t *block_table, int batch, int num_q_heads,
                               int num_kv_heads, int head_dim, int max_blocks_per_seq,
                               int num_blocks, int block_size, float softmax_scale,
                               int split_tokens, int in_dtype, int out_dtype,
                               void *workspace, size_t workspace_bytes, void *stream) {
    attn::DecodeArgs a;
    DecodeLayout L;
    const int st = decode_prepare(q, k_cache, v_cache, o, cache_seqlens, block_table, batch, num_q_heads,
                                  num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, block_size,
                                  softmax_scale, split_tokens, in_dtype, out_dtype, &a, &L);
    if (st != ATTN_OK) return st;
    if (!workspace || workspace_bytes < L.total) return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_WORKSPACE;
    return decode_launch(&a, L, workspace, stream);
}

ATTN_API int attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                       void *o, const int32_t *cache_seqlens,
                                       const int32_t *block_table, int batch, int num_q_heads,
                                       int num_kv_heads, int head_dim, int max_blocks_per_seq,
                                       int num_blocks, int block_size, float softmax_scale,
                                       int split_tokens, int in_dtype, int out_dtype, void *stream) {
    attn::DecodeArgs a;
    DecodeLayout L;
    const int st = decode_prepare(q, k_cache, v_cache, o, cache_seqlens, block_table, batch, num_q_heads,
                                  num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, block_size,
                                  softmax_scale, split_tokens, in_dtype, out_dtype, &a, &L);
    if (st != ATTN_OK) return st;
    // a one-run layout is the smallest any device needs: a call beyond the
    // scratch even then is rejected before any HIP call
    if (!decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                       split_tokens, 1, &L) ||
        L.total > attn::kDecodeScratchBytes)
        return ATTN_ERR_WORKSPACE;
    // the layout for the runs this device uses; it must fit the per-device
    // scratch array
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return ATTN_ERR_HIP;
    if (!decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                       split_tokens, attn::decode_runs(num_kv_heads, cus), &L))
        return ATTN_ERR_SHAPE;
    if (L.total > attn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (attn::decode_scratch(&ws) != hipSuccess || ws == nullptr) return ATTN_ERR_HIP;
    return decode_launch(&a, L, ws, stream);
}

namespace {

// Unfused-baseline workspace: X fp32 then (256-aligned) A bf16, each
// [batch, hq, max_seqlen_q, ldx] with ldx = max_seqlen_k rounded up to 64,
// plus 64 (rows a power-of-two apart would fall on the same few memory
// channels when a wavefront writes 32 of them at once).
bool unfused_layout(int batch, int hq, int max_q, int max_k, int64_t *ldx, size_t *a_off, size_t *total) {
    if (batch <= 0 || hq <= 0 || max_q < 0 || max_k < 0) return false;
    const int64_t l = ((int64_t)max_k + 63) / 64 * 64 + 64;
    const size_t elems = (size_t)batch * hq * (size_t)max_q * (size_t)l;
    *ldx = l;
    *a_off = (elems * sizeof(float) + 255) / 256 * 256;
    *total = *a_off + elems * 2;
    return true;
}

}  // namespace

ATTN_API size_t attn_unfused_workspace_bytes(int batch, int num_q_heads, int max_seqlen_q,
                                             int max_seqlen_k) {
    int64_t ldx;
    size_t a_off, total;
    if (!unfused_layout(batch, num_q_heads, max_seqlen_q, max_seqlen_k, &ldx, &a_off, &total)) return 0;
    return total;
}

ATTN_API int attn_prefill_unfused(const void *q, const void *k, const void *v, void *o,
                                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                  int batch, int max_seqlen_q, int max_seqlen_k,
                                  int total_q, int total_k, int num_q_heads, int num_kv_heads,
                                  int head_dim, float softmax_scale, int causal, int in_dtype,
                                  int out_dtype, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL;
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seqlen_q < 0 ||
        max_seqlen_k < 0 || total_q < 0 || total_k < 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (!scale_ok(softmax_scale)) return ATTN_ERR_SHAPE;
    if (in_dtype != ATTN_BF16 || head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)batch * num_q_heads > 65535) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
    int64_t ldx;
    size_t a_off, total;
    if (!unfused_layout(batch, num_q_heads, max_seqlen_q, max_seqlen_k, &ldx, &a_off, &total))
        return ATTN_ERR_SHAPE;
    if (!workspace || workspace_bytes < total) return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_WORKSPACE;
    if (total_q == 0) return ATTN_OK;

    attn::UnfusedArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.batch = batch; a.max_seqlen_q = max_seqlen_q; a.max_seqlen_k = max_seqlen_k;
    a.total_q = total_q; a.total_k = total_k;
    a.hq = num_q_heads; a.hkv = num_kv_heads;
    a.scale = softmax_scale;
    a.causal = causal ? 1 : 0;
    a.x = reinterpret_cast<float *>(workspace);
    a.a = reinterpret_cast<char *>(workspace) + a_off;
    a.ldx = ldx;
    a.out_f32 = out_dtype == ATTN_F32;
    return hip_status(attn::launch_unfused(a, (hipStream_t)stream));
}
