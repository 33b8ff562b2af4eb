// launch.h -- host-side launchers of the gfx950 kernels (internal to
// libattn.so; the public surface is include/attn.h).  Arguments have already
// been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

hipError_t launch_kv_store(const void *k, const void *v, void *k_cache, void *v_cache,
                           const int32_t *slot_mapping, int num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream);

// Sequence metadata and K/V addressing shared by the prefill kernels.
struct VarlenArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    const int32_t *cu_q;
    const int32_t *cu_k;
    const int32_t *block_table;  // NULL: contiguous K/V
    int batch;
    int max_seqlen_q;
    int64_t total_q;
    int64_t total_k;
    int hq;
    int hkv;
    int d;
    float scale_log2;  // softmax_scale * log2(e)
    int causal;
    int max_blocks_per_seq;
    int num_blocks;
    int block_size;
    int out_f32;  // 1: fp32 output, 0: bf16 output
};

hipError_t launch_prefill_f32(const VarlenArgs &a, hipStream_t stream);
hipError_t launch_prefill_bf16(const VarlenArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    void *o;
    const int32_t *cache_seqlens;
    const int32_t *block_table;
    int batch;
    int hq;
    int hkv;
    int d;
    int max_blocks_per_seq;
    int num_blocks;
    int block_size;
    float scale_log2;
    int split_tokens;  // resolved, > 0, multiple of 64
    int max_splits;    // ceil(max_blocks_per_seq * block_size / split_tokens)
    float *ws_o;       // [batch, hq, max_splits, d]
    float *ws_ml;      // [batch, hq, max_splits, 4]: m, d', split count (int bits), pad
    int out_f32;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace attn
