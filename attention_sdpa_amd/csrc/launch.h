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
    int max_seqlen_k;  // bound of the key counts (only orders the unit schedule)
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
    int out_f32;  // 1: fp32 output, 0: output in the 16-bit input type
    int in_f16;   // 16-bit inputs: 1 fp16, 0 bf16
    // Padded batches: pad_q > 0 places sequence b's queries at rows
    // b * pad_q .. with seqlens_q[b] of them, and its keys at rows
    // b * pad_k .. with min(seqlens_k[b], pad_k) of them (cu_q, cu_k and
    // block_table unused).  pad_q == 0: the varlen layout of cu_q / cu_k.
    const int32_t *seqlens_q;
    const int32_t *seqlens_k;
    int pad_q;
    int pad_k;
};

hipError_t launch_prefill_f32(const VarlenArgs &a, hipStream_t stream);
// bf16 or fp16 inputs (VarlenArgs::in_f16) on the matrix cores
hipError_t launch_prefill_mfma(const VarlenArgs &a, hipStream_t stream);

// Persistent decode runs (one workgroup per CU and head block) are at most
// this many; the workspace holds kDecodeMaxRuns + batch partial slots.
constexpr int kDecodeMaxRuns = 1024;

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
    int split_tokens;  // keys per item, resolved, > 0, multiple of 32
    int n_runs;        // runs the item stream is cut into, <= kDecodeMaxRuns
    float *ws_o;       // [n_runs + batch slots, hq, d]
    float *ws_ml;      // [n_runs + batch slots, hq, 2]: m (log2-scaled), d'
    int32_t *ws_runs;  // [batch, 2]: runs holding each sequence's first and last item
    int out_f32;       // 1: fp32 output, 0: output in the input type
    int in_f16;        // 1: fp16 inputs, 0: bf16
};

// Runs of a decode launch on a device with `cus` compute units.
int decode_runs(int hkv, int cus);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// Size of the per-device scratch array behind the allocation-free decode
// entry point, and its device address on the current device (resolved once
// per device by symbol lookup, then cached).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void **ptr);

// The unfused three-step baseline (logits, softmax and A V as separate
// kernels with X and A in the workspace).
struct UnfusedArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    const int32_t *cu_q;
    const int32_t *cu_k;
    int batch;
    int max_seqlen_q;
    int max_seqlen_k;
    int total_q;
    int total_k;
    int hq;
    int hkv;
    float scale;       // softmax_scale
    int causal;
    float *x;          // [batch, hq, max_seqlen_q, ldx] fp32 logits
    void *a;           // [batch, hq, max_seqlen_q, ldx] bf16 probabilities
    int64_t ldx;       // max_seqlen_k rounded up to 64
    int out_f32;
};

hipError_t launch_unfused(const UnfusedArgs &a, hipStream_t stream);

}  // namespace attn
