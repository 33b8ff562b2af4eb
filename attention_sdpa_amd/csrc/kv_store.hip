// kv_store.hip -- the store_kvcache scatter (blog post "从零实现 vLLM (1.3)：
// 如何加速 Attention 计算", section Attention 源码分析): every new token's K and
// V rows go to cache slot slot_mapping[t] = block_id * block_size + offset.
//
// The cache is [num_blocks, block_size, Hkv, d], so one slot is one
// contiguous row of Hkv * d elements.  Each thread moves one 16-byte chunk of
// K and the matching chunk of V; consecutive threads cover consecutive
// chunks of a row, so reads and writes are fully coalesced.  Pure data
// movement: HBM-bound, bit-exact.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

__global__ void __launch_bounds__(256)
kv_store_kernel(const uint4 *__restrict__ k, const uint4 *__restrict__ v,
                uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
                const int32_t *__restrict__ slot_mapping, int64_t total_chunks,
                int row_chunks, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_chunks) return;
    const int64_t t = i / row_chunks;
    const int c = (int)(i - t * row_chunks);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;  // padding token / out-of-range slot
    const int64_t dst = slot * row_chunks + c;
    const uint4 kv = k[i];
    const uint4 vv = v[i];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
}

}  // namespace

hipError_t launch_kv_store(const void *k, const void *v, void *k_cache, void *v_cache,
                           const int32_t *slot_mapping, int num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream) {
    const int row_chunks = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * row_chunks;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4 *)k, (const uint4 *)v, (uint4 *)k_cache, (uint4 *)v_cache,
                       slot_mapping, total, row_chunks, num_slots);
    return hipGetLastError();
}

}  // namespace attn
