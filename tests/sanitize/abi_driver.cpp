// Drives the host-side validation of the C ABI (attention_sdpa_amd/csrc/
// attn_abi.cpp, compiled into this program) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU: every call below has an invalid
// argument, so each must return its documented status before any launch.
// The kernel launchers are replaced by stubs that abort, which proves that
// no invalid call reaches them.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include <hip/hip_runtime.h>

#include "attn.h"
#include "launch.h"

namespace attn {
hipError_t launch_kv_store(const void *, const void *, void *, void *, const int32_t *, int, int, int64_t,
                           hipStream_t) { std::abort(); }
hipError_t launch_prefill_f32(const VarlenArgs &, hipStream_t) { std::abort(); }
hipError_t launch_prefill_mfma(const VarlenArgs &, hipStream_t) { std::abort(); }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { std::abort(); }
hipError_t launch_unfused(const UnfusedArgs &, hipStream_t) { std::abort(); }
int decode_runs(int, int) { std::abort(); }
hipError_t decode_scratch(void **) { std::abort(); }
int decode_head_blocks(int hkv) { return (hkv + 7) / 8; }
}  // namespace attn

static int fails = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        std::printf("%s: status %d, expected %d\n", what, got, want);
        ++fails;
    }
}

int main() {
    void *P = reinterpret_cast<void *>(0x100000);
    void *MIS = reinterpret_cast<void *>(0x100008);
    const int32_t *I = reinterpret_cast<const int32_t *>(0x200000);
    expect(kv_store_slots(nullptr, P, P, P, I, 4, 8, 128, 16, 64, ATTN_BF16, nullptr), ATTN_ERR_NULL, "kv null");
    expect(kv_store_slots(P, P, P, P, I, 4, 8, 128, 16, 64, 7, nullptr), ATTN_ERR_UNSUPPORTED, "kv dtype");
    expect(kv_store_slots(P, P, MIS, P, I, 4, 8, 128, 16, 64, ATTN_BF16, nullptr), ATTN_ERR_UNSUPPORTED, "kv align");
    expect(attn_prefill_varlen(P, P, P, P, nullptr, I, 2, 16, 16, 20, 20, 32, 8, 128, 0.1f, 1, nullptr, 0, 0, 0,
                               ATTN_BF16, ATTN_F32, nullptr), ATTN_ERR_NULL, "prefill null");
    expect(attn_prefill_varlen(P, P, P, P, I, I, 2, 16, 16, 20, 20, 12, 8, 128, 0.1f, 1, nullptr, 0, 0, 0,
                               ATTN_BF16, ATTN_F32, nullptr), ATTN_ERR_SHAPE, "prefill groups");
    expect(attn_prefill_varlen(P, P, P, P, I, I, 2, 16, 16, 20, 20, 32, 8, 64, 0.1f, 1, nullptr, 0, 0, 0,
                               ATTN_BF16, ATTN_F32, nullptr), ATTN_ERR_UNSUPPORTED, "prefill head_dim");
    expect(attn_prefill_varlen(P, P, P, P, I, I, 2, 16, 16, 20, 20, 32, 8, 128, -1.f, 1, nullptr, 0, 0, 0,
                               ATTN_F16, ATTN_F32, nullptr), ATTN_ERR_SHAPE, "prefill scale");
    expect(attn_prefill_varlen(P, P, P, P, I, I, 2, 16, 16, 20, 20, 32, 8, 128, 0.1f, 1, I, 4, 10, 96,
                               ATTN_BF16, ATTN_F32, nullptr), ATTN_ERR_UNSUPPORTED, "prefill block size");
    expect(attn_prefill_padded(P, P, P, P, I, I, 1 << 20, 1 << 12, 16, 32, 8, 128, 0.1f, 1, ATTN_BF16, ATTN_F32,
                               nullptr), ATTN_ERR_SHAPE, "padded rows");
    expect(attn_prefill_padded(P, P, P, P, I, I, 2, 16, 16, 32, 8, 128, 0.1f, 1, ATTN_F16, ATTN_BF16, nullptr),
           ATTN_ERR_UNSUPPORTED, "padded dtype pair");
    const size_t need = attn_decode_workspace_bytes(4, 32, 8, 128, 32, 256, 0);
    if (need == 0) ++fails;
    expect(attn_decode_paged(P, P, P, P, I, I, 4, 32, 8, 128, 32, 200, 256, 0.1f, 0, ATTN_BF16, ATTN_F32, P,
                             need - 1, nullptr), ATTN_ERR_WORKSPACE, "decode workspace");
    expect(attn_decode_paged(P, P, P, P, I, I, 4, 32, 8, 128, 32, 200, 256, 0.1f, 48, ATTN_BF16, ATTN_F32, P,
                             need, nullptr), ATTN_ERR_UNSUPPORTED, "decode split");
    expect(attn_decode_paged(P, P, P, P, I, I, 4, 64, 2, 128, 32, 200, 256, 0.1f, 0, ATTN_BF16, ATTN_F32, P,
                             need, nullptr), ATTN_ERR_UNSUPPORTED, "decode group");
    expect(attn_decode_paged_noalloc(P, P, P, P, I, I, 2015, 32, 8, 128, 32, 200, 256, 0.1f, 0, ATTN_BF16,
                                     ATTN_F32, nullptr), ATTN_ERR_WORKSPACE, "decode noalloc beyond scratch");
    expect(attn_decode_paged_noalloc(P, P, P, P, I, I, 4, 32, 8, 128, 32, 200, 256, 0.f, 0, ATTN_BF16,
                                     ATTN_F32, nullptr), ATTN_ERR_SHAPE, "decode noalloc scale");
    const size_t uneed = attn_unfused_workspace_bytes(2, 32, 16, 16);
    expect(attn_prefill_unfused(P, P, P, P, I, I, 2, 16, 16, 20, 20, 32, 8, 128, 0.1f, 1, ATTN_BF16, ATTN_F32, P,
                                uneed - 1, nullptr), ATTN_ERR_WORKSPACE, "unfused workspace");
    expect(attn_prefill_unfused(P, P, P, P, I, I, 2, 16, 16, 20, 20, 32, 8, 128, 0.1f, 1, ATTN_F16, ATTN_F32, P,
                                uneed, nullptr), ATTN_ERR_UNSUPPORTED, "unfused dtype");
    for (int s = -1; s < 8; ++s)
        if (!attn_status_str(s)) ++fails;
    std::printf(fails ? "FAIL %d\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
