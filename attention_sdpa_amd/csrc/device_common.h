// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define ATTN_LDS __attribute__((address_space(3)))
#define ATTN_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// 2^x with the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }

// ---- the two 16-bit input types (bf16, fp16) ---------------------------
// Vectors of a 16-bit element type, and the matrix-core instructions and
// conversions that go with it.  Data move as raw 16-bit values (LDS copies,
// transposing LDS reads), so only arithmetic needs the type.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x2 x2; typedef bf16x4 x4; typedef bf16x8 x8; };
template <> struct Vec16<f16> { typedef f16x2 x2; typedef f16x4 x4; typedef f16x8 x8; };

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// c + a.x * b.x + a.y * b.y with fp32 accumulation (v_dot2_f32_*)
__device__ __forceinline__ float dot2_acc(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ float dot2_acc(f16x2 a, f16x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}
// Round-to-nearest-even float -> T.
template <typename T>
__device__ __forceinline__ T to16(float x) { return (T)x; }

// Transposing LDS read of 4 16-bit values (ds_read_b64_tr_b16), as T.
template <typename T>
__device__ __forceinline__ typename Vec16<T>::x4 ds_read_tr4(const void *p) {
    const bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)(p));
    return __builtin_bit_cast(typename Vec16<T>::x4, r);
}

// Value held by lane (lane ^ 32): exchanges the two 32-lane halves.
__device__ __forceinline__ float swap_halves(float x) {
    return __shfl_xor(x, 32, 64);
}

// Read-only int32 metadata (block tables, sequence offsets): read through the
// constant address space so that uniform indices become scalar loads, which
// do not wait behind outstanding vector-memory loads.
__device__ __forceinline__ int32_t ld_meta(const int32_t *p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)(p))[i];
}

// Direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4 with
// a scalar base address and a per-lane 32-bit offset): lane l's 16 bytes at
// sbase + voff land at LDS byte address lds + 16*l.  Issued from inline
// assembly so that the compiler, which cannot tell which LDS buffer a later
// LDS read touches, does not wait for every such load before every read;
// the kernels order them themselves (s_waitcnt vmcnt, plus s_barrier where
// several waves share a buffer).  M0 carries the LDS address and is
// restored afterwards.
__device__ __forceinline__ void lds_dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}

// Four such loads into consecutive LDS blocks of STEP bytes (lds, lds +
// STEP, ...), lane offsets o0..o3 from one scalar base, with M0 saved and
// restored once for the four.
template <int STEP>
__device__ __forceinline__ void lds_dma16x4(const void *sbase, uint32_t o0, uint32_t o1, uint32_t o2,
                                            uint32_t o3, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "s_add_u32 m0, m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "s_add_u32 m0, m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %6\n\t"
        "s_add_u32 m0, m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(lds), "s"(sbase), "i"(STEP)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const ATTN_LDS void *)p;
}

// 16-byte global load/store helpers.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace attn
