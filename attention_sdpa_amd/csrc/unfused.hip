// unfused.hip -- the standard, unfused attention of the blog post "从零实现
// vLLM (1.3)：如何加速 Attention 计算" (section 标准实现方法), as a baseline for
// the fused kernels: three kernels with the logits X and the probabilities A
// stored in HBM between them.
//
//   1. X = s * Q K^T       (logits_kernel: MFMA, X written as fp32)
//   2. A = softmax(X)      (softmax_kernel: per row, 3-pass safe softmax of
//                           section 计算流程: max, then sum of exponentials,
//                           then the normalised weights, A written as bf16;
//                           the causal mask is applied here)
//   3. O = A V             (av_kernel: MFMA over the stored A)
//
// The section's point is that steps 1 and 2 each write an Lq x Lk matrix
// that the next step reads back: this file exists to measure that traffic
// on this GPU next to the one-pass kernel.  X and A are computed for every
// (query, key) pair of each sequence, as the standard method does; only the
// softmax skips masked keys.
//
// Layout of the workspace: X [batch, hq, max_seqlen_q, ldx] fp32, then A
// [batch, hq, max_seqlen_q, ldx] bf16, ldx = max_seqlen_k rounded up to 64,
// plus 64 so that rows are not a power of two apart.
// Each sequence uses the leading Lq x Lk corner of its slices (A rows are
// zero-filled up to the next multiple of 64 keys so that step 3 reads whole
// 64-key tiles).
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16, 64 lanes, n = lane & 31,
// hf = lane >> 5): the A operand lane holds row n, k = 8hf .. 8hf+7; the B
// operand lane holds column n, k = 8hf .. 8hf+7; accumulator register
// 4j + t holds row 8j + 4hf + t, column n.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kUD = 128;     // head_dim
constexpr int kUT = 64;      // tile edge (queries and keys)

__device__ __forceinline__ void seq_bounds(const UnfusedArgs &a, int b, int &q0, int &Lq, int &k0, int &Lk) {
    int x0 = ld_meta(a.cu_q, b), x1 = ld_meta(a.cu_q, b + 1);
    x0 = x0 < 0 ? 0 : (x0 > a.total_q ? a.total_q : x0);
    x1 = x1 < x0 ? x0 : (x1 > a.total_q ? a.total_q : x1);
    q0 = x0;
    Lq = min(x1 - x0, a.max_seqlen_q);
    int y0 = ld_meta(a.cu_k, b), y1 = ld_meta(a.cu_k, b + 1);
    y0 = y0 < 0 ? 0 : (y0 > a.total_k ? a.total_k : y0);
    y1 = y1 < y0 ? y0 : (y1 > a.total_k ? a.total_k : y1);
    k0 = y0;
    Lk = min(y1 - y0, a.max_seqlen_k);
}

// Step 1: a 64-query x 256-key strip of X per workgroup; wave w takes
// queries 32 (w & 1) .. and keys 128 (w >> 1) .. in four 32-key blocks.
// The product is formed transposed, X^T = K Q^T (keys as M), so that each
// lane holds 4 consecutive keys of one query and stores them as 16 bytes.
// Q and K operands are loaded into registers from global memory up front.
constexpr int kStrip = 256;

__global__ void __launch_bounds__(256) logits_kernel(UnfusedArgs a) {
    // per wave, one 32 x 32 block of X staged for whole-line stores
    __shared__ __align__(16) float sX[4][32][32 + 4];
    const int bh = blockIdx.z, b = bh / a.hq, h = bh % a.hq;
    int q0, Lq, k0, Lk;
    seq_bounds(a, b, q0, Lq, k0, Lk);
    const int i0 = blockIdx.x * kUT, j0 = blockIdx.y * kStrip;
    if (i0 >= Lq || j0 >= Lk) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int g = h / (a.hq / a.hkv);
    const int wi = i0 + 32 * (w & 1), wj = j0 + 128 * (w >> 1);
    if (wj >= Lk) return;
    const int qi = min(wi + n, Lq - 1);   // clamped rows stay in bounds
    const bf16 *qp = (const bf16 *)a.q + ((int64_t)(q0 + qi) * a.hq + h) * kUD + 8 * hf;
    uint4 qf[kUD / 16];
#pragma unroll
    for (int kk = 0; kk < kUD / 16; ++kk) qf[kk] = ld16(qp + 16 * kk);
    // all four 32-key blocks' K operands are loaded up front (rows past Lk
    // are clamped; their keys are not stored)
    uint4 kf[4][kUD / 16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int kj = min(wj + 32 * kb + n, Lk - 1);
        const bf16 *kp = (const bf16 *)a.k + ((int64_t)(k0 + kj) * a.hkv + g) * kUD + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < kUD / 16; ++kk) kf[kb][kk] = ld16(kp + 16 * kk);
    }
    float *X = a.x + ((int64_t)bh * a.max_seqlen_q) * a.ldx;
    // store lanes: 8 lanes per query row, 16 bytes (4 keys) each
    const int sr = lane >> 3, sc = 4 * (lane & 7);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int kj0 = wj + 32 * kb;
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < kUD / 16; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<bf16x8 *>(&kf[kb][kk]),
                                                          *reinterpret_cast<bf16x8 *>(&qf[kk]), acc, 0, 0, 0);
        if (kj0 >= Lk) continue;
        // lane holds query n, keys 8jb + 4hf + t: to LDS as [query][key]
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            *reinterpret_cast<float4 *>(&sX[w][n][8 * jb + 4 * hf]) =
                make_float4(acc[4 * jb] * a.scale, acc[4 * jb + 1] * a.scale,
                            acc[4 * jb + 2] * a.scale, acc[4 * jb + 3] * a.scale);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the block is in LDS
        __builtin_amdgcn_wave_barrier();
        // 8 whole 128-byte rows per store instruction (keys >= Lk: padding)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = 8 * p + sr, i = wi + r;
            const float4 v = *reinterpret_cast<const float4 *>(&sX[w][r][sc]);
            if (i < Lq) *reinterpret_cast<float4 *>(X + (int64_t)i * a.ldx + kj0 + sc) = v;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next block lands
        __builtin_amdgcn_wave_barrier();
    }
}

// Step 2: one wavefront per row of X; 3-pass safe softmax over the visible
// keys [0, J), A written as bf16 (zeros for masked keys and up to the next
// multiple of 64 keys).  Lane l reads keys 4l + 256u .. +3 as 16 bytes.
// Rows of up to 4096 keys are read once and kept in registers for the
// three passes; longer rows are read once per pass.
constexpr int kRegChunks = 16;           // 16 x 256 keys

__global__ void __launch_bounds__(256) softmax_kernel(UnfusedArgs a) {
    const int bh = blockIdx.y, b = bh / a.hq;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    int q0, Lq, k0, Lk;
    seq_bounds(a, b, q0, Lq, k0, Lk);
    if (i >= Lq) return;
    const int J = a.causal ? max(0, min(Lk, i + (Lk - Lq) + 1)) : Lk;   // visible keys [0, J)
    const int64_t row = ((int64_t)bh * a.max_seqlen_q + i) * a.ldx;
    const float *x = a.x + row;
    bf16 *A = (bf16 *)a.a + row;
    const int Jpad = (Lk + kUT - 1) / kUT * kUT;
    auto ld4 = [&](int j) ATTN_INLINE {          // keys j .. j+3, masked past J
        float4 v = *reinterpret_cast<const float4 *>(x + j);
        if (j + 3 >= J) {
            v.x = j < J ? v.x : kNegInf;
            v.y = j + 1 < J ? v.y : kNegInf;
            v.z = j + 2 < J ? v.z : kNegInf;
            v.w = j + 3 < J ? v.w : kNegInf;
        }
        return v;
    };
    auto st4 = [&](int j, float4 p) ATTN_INLINE {
        bf16x4 o4 = {f32_to_bf16(p.x), f32_to_bf16(p.y), f32_to_bf16(p.z), f32_to_bf16(p.w)};
        *reinterpret_cast<bf16x4 *>(A + j) = o4;
    };
    float m = kNegInf, l = 0.f;
    if (Jpad <= kRegChunks * 256) {
        float4 xr[kRegChunks];
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const int j = 4 * lane + 256 * u;
            xr[u] = j < J ? ld4(j) : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
            m = fmaxf(m, fmaxf(fmaxf(xr[u].x, xr[u].y), fmaxf(xr[u].z, xr[u].w)));
        }
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const float mc = J > 0 ? m : 0.f;
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            xr[u].x = fast_exp2((xr[u].x - mc) * kLog2e);
            xr[u].y = fast_exp2((xr[u].y - mc) * kLog2e);
            xr[u].z = fast_exp2((xr[u].z - mc) * kLog2e);
            xr[u].w = fast_exp2((xr[u].w - mc) * kLog2e);
            l += (xr[u].x + xr[u].y) + (xr[u].z + xr[u].w);
        }
        for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
        const float inv = J > 0 ? 1.f / l : 0.f;
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const int j = 4 * lane + 256 * u;
            if (j < Jpad) st4(j, make_float4(xr[u].x * inv, xr[u].y * inv, xr[u].z * inv, xr[u].w * inv));
        }
        return;
    }
    for (int j = 4 * lane; j < J; j += 256) {
        const float4 v = ld4(j);
        m = fmaxf(m, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float mc = J > 0 ? m : 0.f;
    for (int j = 4 * lane; j < J; j += 256) {
        const float4 v = ld4(j);
        l += (fast_exp2((v.x - mc) * kLog2e) + fast_exp2((v.y - mc) * kLog2e)) +
             (fast_exp2((v.z - mc) * kLog2e) + fast_exp2((v.w - mc) * kLog2e));
    }
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
    const float inv = J > 0 ? 1.f / l : 0.f;
    for (int j = 4 * lane; j < Jpad; j += 256) {
        float4 v = j < J ? ld4(j) : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        st4(j, make_float4(fast_exp2((v.x - mc) * kLog2e) * inv, fast_exp2((v.y - mc) * kLog2e) * inv,
                           fast_exp2((v.z - mc) * kLog2e) * inv, fast_exp2((v.w - mc) * kLog2e) * inv));
    }
}

// Step 3: O rows [i0, i0 + 64) x 128 of one (sequence, head) per workgroup;
// wave w takes rows 32 (w & 1) .. and d 64 (w >> 1) .. (two 32-column
// blocks).  A operands come from global memory; each 64-key V tile is
// staged in LDS and read transposed (ds_read_b64_tr_b16).
__global__ void __launch_bounds__(256) av_kernel(UnfusedArgs a) {
    __shared__ __align__(16) bf16 sV[kUT * kUD];
    const int bh = blockIdx.y, b = bh / a.hq, h = bh % a.hq;
    int q0, Lq, k0, Lk;
    seq_bounds(a, b, q0, Lq, k0, Lk);
    const int i0 = blockIdx.x * kUT;
    if (i0 >= Lq) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hf = lane >> 5;
    const int g = h / (a.hq / a.hkv);
    const int wi = i0 + 32 * (w & 1), wd = 64 * (w >> 1);
    const int ai = min(wi + n, Lq - 1);
    const bf16 *Ap = (const bf16 *)a.a + ((int64_t)bh * a.max_seqlen_q + ai) * a.ldx + 8 * hf;
    const int G = lane >> 4, s = lane & 15;   // 16-lane group, lane in group
    f32x16 acc[2] = {};
    const int nt = (Lk + kUT - 1) / kUT;
    for (int t = 0; t < nt; ++t) {
        __syncthreads();   // the previous tile is no longer read
        // V tile rows t*64 .. +63 -> LDS (rows past Lk repeat the last key;
        // their weights in A are zero)
#pragma unroll
        for (int c = 0; c < kUT * kUD / 8 / 256; ++c) {
            const int e = tid + 256 * c;
            const int r = e >> 4, ch = e & 15;
            const int kj = min(t * kUT + r, Lk - 1);
            const uint4 v = ld16((const bf16 *)a.v + ((int64_t)(k0 + kj) * a.hkv + g) * kUD + 8 * ch);
            *reinterpret_cast<uint4 *>(&sV[r * kUD + 8 * ch]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kUT / 16; ++ks) {
            uint4 av = ld16(Ap + t * kUT + 16 * ks);
            const bf16x8 af = *reinterpret_cast<bf16x8 *>(&av);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                // B operand: lane (n, hf) needs V[key 16ks + 8hf + e][d = wd + 32db + n];
                // source lane s of 16-lane group G reads 4 consecutive d of
                // key 16ks + 8(G >> 1) + (s >> 2) (+4 for the second half)
                const int key = 16 * ks + 8 * (G >> 1) + (s >> 2);
                const int d = wd + 32 * db + 16 * (G & 1) + 4 * (s & 3);
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)&sV[key * kUD + d]);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)&sV[(key + 4) * kUD + d]);
                const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, vf, acc[db], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = wi + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (i >= Lq) continue;
            const int64_t idx = ((int64_t)(q0 + i) * a.hq + h) * kUD + wd + 32 * db + n;
            if (a.out_f32) ((float *)a.o)[idx] = acc[db][r];
            else ((bf16 *)a.o)[idx] = f32_to_bf16(acc[db][r]);
        }
}

}  // namespace

hipError_t launch_unfused(const UnfusedArgs &a, hipStream_t stream) {
    if (a.batch == 0 || a.max_seqlen_q == 0) return hipSuccess;
    const unsigned bh = (unsigned)(a.batch * a.hq);
    const unsigned qt = (unsigned)((a.max_seqlen_q + kUT - 1) / kUT);
    const unsigned kt = (unsigned)((a.max_seqlen_k + kStrip - 1) / kStrip);
    if (kt > 0) {
        hipLaunchKernelGGL(logits_kernel, dim3(qt, kt, bh), dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(softmax_kernel, dim3((unsigned)((a.max_seqlen_q + 3) / 4), bh), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(av_kernel, dim3(qt, bh), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
