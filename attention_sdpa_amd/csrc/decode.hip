// decode.hip -- single-token decode against a paged KV cache, split over
// the key range, plus the pass that merges the splits.
//
// What is computed is the Decode section of the blog post "从零实现 vLLM
// (1.3)：如何加速 Attention 计算": one new query per sequence attends to every
// cached token, reading K/V blocks through the block table (the page-table
// analogy of its Prefill section).  The key range of each (sequence, KV head)
// is cut into splits; every split runs the online-softmax recurrence of
// section FlashAttention 的最终实现 over its keys and leaves a partial state
// (m, d', o' unnormalised).  Because the tile updates are associative (section
// 计算流程(1-Pass 算法与分块)), the combine kernel merges the partials with the
// same rescaling: M = max m_s, d' = sum d'_s 2^(m_s - M), o = sum o'_s
// 2^(m_s - M) / d'.
//
// Decode reads every K/V byte once and does ~4 flops per byte, so it is
// HBM-bound.  Design for that on CDNA4:
// * one workgroup = (sequence, KV head, split); its GQA group's query heads
//   share every K/V byte it reads;
// * 4 wavefronts per workgroup take 64-key chunks of the split round-robin,
//   each with its own running state, and merge through LDS at the end;
// * K rows go from global memory straight into registers as the A operand of
//   S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys = M, query heads = N);
// * V rows go through a per-wavefront LDS buffer and come back transposed
//   (ds_read_b64_tr_b16) as the A operand of O^T += V^T P^T;
// * all loads of a chunk are 16 bytes wide and issued together.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kChunk = 64;  // keys per wavefront step

__device__ __forceinline__ int swz_dv(int row) { return (row & 7) << 1; }

template <int D>
__global__ void __launch_bounds__(kDecThreads, 2)
decode_split_kernel(DecodeArgs a) {
    constexpr int KK = D / 32;          // k-steps of 32 over head_dim
    constexpr int DB = D / 16;          // 16-row blocks of d in O^T
    constexpr int VL = kChunk * D / 8 / 64;  // 16-byte V loads per lane per chunk
    __shared__ __align__(16) bf16 sV[kDecWaves][kChunk * D];
    __shared__ float sMerge[kDecWaves][16][2];

    int id = blockIdx.x;
    const int g = id % a.hkv;
    id /= a.hkv;
    const int s = id % a.max_splits;
    const int b = id / a.max_splits;

    int L = ld_meta(a.cache_seqlens, b);
    const int cap = a.max_blocks_per_seq * a.block_size;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int kbeg = s * a.split_tokens;
    if (kbeg >= L) return;
    const int kend = min(L, kbeg + a.split_tokens);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = a.hq / a.hkv;
    const int n = lane & 15;            // query column of this lane (head g*group + n)
    const int gq = lane >> 4;           // lane group 0..3
    const bool qv = n < group;
    const int head = g * group + (qv ? n : 0);

    // Q^T operand: B[k = d][n = head], lane group gq holds d in [32gq, 32gq+32)
    bf16x8 qf[KK];
    {
        const bf16 *qp = (const bf16 *)a.q + ((int64_t)b * a.hq + head) * D + 32 * gq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 t = qv ? ld16(qp + 8 * kk) : make_uint4(0, 0, 0, 0);
            qf[kk] = *reinterpret_cast<bf16x8 *>(&t);
        }
    }
    f32x4 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x4{};
    float m_run = kNegInf, mc_run = 0.f, l_run = 0.f;
    const float cl = a.scale_log2;
    bf16 *vbuf = sV[w];

    for (int c0 = kbeg + w * kChunk; c0 < kend; c0 += kDecWaves * kChunk) {
        const int blk = ld_meta(a.block_table, (int64_t)b * a.max_blocks_per_seq + c0 / a.block_size);
        const bool bok = blk >= 0 && blk < a.num_blocks;
        const int64_t base = bok ? ((((int64_t)blk * a.block_size + c0 % a.block_size) * a.hkv + g) * D) : 0;
        const int64_t rstride = (int64_t)a.hkv * D;
        // K: 4 row-blocks of 16 keys; lane holds key (16mb + n), d in [32gq, +32)
        uint4 kr[4][KK];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int key = c0 + 16 * mb + n;
            const bool ok = bok && key < kend;
            const bf16 *kp = (const bf16 *)a.k_cache + base + (int64_t)(16 * mb + n) * rstride + 32 * gq;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) kr[mb][kk] = ok ? ld16(kp + 8 * kk) : make_uint4(0, 0, 0, 0);
        }
        // V: row (4i + gq), chunk n -- row-wise coalesced
        uint4 vr[VL];
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int row = 4 * i + gq;
            const bool ok = bok && c0 + row < kend;
            vr[i] = ok ? ld16((const bf16 *)a.v_cache + base + (int64_t)row * rstride + 8 * n)
                       : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int row = 4 * i + gq;
            st16(vbuf + row * D + ((n ^ swz_dv(row)) * 8), vr[i]);
        }
        // S^T = K Q^T
        f32x4 sacc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            sacc[mb] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    *reinterpret_cast<bf16x8 *>(&kr[mb][kk]), qf[kk], sacc[mb], 0, 0, 0);
        }
        // mask keys past the split end: lane holds keys 16mb + 4gq + i
        if (c0 + kChunk > kend) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (c0 + 16 * mb + 4 * gq + i >= kend) sacc[mb][i] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[mb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float mc_new = (m_new == kNegInf) ? 0.f : m_new * cl;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(mc_run - mc_new);
        float psum = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(fmaf(sacc[mb][i], cl, -mc_new));
                psum += p;
                pb[mb >> 1][4 * (mb & 1) + i] = f32_to_bf16(p);
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        mc_run = mc_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        // the V tile written above must be complete before the transposing reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // O^T += V^T P^T: K = 32 keys per step (keys 32jj + 4gq + e, +16)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int r0 = 32 * jj + 4 * gq + (n >> 2);
                const int col = 16 * db + 4 * (n & 3);
                const int ch = col >> 3, sub = col & 7;
                const bf16 *p0 = vbuf + r0 * D + ((ch ^ swz_dv(r0)) * 8) + sub;
                const bf16 *p1 = vbuf + (r0 + 16) * D + ((ch ^ swz_dv(r0 + 16)) * 8) + sub;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)p0);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)p1);
                const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[jj], o[db], 0, 0, 0);
            }
        }
        // reads of vbuf must finish before the next chunk overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the 4 wavefronts' states through LDS ----
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    const float mlog = (m_run == kNegInf) ? kNegInf : mc_run;  // log2-scaled max or -inf
    if (gq == 0) {
        sMerge[w][n][0] = mlog;
        sMerge[w][n][1] = l_run;
    }
    __syncthreads();  // every wave is done with its V buffer and has posted m, l
    float *sO = reinterpret_cast<float *>(&sV[0][0]);  // [waves][16][D] floats (reuse)
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, sMerge[ww][n][0]);
    const float myscale = (mlog == kNegInf) ? 0.f : fast_exp2(mlog - M);
    __syncthreads();
    // O^T layout: lane holds query n, d = 16db + 4gq + i
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sO[(w * 16 + n) * D + 16 * db + 4 * gq + i] = o[db][i] * myscale;
    __syncthreads();
    // threads (query qi, d) sum the 4 waves and write the partial
    for (int e = tid; e < group * D; e += kDecThreads) {
        const int qi = e / D, d = e % D;
        float Mq = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) Mq = fmaxf(Mq, sMerge[ww][qi][0]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            acc += sO[(ww * 16 + qi) * D + d];
            const float mw = sMerge[ww][qi][0];
            lsum += (mw == kNegInf) ? 0.f : sMerge[ww][qi][1] * fast_exp2(mw - Mq);
        }
        const int64_t row = ((int64_t)b * a.hq + g * group + qi) * a.max_splits + s;
        a.ws_o[row * D + d] = acc;
        if (d == 0) {
            a.ws_ml[row * 2] = Mq;
            a.ws_ml[row * 2 + 1] = lsum;
        }
    }
}

template <int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(DecodeArgs a) {
    const int bh = blockIdx.x;  // b * hq + h
    const int b = bh / a.hq;
    const int d = threadIdx.x;
    int L = ld_meta(a.cache_seqlens, b);
    const int cap = a.max_blocks_per_seq * a.block_size;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int ns = (L + a.split_tokens - 1) / a.split_tokens;
    const int64_t row0 = (int64_t)bh * a.max_splits;
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_ml[(row0 + s) * 2]);
    float acc = 0.f, lsum = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float ms = a.ws_ml[(row0 + s) * 2];
        if (ms == kNegInf) continue;
        const float f = fast_exp2(ms - M);
        lsum += a.ws_ml[(row0 + s) * 2 + 1] * f;
        acc += a.ws_o[(row0 + s) * D + d] * f;
    }
    const float r = lsum > 0.f ? acc / lsum : 0.f;
    if (a.out_f32)
        ((float *)a.o)[(int64_t)bh * D + d] = r;
    else
        ((bf16 *)a.o)[(int64_t)bh * D + d] = f32_to_bf16(r);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    constexpr int D = 128;
    const int64_t units = (int64_t)a.batch * a.max_splits * a.hkv;
    if (a.batch == 0) return hipSuccess;
    if (units > 0)
        hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)units), dim3(kDecThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(a.batch * a.hq)), dim3(D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
