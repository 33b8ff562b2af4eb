// prefill_f32.hip -- fp32 varlen causal attention on the vector ALUs.
//
// The FlashAttention one-pass algorithm of the blog post "从零实现 vLLM (1.3)：
// 如何加速 Attention 计算" (sections FlashAttention 的最终实现 and 计算流程
// (1-Pass 算法与分块)): K and V are cut into tiles along the sequence, each
// tile is staged in LDS, and every query row updates its running state
// (m, d', o') tile by tile.  o' is kept unnormalised and divided by d' once at
// the end (algebraically the same recurrence).
//
// This path exists for fp32 inputs, where the bf16 matrix cores do not apply:
// every product and sum is an fp32 FMA.  One thread (head_dim 64) or a
// pair of lanes (head_dim 128) owns one query row: q and o live in
// registers, K/V rows are broadcast from LDS.
//
// Exponentials run in base 2 with the scale folded in: with c = s*log2(e),
// p = 2^(fma(x, c, -m*c)).  The same rounded m*c is used for p and for the
// rescale factor 2^(m_old*c - m_new*c), so the rounding of m*c cancels in
// o/d' even when logits are near 700.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kF32Threads = 128;
constexpr int kF32Tile = 32;  // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(kF32Threads)
prefill_f32_kernel(VarlenArgs a, int nqt) {
    constexpr int TPR = D / 64;                   // lanes per query row
    constexpr int ROWS = kF32Threads / TPR;       // query rows per workgroup
    constexpr int DC = 64;                        // columns per lane
    __shared__ float4 sK[kF32Tile * D / 4];
    __shared__ float4 sV[kF32Tile * D / 4];

    // unit -> (query tile, sequence, head); heavy (late) tiles first
    int id = blockIdx.x;
    const int h = id % a.hq;
    id /= a.hq;
    const int b = id % a.batch;
    const int qt = nqt - 1 - id / a.batch;

    int64_t q0, q1;
    if (a.pad_q) {   // padded batch: rows b * pad_q .., seqlens_q[b] of them
        const int L = a.seqlens_q[b];
        q0 = (int64_t)b * a.pad_q;
        q1 = q0 + (L < 0 ? 0 : (L > a.pad_q ? a.pad_q : L));
    } else {
        q0 = a.cu_q[b];
        q1 = a.cu_q[b + 1];
        q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
        q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
    }
    const int Lq = (int)(q1 - q0);
    int64_t k0 = 0, k1 = 0;
    int Lk;
    if (a.pad_q) {
        const int L = a.seqlens_k[b];
        k0 = (int64_t)b * a.pad_k;
        Lk = L < 0 ? 0 : (L > a.pad_k ? a.pad_k : L);
    } else if (a.block_table) {
        k0 = a.cu_k[b];
        k1 = a.cu_k[b + 1];
        k1 = k1 < k0 ? k0 : k1;
        const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
        Lk = (int)((k1 - k0) > cap ? cap : (k1 - k0));
    } else {
        k0 = a.cu_k[b];
        k1 = a.cu_k[b + 1];
        k0 = k0 < 0 ? 0 : (k0 > a.total_k ? a.total_k : k0);
        k1 = k1 < k0 ? k0 : (k1 > a.total_k ? a.total_k : k1);
        Lk = (int)(k1 - k0);
    }
    const int p0 = qt * ROWS;
    if (p0 >= Lq) return;

    const int g = h / (a.hq / a.hkv);
    const int tid = threadIdx.x;
    const int row = tid / TPR;
    const int half = tid % TPR;
    const int pos = p0 + row;
    const bool valid = pos < Lq;
    const int off = Lk - Lq;  // causal alignment to the end of the sequence
    const int lim = valid ? (a.causal ? min(Lk, pos + off + 1) : Lk) : 0;
    const int last = min(p0 + ROWS, Lq) - 1;
    const int kv_end = a.causal ? min(Lk, last + off + 1) : Lk;

    float qr[DC], o[DC];
    {
        const float4 *qp = (const float4 *)((const float *)a.q +
                                            ((q0 + (valid ? pos : 0)) * a.hq + h) * (int64_t)D + half * DC);
#pragma unroll
        for (int c = 0; c < DC / 4; ++c) {
            float4 t = valid ? qp[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            qr[4 * c] = t.x; qr[4 * c + 1] = t.y; qr[4 * c + 2] = t.z; qr[4 * c + 3] = t.w;
        }
    }
#pragma unroll
    for (int c = 0; c < DC; ++c) o[c] = 0.f;
    float m = kNegInf, mc = 0.f, l = 0.f;
    const float cl = a.scale_log2;

    for (int t0 = 0; t0 < kv_end; t0 += kF32Tile) {
        __syncthreads();
        for (int i = tid; i < kF32Tile * D / 4; i += kF32Threads) {
            const int r = i / (D / 4), c4 = i % (D / 4);
            const int j = t0 + r;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (j < kv_end) {
                int64_t rowoff = -1;
                if (a.block_table) {
                    const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + j / a.block_size];
                    if (blk >= 0 && blk < a.num_blocks)
                        rowoff = ((int64_t)blk * a.block_size + j % a.block_size) * a.hkv + g;
                } else {
                    rowoff = (k0 + j) * a.hkv + g;
                }
                if (rowoff >= 0) {
                    kv = ((const float4 *)a.k)[rowoff * (D / 4) + c4];
                    vv = ((const float4 *)a.v)[rowoff * (D / 4) + c4];
                }
            }
            sK[i] = kv;
            sV[i] = vv;
        }
        __syncthreads();
        if (t0 >= lim) continue;

        // logits of this tile, masked
        float s[kF32Tile];
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            const float4 *kr = sK + j * (D / 4) + half * (DC / 4);
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < DC / 4; ++c) {
                const float4 kk = kr[c];
                acc = fmaf(qr[4 * c], kk.x, acc);
                acc = fmaf(qr[4 * c + 1], kk.y, acc);
                acc = fmaf(qr[4 * c + 2], kk.z, acc);
                acc = fmaf(qr[4 * c + 3], kk.w, acc);
            }
            if (TPR == 2) acc += __shfl_xor(acc, 1, 64);
            s[j] = (t0 + j < lim) ? acc : kNegInf;
            tmax = fmaxf(tmax, s[j]);
        }
        // online update of (m, d', o')
        const float m_new = fmaxf(m, tmax);
        const float mc_new = (m_new == kNegInf) ? 0.f : m_new * cl;
        const float alpha = (m == kNegInf) ? 0.f : fast_exp2(mc - mc_new);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < DC; ++c) o[c] *= alpha;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            const float p = fast_exp2(fmaf(s[j], cl, -mc_new));
            l += p;
            const float4 *vr = sV + j * (D / 4) + half * (DC / 4);
#pragma unroll
            for (int c = 0; c < DC / 4; ++c) {
                const float4 vv = vr[c];
                o[4 * c] = fmaf(p, vv.x, o[4 * c]);
                o[4 * c + 1] = fmaf(p, vv.y, o[4 * c + 1]);
                o[4 * c + 2] = fmaf(p, vv.z, o[4 * c + 2]);
                o[4 * c + 3] = fmaf(p, vv.w, o[4 * c + 3]);
            }
        }
        m = m_new;
        mc = mc_new;
    }

    if (!valid) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t obase = ((q0 + pos) * a.hq + h) * (int64_t)D + half * DC;
    if (a.out_f32) {
        float4 *op = (float4 *)((float *)a.o + obase);
#pragma unroll
        for (int c = 0; c < DC / 4; ++c)
            op[c] = make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv);
    } else {
        bf16x4 *op = (bf16x4 *)((bf16 *)a.o + obase);
#pragma unroll
        for (int c = 0; c < DC / 4; ++c) {
            bf16x4 r;
            r[0] = f32_to_bf16(o[4 * c] * inv);
            r[1] = f32_to_bf16(o[4 * c + 1] * inv);
            r[2] = f32_to_bf16(o[4 * c + 2] * inv);
            r[3] = f32_to_bf16(o[4 * c + 3] * inv);
            op[c] = r;
        }
    }
}

}  // namespace

hipError_t launch_prefill_f32(const VarlenArgs &a, hipStream_t stream) {
    const int rows = kF32Threads / (a.d / 64);
    const int nqt = (a.max_seqlen_q + rows - 1) / rows;
    const int64_t units = (int64_t)nqt * a.batch * a.hq;
    if (units == 0) return hipSuccess;
    if (a.d == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)units), dim3(kF32Threads), 0, stream, a, nqt);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)units), dim3(kF32Threads), 0, stream, a, nqt);
    return hipGetLastError();
}

}  // namespace attn
