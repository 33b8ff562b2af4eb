// prefill_bf16.hip -- fused varlen causal prefill on the gfx950 matrix cores.
//
// Algorithm: the FlashAttention one-pass recurrence of the blog post
// "从零实现 vLLM (1.3)：如何加速 Attention 计算" (sections FlashAttention 的最终
// 实现 and 计算流程(1-Pass 算法与分块)): K/V are cut into 64-key tiles along the
// sequence; each tile is staged in LDS and every query row updates its
// running (m, d', o') from it, so logits and probabilities stay in registers.
// o' is kept unnormalised and divided by d' once at the end.  Query rows run
// in parallel, each one serially over its key tiles.
//
// Mapping onto CDNA4:
// * A workgroup is 4 wavefronts.  It owns one KV head g, a block of query
//   positions and the (up to 4) query heads of g's GQA group, so every K/V
//   tile brought into LDS serves 128 query rows.  Each wavefront owns one
//   query head and 32 consecutive positions.
// * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys are the M dimension, so
//   the accumulator puts one query per lane and 16 of its keys in that lane's
//   registers.  Row max / row sum are then lane-local plus one exchange with
//   lane^32.  The key order inside each 32-key block is permuted (bits 2 and 3
//   of the row index swapped) so that the accumulator registers, rounded to
//   bf16, are directly the B operand of the next product.
// * O^T += V^T P^T with the same instruction (d is M, keys are K).  V^T
//   operands come straight from the row-major V tile through the gfx950
//   transposing LDS read (ds_read_b64_tr_b16); the accumulator again holds
//   one query per lane, so the rescale by 2^(m_old - m_new) is lane-local.
// * K and V tiles live in LDS with an XOR swizzle of 16-byte chunks chosen so
//   that both the row-wise 16-byte writes and the operand reads are free of
//   bank conflicts; two tile buffers let the global loads of tile t+1 overlap
//   the math of tile t with one barrier per tile.
// * Causal: tiles past the last visible key are never loaded; only tiles
//   that cross the diagonal (or the sequence end) are masked.  Work units are
//   issued heavy-first (latest query tiles first) and the KV head is the
//   fastest-varying index, so that with 8 KV heads each XCD keeps reusing
//   one head's K/V in its L2.
// * Exponentials in base 2 with c = s*log2(e): p = 2^(fma(x, c, -m*c)); the
//   rescale factor uses the same rounded m*c.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 64;      // keys per tile
constexpr int kRowsPerWave = 32;

// Swap bits 2 and 3: the key order inside a 32-key block.
__device__ __forceinline__ int perm23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte-chunk swizzles of the K and V tiles (see the file comment).
__device__ __forceinline__ int swz_k(int row) { return perm23(row & 15); }
__device__ __forceinline__ int swz_v(int row) {
    return (((row & 3) ^ ((row & 1) << 2)) << 1);
}

template <int D>
struct Smem {
    bf16 k[2][kBN * D];
    bf16 v[2][kBN * D];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 2)
prefill_bf16_kernel(VarlenArgs a, int nqt, int hpw, int head_chunks) {
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int KK = D / 16;         // MFMA k-steps over head_dim
    constexpr int DB = D / 32;         // 32-row blocks of d in O^T
    constexpr int LOADS = kBN * CH / kThreads;  // 16-byte loads per thread per tile
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);

    // ---- work unit -------------------------------------------------------
    int id = blockIdx.x;
    const int g = id % a.hkv;
    id /= a.hkv;
    const int hc = id % head_chunks;
    id /= head_chunks;
    const int b = id % a.batch;
    const int qt = nqt - 1 - id / a.batch;
    const int pos_per_wg = kRowsPerWave * (kWaves / hpw);

    int64_t q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
    q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
    q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
    const int Lq = (int)(q1 - q0);
    int64_t k0 = a.cu_k[b], k1 = a.cu_k[b + 1];
    int Lk;
    if (a.block_table) {
        k1 = k1 < k0 ? k0 : k1;
        const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
        Lk = (int)((k1 - k0) > cap ? cap : (k1 - k0));
    } else {
        k0 = k0 < 0 ? 0 : (k0 > a.total_k ? a.total_k : k0);
        k1 = k1 < k0 ? k0 : (k1 > a.total_k ? a.total_k : k1);
        Lk = (int)(k1 - k0);
    }
    const int p0 = qt * pos_per_wg;
    if (p0 >= Lq) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int group = a.hq / a.hkv;
    const int head = g * group + hc * hpw + (w % hpw);
    const int wp0 = p0 + kRowsPerWave * (w / hpw);   // first position of this wave
    const int n = lane & 31;                           // this lane's query
    const int hf = lane >> 5;                          // lane half
    const int pos = wp0 + n;
    const bool row_valid = pos < Lq;
    const int off = Lk - Lq;                           // end-aligned causal offset

    const int last = min(p0 + pos_per_wg, Lq) - 1;
    const int kv_end = a.causal ? max(0, min(Lk, last + off + 1)) : Lk;
    const int wlast = min(wp0 + kRowsPerWave, Lq) - 1;
    const int w_kv_end = (wp0 < Lq) ? (a.causal ? max(0, min(Lk, wlast + off + 1)) : Lk) : 0;
    const int w_kv_full = a.causal ? max(0, min(Lk, wp0 + off + 1)) : Lk;  // unmasked below this
    const int lim = row_valid ? (a.causal ? min(Lk, pos + off + 1) : Lk) : 0;

    // ---- Q operand: B[k = d][n = query], 8 consecutive d per lane ---------
    bf16x8 qf[KK];
    {
        const bf16 *qp = (const bf16 *)a.q + ((q0 + (row_valid ? pos : 0)) * a.hq + head) * (int64_t)D + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 t = row_valid ? ld16(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
            qf[kk] = *reinterpret_cast<bf16x8 *>(&t);
        }
    }

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m_run = kNegInf, mc_run = 0.f, l_run = 0.f;
    const float cl = a.scale_log2;

    // ---- global -> register staging of one K/V tile ----------------------
    const int ld_col = tid % CH;     // 16-byte chunk this thread moves
    const int ld_row0 = tid / CH;    // first tile row; rows ld_row0 + i*(kThreads/CH)
    uint4 stk[LOADS], stv[LOADS];

    auto load_tile = [&](int t0) {
        int64_t base = -1;  // element offset of row t0 (paged: of the tile's block row)
        if (a.block_table) {
            const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + t0 / a.block_size];
            if (blk >= 0 && blk < a.num_blocks)
                base = (((int64_t)blk * a.block_size + t0 % a.block_size) * a.hkv + g) * (int64_t)D;
        } else {
            base = ((k0 + t0) * a.hkv + g) * (int64_t)D;
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = ld_row0 + i * (kThreads / CH);
            if (base >= 0 && t0 + r < kv_end) {
                const int64_t e = base + (int64_t)r * a.hkv * D + ld_col * 8;
                stk[i] = ld16((const bf16 *)a.k + e);
                stv[i] = ld16((const bf16 *)a.v + e);
            } else {
                stk[i] = make_uint4(0, 0, 0, 0);
                stv[i] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = ld_row0 + i * (kThreads / CH);
            st16(&sm.k[buf][r * D + ((ld_col ^ swz_k(r)) * 8)], stk[i]);
            st16(&sm.v[buf][r * D + ((ld_col ^ swz_v(r)) * 8)], stv[i]);
        }
    };

    // per-lane LDS read offsets (elements)
    // K operand: row perm23(n) (+32 per key block), chunk (2kk + hf) ^ (lane & 15)
    const int k_row = perm23(n);
    // V^T operand via transposing reads: lane group gq = lane/16, s = lane%16
    const int gq = lane >> 4, s16 = lane & 15;
    const int v_row_part = 8 * (gq >> 1) + (s16 >> 2);             // + 32kb + 16j + 4r
    const int v_col_elem = 16 * (gq & 1) + 4 * (s16 & 3);          // + 32*dblk

    const int n_tiles = (kv_end + kBN - 1) / kBN;
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    for (int t = 0; t < n_tiles; ++t) {
        const int t0 = t * kBN;
        const int buf = t & 1;
        if (t + 1 < n_tiles) load_tile(t0 + kBN);
        __syncthreads();
        if (t0 < w_kv_end) {
            const bf16 *Kt = sm.k[buf];
            const bf16 *Vt = sm.v[buf];
            // ---- S^T = K Q^T for two 32-key blocks ----
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
                const bf16 *krow = Kt + (32 * kb + k_row) * D;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int ch = (2 * kk + hf) ^ (lane & 15);
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + ch * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
                }
            }
            // ---- mask (only tiles crossing the diagonal or the end) ----
            if (t0 + kBN > w_kv_full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = t0 + 32 * kb + (i < 8 ? 8 * hf + i : 16 + 8 * hf + (i - 8));
                        if (key >= lim) sacc[kb][i] = kNegInf;
                    }
            }
            // ---- online softmax update ----
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
            mx = fmaxf(mx, swap_halves(mx));
            const float m_new = fmaxf(m_run, mx);
            const float mc_new = (m_new == kNegInf) ? 0.f : m_new * cl;
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(mc_run - mc_new);
            float psum = 0.f;
            bf16x8 pb[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(fmaf(sacc[kb][i], cl, -mc_new));
                    psum += p;
                    pb[2 * kb + (i >> 3)][i & 7] = f32_to_bf16(p);
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            mc_run = mc_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int kb = jj >> 1, j = jj & 1;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    bf16x4 lo, hi;
                    {
                        const int r = 32 * kb + 16 * j + v_row_part;        // r-th read: +4r
                        const int col = 32 * db + v_col_elem;
                        const int ch0 = col >> 3, sub = col & 7;
                        const bf16 *p0 = Vt + r * D + ((ch0 ^ swz_v(r)) * 8) + sub;
                        const bf16 *p1 = Vt + (r + 4) * D + ((ch0 ^ swz_v(r + 4)) * 8) + sub;
                        lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)(p0));
                        hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)(p1));
                    }
                    const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[jj], o[db], 0, 0, 0);
                }
            }
        }
        if (t + 1 < n_tiles) store_tile(buf ^ 1);
    }

    // ---- epilogue: O = o' / d' ----
    if (!row_valid) return;
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((q0 + pos) * a.hq + head) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d0 = 32 * db + 8 * a4 + 4 * hf;
            const float v0 = o[db][4 * a4] * inv, v1 = o[db][4 * a4 + 1] * inv;
            const float v2 = o[db][4 * a4 + 2] * inv, v3 = o[db][4 * a4 + 3] * inv;
            if (a.out_f32) {
                *reinterpret_cast<float4 *>((float *)a.o + obase + d0) = make_float4(v0, v1, v2, v3);
            } else {
                bf16x4 r;
                r[0] = f32_to_bf16(v0); r[1] = f32_to_bf16(v1);
                r[2] = f32_to_bf16(v2); r[3] = f32_to_bf16(v3);
                *reinterpret_cast<bf16x4 *>((bf16 *)a.o + obase + d0) = r;
            }
        }
}

}  // namespace

hipError_t launch_prefill_bf16(const VarlenArgs &a, hipStream_t stream) {
    constexpr int D = 128;
    const int group = a.hq / a.hkv;
    const int hpw = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
    const int head_chunks = group / hpw;
    const int pos_per_wg = kRowsPerWave * (kWaves / hpw);
    const int nqt = (a.max_seqlen_q + pos_per_wg - 1) / pos_per_wg;
    const int64_t units = (int64_t)nqt * a.batch * head_chunks * a.hkv;
    if (units == 0) return hipSuccess;
    const size_t smem = sizeof(Smem<D>);
    hipError_t e = hipFuncSetAttribute((const void *)prefill_bf16_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)units), dim3(kThreads), smem, stream,
                       a, nqt, hpw, head_chunks);
    return hipGetLastError();
}

}  // namespace attn
