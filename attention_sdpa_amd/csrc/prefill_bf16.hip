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
// * A workgroup is 8 wavefronts and owns one KV head g, a block of query
//   positions and the (up to 4) query heads of g's GQA group, so every K/V
//   tile brought into LDS serves 256 query rows.  Each wavefront owns one
//   query head and 32 consecutive positions.
// * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys are the M dimension, so
//   the accumulator puts one query per lane and 16 of its keys in that lane's
//   registers.  Row max / row sum are then lane-local plus one exchange of the
//   two 32-lane halves (v_permlane32_swap).  The key order inside each 32-key
//   block is permuted (bits 2 and 3 of the row index swapped) so that the
//   accumulator registers, rounded to bf16, are directly the B operand of the
//   next product.
// * O^T += V^T P^T with the same instruction (d is M, keys are K).  V^T
//   operands come straight from the row-major V tile through the gfx950
//   transposing LDS read (ds_read_b64_tr_b16); the accumulator again holds
//   one query per lane, so any rescale is lane-local.
// * K/V tiles reach LDS by direct global->LDS loads (global_load_lds_dwordx4,
//   no register staging) into a ring of three stages: the loads of tile t+2
//   are issued while tile t is computed, and one barrier per tile suffices.
//   16-byte chunks are XOR-swizzled (the swizzle is applied by choosing which
//   global chunk each lane fetches) so that the operand reads are free of
//   bank conflicts.
// * Causal: tiles past the last visible key are never loaded; only tiles
//   that cross the diagonal (or the sequence end) are masked.  Work units are
//   issued heavy-first (latest query tiles first) and the KV head is the
//   fastest-varying index, so that with 8 KV heads each XCD keeps reusing
//   one head's K/V in its L2.
// * Exponentials in base 2 with c = s*log2(e): p = 2^(fma(x, c, -r*c)) for a
//   per-row reference r.  r follows the running maximum lazily: it is raised
//   (and o', d' rescaled by 2^(r_old*c - r_new*c), the same rounded
//   products) only when the maximum exceeds it by more than 2^8, which keeps
//   p <= 256 and leaves the result unchanged in exact arithmetic.
// * Row sums are accumulated from the bf16-rounded P with v_dot2_f32_bf16,
//   i.e. from exactly the weights the P V product uses.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 64;              // keys per tile
constexpr int kRowsPerWave = 32;
constexpr int kD = 128;
constexpr int kTileElems = kBN * kD;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)

// Swap bits 2 and 3: the key order inside a 32-key block.
__device__ __forceinline__ int perm23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte-chunk swizzles of the K and V tiles (see the file comment).
__device__ __forceinline__ int swz_k(int row) { return perm23(row & 15); }
__device__ __forceinline__ int swz_v(int row) {
    return (((row & 3) ^ ((row & 1) << 2)) << 1);
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with lgkmcnt(0), expcnt off.
constexpr int kWaitVm0 = 0x0070;
constexpr int kWaitVm2 = 0x0072;
constexpr int kWaitVm4 = 0x0074;
constexpr int kWaitVm6 = 0x0076;
constexpr int kWaitVm8 = 0x0078;
constexpr int kWaitNone = 0xC07F;   // no counter wait (vmcnt 63, lgkmcnt 15)

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

#define LDS_PTR(p) ((ATTN_LDS void *)(p))
#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void *)(p))

// All waves' loads of the current stage have landed; nobody still reads the
// stage about to be refilled.  The empty asm statements keep the compiler
// from moving memory operations across the barrier.
template <int WAIT>
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAIT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__global__ void __launch_bounds__(kThreads, 1)
prefill_bf16_kernel(VarlenArgs a, int nqt, int hpw, int head_chunks) {
    constexpr int KK = kD / 16;         // MFMA k-steps over head_dim
    constexpr int DB = kD / 32;         // 32-row blocks of d in O^T
    // three-stage rings; stage s of K is sK[s] (one array per tensor, so that
    // stage addresses differ from a shared base by constants)
    __shared__ __align__(16) bf16 sK[3][kTileElems];
    __shared__ __align__(16) bf16 sV[3][kTileElems];

    // ---- work unit -------------------------------------------------------
    int id = blockIdx.x;
    const int g = id % a.hkv;
    id /= a.hkv;
    const int hc = id % head_chunks;
    id /= head_chunks;
    const int b = id % a.batch;
    const int qt = nqt - 1 - id / a.batch;
    const int pos_per_wg = kRowsPerWave * (kWaves / hpw);

    int64_t q0 = ld_meta(a.cu_q, b), q1 = ld_meta(a.cu_q, b + 1);
    q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
    q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
    const int Lq = (int)(q1 - q0);
    int64_t k0 = ld_meta(a.cu_k, b), k1 = ld_meta(a.cu_k, b + 1);
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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = a.hq / a.hkv;
    const int head = g * group + hc * hpw + (w % hpw);
    const int wp0 = p0 + kRowsPerWave * (w / hpw);    // first position of this wave
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
        const bf16 *qp = (const bf16 *)a.q + ((q0 + (row_valid ? pos : 0)) * a.hq + head) * (int64_t)kD + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 t = row_valid ? ld16(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
            qf[kk] = *reinterpret_cast<bf16x8 *>(&t);
        }
    }

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m_ref = kNegInf, mc_ref = 0.f, l_run = 0.f;
    const float cl = a.scale_log2;
    const bf16x2 ones2 = {(bf16)1.f, (bf16)1.f};

    // ---- direct global -> LDS loads of one K or V tile ---------------------
    // Wave w fills tile rows 8w .. 8w+7 with two 1 KiB loads; lane l lands at
    // physical chunk (l & 15) of row 8w + 4i + (l >> 4) and fetches the
    // logical chunk that the swizzle puts there.  Rows past the last needed
    // key repeat that key (finite data; those keys are masked or unused).
    const int dr = lane >> 4, dc = lane & 15;
    auto tile_rowbase = [&](int t0) ATTN_INLINE -> int64_t {
        if (a.block_table) {
            int blk = ld_meta(a.block_table, (int64_t)b * a.max_blocks_per_seq + t0 / a.block_size);
            blk = (blk >= 0 && blk < a.num_blocks) ? blk : 0;   // bad id: stay in bounds
            return (int64_t)blk * a.block_size - t0 + (t0 % a.block_size);
        }
        return k0;
    };
    auto issue_k = [&](int t, bf16 *dst) ATTN_INLINE {
        const int t0 = t * kBN;
        const int64_t base = tile_rowbase(t0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 8 * w + 4 * i + dr;
            const int j = min(t0 + r, kv_end - 1);
            const bf16 *src = (const bf16 *)a.k + ((base + j) * a.hkv + g) * (int64_t)kD + ((dc ^ swz_k(r)) * 8);
            __builtin_amdgcn_global_load_lds(GLOBAL_PTR(src), LDS_PTR(dst + (8 * w + 4 * i) * kD), 16, 0, 0);
        }
    };
    auto issue_v = [&](int t, bf16 *dst) ATTN_INLINE {
        const int t0 = t * kBN;
        const int64_t base = tile_rowbase(t0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 8 * w + 4 * i + dr;
            const int j = min(t0 + r, kv_end - 1);
            const bf16 *src = (const bf16 *)a.v + ((base + j) * a.hkv + g) * (int64_t)kD + ((dc ^ swz_v(r)) * 8);
            __builtin_amdgcn_global_load_lds(GLOBAL_PTR(src), LDS_PTR(dst + (8 * w + 4 * i) * kD), 16, 0, 0);
        }
    };

    // per-lane LDS read offsets (elements)
    const int k_row = perm23(n);                                   // + 32 per key block
    const int gq = lane >> 4, s16 = lane & 15;
    const int v_row_part = 8 * (gq >> 1) + (s16 >> 2);             // + 32kb + 16j (+4 second read)
    const int v_col_elem = 16 * (gq & 1) + 4 * (s16 & 3);          // + 32*dblk

    // S^T = K Q^T for a 64-key tile (two 32-key blocks)
    f32x16 sacc[2];
    auto qk = [&](const bf16 *Kt) ATTN_INLINE {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16{};
            const bf16 *krow = Kt + (32 * kb + k_row) * kD;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int ch = (2 * kk + hf) ^ (lane & 15);
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + ch * 8);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[kb], 0, 0, 0);
            }
        }
        // issue order: 4 operand reads ahead, then one read per product
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    };
    // O^T += V^T P^T for a 64-key tile, and the row sums from the same bf16
    // weights
    bf16x8 pb[4];
    auto pv = [&](const bf16 *Vt) ATTN_INLINE {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int r = 16 * jj + v_row_part;
                const int col = 32 * db + v_col_elem;
                const int ch0 = col >> 3, sub = col & 7;
                const bf16 *p0r = Vt + r * kD + ((ch0 ^ swz_v(r)) * 8) + sub;
                const bf16 *p1r = Vt + (r + 4) * kD + ((ch0 ^ swz_v(r + 4)) * 8) + sub;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)(p0r));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4 *)(p1r));
                const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[jj], o[db], 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bf16x2 pr;
                pr[0] = pb[jj][2 * e];
                pr[1] = pb[jj][2 * e + 1];
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_run, false);
            }
        }
        // issue order: two products' operands ahead, then per product its
        // next operands and one row-sum step
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 14; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 1, 0);
        }
    };
    // softmax phase of tile t: mask (diagonal/end tiles only), row max, lazy
    // reference update (rescaling o', d' if it moves), P = 2^(S c - r c) in
    // bf16 -- the B operand of the next P V
    auto softmax = [&](int t) ATTN_INLINE {
        const int t0 = t * kBN;
        if (t0 + kBN > w_kv_full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = t0 + 32 * kb + (i < 8 ? 8 * hf + i : 16 + 8 * hf + (i - 8));
                    if (key >= lim) sacc[kb][i] = kNegInf;
                }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const bool need = mx > m_ref && (m_ref == kNegInf || mx * cl > mc_ref + kRescaleLog2);
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float m_new = fmaxf(m_ref, mx);
            const float mc_new = (m_new == kNegInf) ? 0.f : m_new * cl;
            const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2(mc_ref - mc_new);
            m_ref = m_new;
            mc_ref = mc_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pb[2 * kb + (i >> 3)][i & 7] = f32_to_bf16(fast_exp2(fmaf(sacc[kb][i], cl, -mc_ref)));
    };

    // ---- ping-pong schedule ---------------------------------------------
    // Waves 0-3 (group A) and 4-7 (group B) sit on the four SIMDs in pairs.
    // Every wave runs the same program -- matrix half-step for tile t
    // (S(t+1) = K(t+1) Q^T and O += P(t) V(t)), then the vector softmax of
    // tile t+1 -- but group B runs it one half-step behind group A, so on each
    // SIMD the matrix core works for one wave while the vector ALU works for
    // the other.  A barrier separates half-steps.  K and V use three-stage
    // rings: K(t+3) and V(t+2) are issued at absolute half-step 2t, four
    // half-steps before their first use, into stages freed at half-step 2t-1.
    const int n_tiles = (kv_end + kBN - 1) / kBN;        // tiles of the workgroup
    const int nw = (w_kv_end + kBN - 1) / kBN;           // tiles this wave computes
    const bool grpA = w < 4;
    // the barrier opening absolute half-step 2t: tiles K(t+1), V(t) must have
    // landed (loads of tile t+1's half-steps -- K(t+2), V(t+1) -- may still be
    // in flight), then the freed stages are refilled
    auto even_barrier = [&](int t, bf16 *Kf, bf16 *Vf) ATTN_INLINE {
        const int pend = 2 * (t + 2 < n_tiles) + 2 * (t + 1 < n_tiles);
        if (pend == 4) stage_barrier<kWaitVm4>();
        else if (pend == 2) stage_barrier<kWaitVm2>();
        else stage_barrier<kWaitVm0>();
        if (t + 3 < n_tiles) issue_k(t + 3, Kf);
        if (t + 2 < n_tiles) issue_v(t + 2, Vf);
    };
    auto mfma_phase = [&](int t, const bf16 *Kn, const bf16 *Vc) ATTN_INLINE {
        __builtin_amdgcn_s_setprio(1);
        if (t < nw) {
            if (t + 1 < nw) qk(Kn);
            pv(Vc);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // prologue: K(0), K(1), V(0), K(2), V(1) in that order
    if (n_tiles > 0) issue_k(0, sK[0]);
    if (n_tiles > 1) issue_k(1, sK[1]);
    if (n_tiles > 0) issue_v(0, sV[0]);
    if (n_tiles > 2) issue_k(2, sK[2]);
    if (n_tiles > 1) issue_v(1, sV[1]);
    {
        // half-step -2: K(0) landed; everything issued after it may be in flight
        const int after = (n_tiles > 1 ? 4 : 0) + 2 + (n_tiles > 2 ? 2 : 0);
        if (after == 8) stage_barrier<kWaitVm8>();
        else if (after == 6) stage_barrier<kWaitVm6>();
        else stage_barrier<kWaitVm2>();
    }
    if (grpA && nw > 0) qk(sK[0]);
    stage_barrier<kWaitNone>();                          // half-step -1
    if (grpA) {
        if (nw > 0) softmax(0);
    } else {
        if (nw > 0) qk(sK[0]);
        even_barrier(0, sK[0], sV[2]);                   // half-step 0
        if (nw > 0) softmax(0);
    }
    // iteration t: A runs half-steps 2t, 2t+1; B runs 2t+1, 2t+2
    auto iter = [&](int t, const bf16 *Kn, const bf16 *Vc, bf16 *KfA, bf16 *VfA, bf16 *KfB, bf16 *VfB)
        ATTN_INLINE {
        if (grpA) even_barrier(t, KfA, VfA);
        else stage_barrier<kWaitNone>();
        mfma_phase(t, Kn, Vc);
        if (grpA) stage_barrier<kWaitNone>();
        else even_barrier(t + 1, KfB, VfB);
        if (t + 1 < nw) softmax(t + 1);
    };
    for (int t = 0; t < n_tiles; t += 3) {
        iter(t, sK[1], sV[0], sK[0], sV[2], sK[1], sV[0]);
        if (t + 1 < n_tiles) iter(t + 1, sK[2], sV[1], sK[1], sV[0], sK[2], sV[1]);
        if (t + 2 < n_tiles) iter(t + 2, sK[0], sV[2], sK[2], sV[1], sK[0], sV[2]);
    }
    if (grpA) stage_barrier<kWaitNone>();                // B's last half-step

    // ---- epilogue: O = o' / d' ----
    if (!row_valid) return;
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((q0 + pos) * a.hq + head) * (int64_t)kD;
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
    const int group = a.hq / a.hkv;
    const int hpw = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
    const int head_chunks = group / hpw;
    const int pos_per_wg = kRowsPerWave * (kWaves / hpw);
    const int nqt = (a.max_seqlen_q + pos_per_wg - 1) / pos_per_wg;
    const int64_t units = (int64_t)nqt * a.batch * head_chunks * a.hkv;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)units), dim3(kThreads), 0, stream,
                       a, nqt, hpw, head_chunks);
    return hipGetLastError();
}

}  // namespace attn
