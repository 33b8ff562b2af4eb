// decode.hip -- single-token decode against a paged KV cache, split over
// the key range, plus the pass that merges the splits.
//
// What is computed is the Decode section of the blog post "从零实现 vLLM
// (1.3)：如何加速 Attention 计算": one new query per sequence attends to every
// cached token, reading K/V blocks through the block table (the page-table
// analogy of its Prefill section).  The key range of each (sequence, KV head)
// is cut into splits; runs of splits keep the online-softmax state of
// section FlashAttention 的最终实现 and leave a partial state (m, d', o'
// unnormalised).  Because the tile updates are associative (section
// 计算流程(1-Pass 算法与分块)), the combine kernel merges the partials with the
// same rescaling: M = max m_s, d' = sum d'_s 2^(m_s - M), o = sum o'_s
// 2^(m_s - M) / d'.
//
// Decode reads every K/V byte once and does ~4 flops per byte, so it is
// HBM-bound: the design keeps as many bytes in flight as possible.
// * The split kernel is persistent, two 4-wavefront workgroups per CU; each
//   wavefront has a whole 32-key chunk (16 KiB of K and V) in flight at a
//   time.  (Measured on this cache layout: a streaming read of 32-key chunks
//   by direct-to-LDS loads at 8 wavefronts per CU runs as fast as 64-key
//   chunks at 4 or 8 wavefronts per CU, ~5.8 TB/s.)
// * Work items are (sequence b, KV head g, split s), s < ceil(L_b / S).
//   Workgroup i of G serves head g = i mod hkv and takes the contiguous
//   range [r*J/R, (r+1)*J/R) of that head's J items (b, s), r = i / hkv,
//   R = G / hkv, so every workgroup reads the same number of splits.
//   Consecutive splits of one sequence are merged in registers: one partial
//   per run of splits (a segment), stored at the run's first split together
//   with the run length, which the combine pass uses to step from one
//   stored partial to the next.
// * Inside an item the 4 wavefronts take 32-key chunks round-robin.  K and V
//   rows go by direct global->LDS loads (four whole 256-byte rows per
//   instruction) into per-wavefront buffers.  K comes back by 16-byte reads
//   as the A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys = M,
//   query heads = N); V comes back transposed (ds_read_b64_tr_b16) as the A
//   operand of O^T += V^T P^T.  (Reading K straight into registers in the
//   operand layout touches 16 rows per instruction and streams ~6 % slower.)
// * Block ids are read one item ahead, so no chunk waits on the block
//   table before its K/V loads.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kChunk = 32;        // keys per wavefront step (16 KiB of K and V)
constexpr int kDecWgsPerCu = 2;   // persistent workgroups per CU (8 wavefronts)
constexpr int kWaitAll = 0x0070;   // s_waitcnt vmcnt(0) lgkmcnt(0)

// 16-byte-chunk swizzle of a V row in the LDS buffer (conflict-free
// transposing reads)
__device__ __forceinline__ int swz_dv(int row) { return (row & 7) << 1; }
// ... and of a K row (conflict-free 16-byte reads of 16 consecutive rows)
__device__ __forceinline__ int swz_dk(int row) { return row & 15; }

template <int D>
__global__ void __launch_bounds__(kDecThreads, kDecWgsPerCu)
decode_split_kernel(DecodeArgs a) {
    constexpr int KK = D / 32;          // k-steps of 32 over head_dim
    constexpr int DB = D / 16;          // 16-row blocks of d in O^T
    constexpr int MB = kChunk / 16;     // 16-key row blocks of a chunk
    constexpr int VI = kChunk / 4;      // direct-to-LDS loads per V chunk (4 rows each)
    constexpr int JJ = kChunk / 32;     // 32-key MFMA steps of P V
    static_assert(kChunk % 32 == 0, "chunks are whole 32-key MFMA steps");
    __shared__ __align__(16) bf16 sK[kDecWaves][kChunk * D];
    __shared__ __align__(16) bf16 sV[kDecWaves][kChunk * D];
    __shared__ float sMerge[kDecWaves][16][2];
    __shared__ int sStart[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = a.hq / a.hkv;
    const int n = lane & 15;            // query column of this lane (head g*group + n)
    const int gq = lane >> 4;           // lane group 0..3
    const bool qv = n < group;
    const int S = a.split_tokens;
    const int cap = a.max_blocks_per_seq * a.block_size;
    auto seq_len = [&](int b) ATTN_INLINE {
        const int L = ld_meta(a.cache_seqlens, b);
        return L < 0 ? 0 : (L > cap ? cap : L);
    };

    // ---- this workgroup's item range: wave 0 scans the per-sequence item
    // counts hkv * ceil(L_b / S) and posts the first item's (b, offset in b)
    if (w == 0) {
        auto items_of = [&](int b) ATTN_INLINE {
            int64_t c = 0;
            if (b < a.batch) {
                const int L = ld_meta(a.cache_seqlens, b);
                const int Lc = L < 0 ? 0 : (L > cap ? cap : L);
                c = (Lc + S - 1) / S;
            }
            return c;
        };
        auto scan = [&](int64_t c) ATTN_INLINE {    // inclusive scan over the wave
            int64_t x = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            return x;
        };
        int64_t total = 0;
        for (int b0 = 0; b0 < a.batch; b0 += 64) total += __shfl(scan(items_of(b0 + lane)), 63, 64);
        const int64_t R = gridDim.x / a.hkv, r = blockIdx.x / a.hkv;
        const int64_t beg = total * r / R;
        const int64_t end = total * (r + 1) / R;
        int64_t run = 0;
        int bsel = a.batch, off_sel = 0;
        for (int b0 = 0; b0 < a.batch && bsel == a.batch; b0 += 64) {
            const int64_t c = items_of(b0 + lane);
            const int64_t x = scan(c);
            const uint64_t hit = __builtin_amdgcn_ballot_w64(b0 + lane < a.batch && run + x > beg);
            if (hit) {
                const int l = (int)__builtin_ctzll(hit);
                bsel = b0 + l;
                off_sel = (int)(beg - (run + __shfl(x - c, l, 64)));
            }
            run += __shfl(x, 63, 64);
        }
        if (lane == 0) {
            sStart[0] = bsel;
            sStart[1] = off_sel;
            sStart[2] = (int)(end - beg);
        }
    }
    __syncthreads();
    int b = __builtin_amdgcn_readfirstlane(sStart[0]);
    const int n_items = __builtin_amdgcn_readfirstlane(sStart[2]);
    if (n_items <= 0 || b >= a.batch) return;
    int L = seq_len(b);
    int ns = (L + S - 1) / S;
    const int g = (int)(blockIdx.x % a.hkv);
    int s = __builtin_amdgcn_readfirstlane(sStart[1]);

    bf16x8 qf[KK];
    auto load_q = [&]() ATTN_INLINE {
        const int head = g * group + (qv ? n : 0);
        const bf16 *qp = (const bf16 *)a.q + ((int64_t)b * a.hq + head) * D + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 t = qv ? ld16(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
            qf[kk] = *reinterpret_cast<bf16x8 *>(&t);
        }
    };
    load_q();
    f32x4 o[DB];
    float m_run, mc_run, l_run;
    auto reset = [&]() ATTN_INLINE {
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] = f32x4{};
        m_run = kNegInf;
        mc_run = 0.f;
        l_run = 0.f;
    };
    reset();
    const float cl = a.scale_log2;
    bf16 *vbuf = sV[w];
    const uint32_t vbuf_lds = lds_addr(vbuf);
    bf16 *kbuf = sK[w];
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const int64_t rstride = (int64_t)a.hkv * D;        // elements between key rows
    const uint32_t row_bytes = (uint32_t)rstride * 2;

    // one chunk [c0, c0 + kChunk) of (b, g) inside block blk, keys >= kend masked
    auto chunk = [&](int c0, int kend, int blk) ATTN_INLINE {
        const bool bok = blk >= 0 && blk < a.num_blocks;
        const int64_t base = ((((int64_t)(bok ? blk : 0) * a.block_size + c0 % a.block_size) * a.hkv + g) * D);
        const int last = kend - 1 - c0;                    // last valid row of the chunk
        // K and V -> LDS: load i covers rows 4i .. 4i+3 (four whole 256-byte
        // rows per instruction); lane l lands at physical chunk (l & 15) of
        // row 4i + (l >> 4) and fetches the logical chunk the swizzle puts
        // there.  Rows past the split end repeat its last key (finite data;
        // their weights are zero).
        if (bok) {
            const bf16 *ksrc = (const bf16 *)a.k_cache + base;
            const bf16 *vsrc = (const bf16 *)a.v_cache + base;
#pragma unroll
            for (int i = 0; i < VI; ++i) {
                const int row = 4 * i + gq;
                const uint32_t roff = (uint32_t)min(row, last) * row_bytes;
                lds_dma16(ksrc, roff + (uint32_t)((n ^ swz_dk(row)) * 16), kbuf_lds + i * 4 * D * 2);
                lds_dma16(vsrc, roff + (uint32_t)((n ^ swz_dv(row)) * 16), vbuf_lds + i * 4 * D * 2);
            }
        } else {
            // a block id outside the pool reads as zero rows
#pragma unroll
            for (int i = 0; i < VI; ++i) {
                st16(kbuf + (4 * i + gq) * D + 8 * n, make_uint4(0, 0, 0, 0));
                st16(vbuf + (4 * i + gq) * D + 8 * n, make_uint4(0, 0, 0, 0));
            }
        }
        // the K and V rows (direct loads, or the zero fill) must have landed
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // K operands: row blocks of 16 keys; lane holds key (16mb + n) and,
        // for k-step kk, d in [32kk + 8gq, +8) (Q uses the same order of d)
        uint4 kr[MB][KK];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int row = 16 * mb + n;
                kr[mb][kk] = *reinterpret_cast<const uint4 *>(kbuf + row * D + (((4 * kk + gq) ^ swz_dk(row)) * 8));
            }
        // S^T = K Q^T
        f32x4 sacc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            sacc[mb] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    *reinterpret_cast<bf16x8 *>(&kr[mb][kk]), qf[kk], sacc[mb], 0, 0, 0);
        }
        // mask keys past the split end: lane holds keys 16mb + 4gq + i
        if (last < kChunk - 1) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * mb + 4 * gq + i > last) sacc[mb][i] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[mb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float mc_new = (m_new == kNegInf) ? 0.f : m_new * cl;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(mc_run - mc_new);
        float psum = 0.f;
        bf16x8 pb[JJ];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
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
        // O^T += V^T P^T, 32 keys per step (keys 32jj + 4gq + e and +16)
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj)
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
        // the reads of kbuf and vbuf must finish before the next chunk's loads land
        __builtin_amdgcn_s_waitcnt(kWaitAll);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // merge the 4 wavefronts' states of the segment that started at split
    // s_first and covered cnt splits; write its partial
    auto write_partial = [&](int s_first, int cnt) ATTN_INLINE {
        float lsum_w = l_run;
        lsum_w += __shfl_xor(lsum_w, 16, 64);
        lsum_w += __shfl_xor(lsum_w, 32, 64);
        const float mlog = (m_run == kNegInf) ? kNegInf : mc_run;   // log2-scaled max or -inf
        if (gq == 0) {
            sMerge[w][n][0] = mlog;
            sMerge[w][n][1] = lsum_w;
        }
        __syncthreads();   // every wave is done with its V buffer and has posted m, l
        float *sO = reinterpret_cast<float *>(&sV[0][0]);   // [waves][16][D] floats (reuse)
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, sMerge[ww][n][0]);
        const float myscale = (mlog == kNegInf) ? 0.f : fast_exp2(mlog - M);
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
            const int64_t row = ((int64_t)b * a.hq + g * group + qi) * a.max_splits + s_first;
            a.ws_o[row * D + d] = acc;
            if (d == 0) {
                a.ws_ml[row * 4] = Mq;
                a.ws_ml[row * 4 + 1] = lsum;
                a.ws_ml[row * 4 + 2] = __int_as_float(cnt);
            }
        }
        __syncthreads();   // sO (the V buffers) and sMerge are free again
    };

    // block id of this wave's first chunk of an item, loaded one item ahead
    // so that no chunk waits on a table read before its K/V loads
    const int bt_last = a.max_blocks_per_seq - 1;
    auto first_blk = [&](int bb, int ss) ATTN_INLINE {
        const int idx = min((ss * S + kChunk * w) / a.block_size, bt_last);
        return ld_meta(a.block_table, (int64_t)bb * a.max_blocks_per_seq + idx);
    };
    int blk_cur = first_blk(b, s);
    int L_next = b + 1 < a.batch ? seq_len(b + 1) : 0;   // length of sequence b + 1
    int s_first = s, cnt = 0;
    for (int it = 0; it < n_items; ++it) {
        // the next item, and its block id
        int nb = b, nsp = s + 1;
        if (nsp == ns) {
            nsp = 0;
            ++nb;
        }
        const bool last = it + 1 == n_items;
        int blk_next = 0;
        if (!last && (nb == b || L_next > 0)) blk_next = first_blk(nb, nsp);
        // split s of (b, g): chunks c0 = s*S + kChunk (w + 4j); a chunk never
        // crosses a block (block_size is a multiple of 64)
        const int kend = min(L, (s + 1) * S);
        const int bi0 = (s * S + kChunk * w) / a.block_size;
        for (int c0 = s * S + kChunk * w; c0 < kend; c0 += kDecWaves * kChunk) {
            const int bi = c0 / a.block_size;
            const int blk = bi == bi0 ? blk_cur
                                      : ld_meta(a.block_table, (int64_t)b * a.max_blocks_per_seq + bi);
            chunk(c0, kend, blk);
        }
        ++cnt;
        if (last || nb != b) {
            write_partial(s_first, cnt);
            if (last) break;
            reset();
            if (nb != b) {
                // the next sequence with items
                L = L_next;
                ns = (L + S - 1) / S;
                while (ns == 0 && nb < a.batch) {
                    ++nb;
                    L = nb < a.batch ? seq_len(nb) : 0;
                    ns = (L + S - 1) / S;
                    nsp = 0;
                    blk_next = nb < a.batch ? first_blk(nb, 0) : 0;
                }
                if (nb >= a.batch) break;
                L_next = nb + 1 < a.batch ? seq_len(nb + 1) : 0;
            }
            b = nb;
            s = nsp;
            s_first = s;
            cnt = 0;
            load_q();
        } else {
            s = nsp;
        }
        blk_cur = blk_next;
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
    // stored partials sit at the first split of each segment, which records
    // how many splits it covers; online merge of the partials
    float M = kNegInf, acc = 0.f, lsum = 0.f;
    for (int s = 0; s < ns;) {
        const float ms = a.ws_ml[(row0 + s) * 4];
        const float ls = a.ws_ml[(row0 + s) * 4 + 1];
        const int cnt = __float_as_int(a.ws_ml[(row0 + s) * 4 + 2]);
        if (ms != kNegInf) {
            const float Mn = fmaxf(M, ms);
            const float fo = (M == kNegInf) ? 0.f : fast_exp2(M - Mn);
            const float fs = fast_exp2(ms - Mn);
            acc = acc * fo + a.ws_o[(row0 + s) * D + d] * fs;
            lsum = lsum * fo + ls * fs;
            M = Mn;
        }
        s += cnt > 0 ? cnt : 1;
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
    if (a.batch == 0) return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // kDecWgsPerCu persistent workgroups per CU, a multiple of hkv (one KV
    // head each), never more than there are items
    const int64_t items_max = (int64_t)a.batch * a.max_splits * a.hkv;
    int64_t grid = kDecWgsPerCu * (int64_t)(cus > 0 ? cus : 1);
    if (grid > items_max) grid = items_max;
    grid -= grid % a.hkv;
    if (grid > 0)
        hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)grid), dim3(kDecThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(a.batch * a.hq)), dim3(D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
