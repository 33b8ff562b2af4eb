// decode.hip -- single-token decode against a paged KV cache, split over
// the key range, plus the pass that merges the splits.
//
// What is computed is the Decode section of the blog post "从零实现 vLLM
// (1.3)：如何加速 Attention 计算": one new query per sequence attends to every
// cached token, reading K/V blocks through the block table (the page-table
// analogy of its Prefill section).  The keys of every sequence are cut into
// items of S keys; a workgroup walks a contiguous run of items with the
// online-softmax state of section FlashAttention 的最终实现 and leaves one
// partial state (m, d', o' unnormalised) per sequence it touches.  Because
// the tile updates are associative (section 计算流程(1-Pass 算法与分块)), the
// combine kernel merges the partials with the same rescaling:
// M = max m_r, d' = sum d'_r 2^(m_r - M), o = sum o'_r 2^(m_r - M) / d'.
//
// Decode reads every K/V byte once and does ~4 flops per byte, so it is
// HBM-bound: the design keeps bytes in flight and every CU busy to the end.
// * Partition by keys, all heads together.  The items of all sequences,
//   in order, form one stream of C items; run r of R takes items
//   [floor(r C / R), floor((r+1) C / R)), so every run holds the same number
//   of keys to within one item (default S = 32 keys).  One workgroup per CU
//   serves a run for a block of up to 8 KV heads: its 8 wavefronts split the
//   heads of the block (one wavefront per head when there are 8), so a CU
//   reads whole cache rows of its keys, and no head or XCD gets more than
//   its share.  (Measured: one workgroup per KV head left the slowest head
//   ~15 % behind the fastest, and a streaming read of whole token rows runs
//   faster than one of a single head's 256-byte slices.)
// * Segments: the part of a run that falls in one sequence.  Its partial
//   goes to slot r + b (unique: runs and sequences both advance along the
//   stream).  The runs holding the first and the last item of b post their
//   indices; every run in use holds an item, so the partials of b are the
//   slots r + b for r between the two, which the combine reads at once.
//   With one wavefront per head, the wavefront writes its partial straight
//   from registers and has already requested the next segment's first
//   chunk, so a sequence boundary leaves no gap in the run's stream
//   (measured: +2.8 % for the whole call).
// * Each wavefront takes 32-key chunks of its head (round-robin when
//   several wavefronts share a head).  K and V rows go by direct
//   global->LDS loads (four whole 256-byte rows per instruction) into
//   per-wavefront buffers.  K comes back by 16-byte reads as the A operand
//   of S^T = K Q^T (v_mfma_f32_16x16x32_bf16 or _f16, keys = M, query heads = N);
//   V comes back by transposing reads (ds_read_b64_tr_b16) as the A operand
//   of O^T += V^T P^T.  Both are read into registers before any arithmetic,
//   and the next chunk's K and V loads are issued into the same buffers
//   right then: a wavefront has a chunk in flight while it computes.
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kChunk = 32;         // keys per wavefront step (16 KiB of K and V)

// 16-byte-chunk swizzle of a V row in the LDS buffer (conflict-free
// transposing reads)
__device__ __forceinline__ int swz_dv(int row) { return (row & 7) << 1; }
// ... and of a K row (conflict-free 16-byte reads of 16 consecutive rows)
__device__ __forceinline__ int swz_dk(int row) { return row & 15; }

// Waits with a memory clobber, so that the compiler moves no memory access
// across them: every vector-memory and LDS access (including the
// direct-to-LDS loads) / every LDS and scalar access is complete.  The full
// wait is the s_waitcnt builtin, not asm text, so that the compiler's own
// wait tracking sees it too: it then knows the query fragments (ordinary
// loads) have landed and adds no wait for them before the MFMAs -- a wait
// that, counted by the hardware, would also cover the next chunk's
// direct-to-LDS loads issued just before and serialise them with the math.
__device__ __forceinline__ void wait_all() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);     // vmcnt(0) expcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Heads per workgroup block: hkv rounded up to a power of two, at most 8.
__host__ __device__ __forceinline__ int heads_per_block(int hkv) {
    return hkv >= 8 ? 8 : (hkv > 4 ? 8 : (hkv > 2 ? 4 : hkv));
}

template <typename T, int D>
__global__ void __launch_bounds__(kDecThreads, 1)
decode_split_kernel(DecodeArgs a) {
    typedef typename Vec16<T>::x4 T4;
    typedef typename Vec16<T>::x8 T8;
    constexpr int KK = D / 32;          // k-steps of 32 over head_dim
    constexpr int DB = D / 16;          // 16-row blocks of d in O^T
    constexpr int MB = kChunk / 16;     // 16-key row blocks of a chunk
    constexpr int VI = kChunk / 4;      // direct-to-LDS loads per chunk (4 rows each)
    constexpr int JJ = kChunk / 32;     // 32-key MFMA steps of P V
    static_assert(kChunk % 32 == 0, "chunks are whole 32-key MFMA steps");
    __shared__ __align__(16) bf16 sK[kDecWaves][kChunk * D];
    __shared__ __align__(16) bf16 sV[kDecWaves][kChunk * D];
    __shared__ float sMerge[kDecWaves][16][2];
    __shared__ int sStart[3];

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
    // head block of this workgroup, and this wave's head and phase in it
    const int HB = heads_per_block(a.hkv);
    const int NB = (a.hkv + HB - 1) / HB;
    const int wpH = kDecWaves / HB;                 // waves per head
    const int hb = (int)blockIdx.x % NB;
    const int r = (int)blockIdx.x / NB;
    const int R = a.n_runs;
    const int hl = w % HB, ph = w / HB;
    const int g = hb * HB + hl;
    const bool active = g < a.hkv;
    // one wavefront per head and every wavefront active: all take the same
    // chunks, so they can meet at a barrier once per chunk
    const bool sync_waves = HB == kDecWaves && a.hkv % kDecWaves == 0;

    // ---- this run's items: wave 0 scans the per-sequence item counts
    // ceil(L_b / S) and posts the first item's (b, offset in b)
    if (w == 0) {
        auto items_of = [&](int b) ATTN_INLINE {
            int64_t c = 0;
            if (b < a.batch) c = ((int64_t)seq_len(b) + S - 1) / S;
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
        // runs that would hold no item are not used, so that every run in
        // use holds at least one
        const int64_t Re = total < R ? total : R;
        const int64_t beg = r < Re ? total * r / Re : 0;
        const int64_t end = r < Re ? total * (r + 1) / Re : 0;
        int64_t run = 0;
        int bsel = a.batch, off_sel = 0;
        for (int b0 = 0; b0 < a.batch && bsel == a.batch && end > beg; b0 += 64) {
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
    int s = __builtin_amdgcn_readfirstlane(sStart[1]);
    const int n_items = __builtin_amdgcn_readfirstlane(sStart[2]);
    if (n_items <= 0 || b >= a.batch) return;

    T8 qf[KK];
    f32x4 o[DB];
    float m_run, mc_run, l_run;
    const float cl = a.scale_log2;
    bf16 *vbuf = sV[w];
    const uint32_t vbuf_lds = lds_addr(vbuf);
    bf16 *kbuf = sK[w];
    const uint32_t kbuf_lds = lds_addr(kbuf);
    const int64_t rstride = (int64_t)a.hkv * D;        // elements between key rows
    const uint32_t row_bytes = (uint32_t)rstride * 2;
    const int gs = active ? g : 0;

    // block id of the chunk starting at key c0 of sequence b (-1: outside the pool)
    auto blk_of = [&](int bb, int c0) ATTN_INLINE {
        const int blk = ld_meta(a.block_table, (int64_t)bb * a.max_blocks_per_seq + c0 / a.block_size);
        return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
    };
    // K (or V) rows of the chunk [c0, c0 + kChunk) -> this wave's buffer.
    // Load i covers rows 4i .. 4i+3 (four whole 256-byte rows per
    // instruction); lane l lands at physical chunk (l & 15) of row 4i + (l >> 4)
    // and fetches the logical chunk the swizzle puts there.  Rows past the
    // segment end repeat its last key (finite data; their weights are zero);
    // a block id outside the pool reads as zero rows.
    auto issue = [&](bool is_v, int c0, int kend, int blk) ATTN_INLINE {
        bf16 *buf = is_v ? vbuf : kbuf;
        if (blk >= 0) {
            const int64_t base = (((int64_t)blk * a.block_size + c0 % a.block_size) * a.hkv + gs) * D;
            const bf16 *src = (const bf16 *)(is_v ? a.v_cache : a.k_cache) + base;
            const uint32_t lds0 = is_v ? vbuf_lds : kbuf_lds;
            const int last = kend - 1 - c0;
#pragma unroll
            for (int i = 0; i < VI; ++i) {
                const int row = 4 * i + gq;
                const uint32_t roff = (uint32_t)min(row, last) * row_bytes;
                const int sw = is_v ? swz_dv(row) : swz_dk(row);
                lds_dma16(src, roff + (uint32_t)((n ^ sw) * 16), lds0 + i * 4 * D * 2);
            }
        } else {
#pragma unroll
            for (int i = 0; i < VI; ++i) st16(buf + (4 * i + gq) * D + 8 * n, make_uint4(0, 0, 0, 0));
        }
    };

    // one chunk whose K and V have been issued; if `more`, issues the loads
    // of the next chunk (key c1 of a segment ending at kend1, block blk1) as
    // soon as the buffers are read
    auto chunk = [&](int c0, int kend, bool more, int c1, int kend1, int blk1) ATTN_INLINE {
        // this chunk's K and V rows have landed
        wait_all();
        wave_sync_lds();
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
        // V^T operands by transposing reads: for MFMA (jj, db) a lane holds
        // 8 keys of one d, the key order matching P's
        T8 vf[JJ][DB];
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int r0 = 32 * jj + 4 * gq + (n >> 2);
                const int col = 16 * db + 4 * (n & 3);
                const int ch = col >> 3, sub = col & 7;
                const bf16 *p0 = vbuf + r0 * D + ((ch ^ swz_dv(r0)) * 8) + sub;
                const bf16 *p1 = vbuf + (r0 + 16) * D + ((ch ^ swz_dv(r0 + 16)) * 8) + sub;
                const T4 lo = ds_read_tr4<T>(p0);
                const T4 hi = ds_read_tr4<T>(p1);
                vf[jj][db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        // both buffers are read: the next chunk's loads go out now and stay
        // in flight while this chunk is computed
        wait_lgkm();
        wave_sync_lds();
        // the heads of the workgroup request the next chunk's rows together
        // (measured +1.4 %: the cache rows of one key are read close in time)
        if (sync_waves) __syncthreads();
        if (more) {
            issue(false, c1, kend1, blk1);
            issue(true, c1, kend1, blk1);
        }
        // S^T = K Q^T
        f32x4 sacc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            sacc[mb] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                sacc[mb] = mfma_16x16x32(*reinterpret_cast<T8 *>(&kr[mb][kk]), qf[kk], sacc[mb]);
        }
        // mask keys past the segment end: lane holds keys 16mb + 4gq + i
        const int last = kend - 1 - c0;
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
        T8 pb[JJ];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the row sum takes the rounded weight, the one P V uses
                const T p = to16<T>(fast_exp2(fmaf(sacc[mb][i], cl, -mc_new)));
                psum += (float)p;
                pb[mb >> 1][4 * (mb & 1) + i] = p;
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
            for (int db = 0; db < DB; ++db)
                o[db] = mfma_16x16x32(vf[jj][db], pb[jj], o[db]);
    };

    // merge the waves' states of one head (wpH waves per head) for the
    // segment of sequence b in this run; write its partial at slot r + b
    auto write_partial = [&](int bb) ATTN_INLINE {
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
        for (int p = 0; p < wpH; ++p) M = fmaxf(M, sMerge[p * HB + hl][n][0]);
        const float myscale = (mlog == kNegInf) ? 0.f : fast_exp2(mlog - M);
        // O^T layout: lane holds query n, d = 16db + 4gq + i
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sO[(w * 16 + n) * D + 16 * db + 4 * gq + i] = o[db][i] * myscale;
        __syncthreads();
        // threads (head hl, query qi, d) sum their head's waves and write
        const int64_t slot = (int64_t)r + bb;
        for (int e = tid; e < HB * group * D; e += kDecThreads) {
            const int d = e % D, hq_i = e / D;
            const int qi = hq_i % group, h_l = hq_i / group;
            const int gg = hb * HB + h_l;
            if (gg >= a.hkv) continue;
            float Mq = kNegInf;
            for (int p = 0; p < wpH; ++p) Mq = fmaxf(Mq, sMerge[p * HB + h_l][qi][0]);
            float acc = 0.f, lsum = 0.f;
            for (int p = 0; p < wpH; ++p) {
                const int ww = p * HB + h_l;
                acc += sO[(ww * 16 + qi) * D + d];
                const float mw = sMerge[ww][qi][0];
                lsum += (mw == kNegInf) ? 0.f : sMerge[ww][qi][1] * fast_exp2(mw - Mq);
            }
            const int64_t row = slot * a.hq + gg * group + qi;
            a.ws_o[row * D + d] = acc;
            if (d == 0) {
                a.ws_ml[row * 2] = Mq;
                a.ws_ml[row * 2 + 1] = lsum;
            }
        }
        __syncthreads();   // sO (the V buffers) and sMerge are free again
    };

    // one wavefront per head (wpH == 1): it holds the head's whole state, so
    // its partial goes out straight from registers (the same values the
    // merge above writes for a single wave), and the next segment's first
    // chunk is requested before that, with the last chunk of this one
    auto write_partial_direct = [&](int bb) ATTN_INLINE {
        float lsum_w = l_run;
        lsum_w += __shfl_xor(lsum_w, 16, 64);
        lsum_w += __shfl_xor(lsum_w, 32, 64);
        const bool none = m_run == kNegInf;
        const float sc = none ? 0.f : 1.f;
        if (qv) {
            const int64_t row = ((int64_t)r + bb) * a.hq + g * group + n;
            float *op = a.ws_o + row * D + 4 * gq;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<float4 *>(op + 16 * db) =
                    make_float4(o[db][0] * sc, o[db][1] * sc, o[db][2] * sc, o[db][3] * sc);
            if (gq == 0) {
                a.ws_ml[row * 2] = none ? kNegInf : mc_run;
                a.ws_ml[row * 2 + 1] = none ? 0.f : lsum_w;
            }
        }
    };
    const bool direct = wpH == 1;

    int L = seq_len(b);
    // item counts and item ends in 64 bits: S may be as large as the caller's
    // item size allows (any positive multiple of 32)
    int ns = (int)(((int64_t)L + S - 1) / S);
    bool pre = false;   // this segment's first chunk went out with the last one of the previous
    for (int it = 0; it < n_items;) {
        // segment: items s .. s + cnt - 1 of sequence b
        const int cnt = min(ns - s, n_items - it);
        const int kbeg = s * S, kend = (int)min((int64_t)L, (int64_t)(s + cnt) * S);
        if (hb == 0 && tid == 0) {
            if (s == 0) a.ws_runs[2 * b] = r;
            if (s + cnt == ns) a.ws_runs[2 * b + 1] = r;
        }
        // the next segment: the next sequence with items, from its first item
        const int itn = it + cnt;
        int bn = b, Ln = 0, nsn = 0;
        if (itn < n_items) {
            do {
                ++bn;
                Ln = bn < a.batch ? seq_len(bn) : 0;
                nsn = (int)(((int64_t)Ln + S - 1) / S);
            } while (nsn == 0 && bn < a.batch);
        }
        const bool has_next = itn < n_items && bn < a.batch;
        const int kendn = has_next ? (int)min((int64_t)Ln, (int64_t)min(nsn, n_items - itn) * S) : 0;
        m_run = kNegInf;
        mc_run = 0.f;
        l_run = 0.f;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] = f32x4{};
        int c0 = kbeg + kChunk * ph;
        if (active && c0 < kend) {
            {
                const int head = g * group + (qv ? n : 0);
                const bf16 *qp = (const bf16 *)a.q + ((int64_t)b * a.hq + head) * D + 8 * gq;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    uint4 t = qv ? ld16(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
                    qf[kk] = *reinterpret_cast<T8 *>(&t);
                }
            }
            if (!pre) {
                const int blk0 = blk_of(b, c0);
                issue(false, c0, kend, blk0);
                issue(true, c0, kend, blk0);
            }
            for (;;) {
                const int c1 = c0 + kChunk * wpH;
                if (c1 < kend) {
                    chunk(c0, kend, true, c1, kend, blk_of(b, c1));
                    c0 = c1;
                    continue;
                }
                const bool pf = direct && has_next;
                chunk(c0, kend, pf, 0, kendn, pf ? blk_of(bn, 0) : 0);
                break;
            }
        }
        if (direct) {
            if (active) write_partial_direct(b);
        } else {
            write_partial(b);
        }
        pre = direct && has_next;
        it = itn;
        if (it < n_items) {
            if (!has_next) break;
            b = bn;
            L = Ln;
            ns = nsn;
            s = 0;
        }
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(D)
decode_combine_kernel(DecodeArgs a) {
    constexpr int kBatchLoads = 8;  // partials read together (a sequence spans few runs)
    const int bh = blockIdx.x;  // b * hq + h
    const int b = bh / a.hq;
    const int d = threadIdx.x;
    // the length and the runs that hold keys of b, read together (the runs
    // are not posted for an empty sequence and are then ignored)
    const int L = ld_meta(a.cache_seqlens, b);
    int r0 = ld_meta(a.ws_runs, 2 * b);
    int r1 = ld_meta(a.ws_runs, 2 * b + 1);
    r0 = r0 < 0 ? 0 : r0;
    r1 = r1 >= a.n_runs ? a.n_runs - 1 : r1;
    if (L <= 0) {
        r0 = 0;
        r1 = -1;
    }
    float M = kNegInf, acc = 0.f, lsum = 0.f;
    for (int rb = r0; rb <= r1; rb += kBatchLoads) {
        float ms[kBatchLoads], ls[kBatchLoads], os[kBatchLoads];
#pragma unroll
        for (int i = 0; i < kBatchLoads; ++i) {
            ms[i] = kNegInf;
            ls[i] = 0.f;
            os[i] = 0.f;
            if (rb + i <= r1) {
                const int64_t row = ((int64_t)rb + i + b) * a.hq + (bh - b * a.hq);
                ms[i] = a.ws_ml[row * 2];
                ls[i] = a.ws_ml[row * 2 + 1];
                os[i] = a.ws_o[row * D + d];
            }
        }
#pragma unroll
        for (int i = 0; i < kBatchLoads; ++i) {
            if (ms[i] != kNegInf) {
                const float Mn = fmaxf(M, ms[i]);
                const float fo = (M == kNegInf) ? 0.f : fast_exp2(M - Mn);
                const float fs = fast_exp2(ms[i] - Mn);
                acc = acc * fo + os[i] * fs;
                lsum = lsum * fo + ls[i] * fs;
                M = Mn;
            }
        }
    }
    const float res = lsum > 0.f ? acc / lsum : 0.f;
    if (a.out_f32)
        ((float *)a.o)[(int64_t)bh * D + d] = res;
    else
        ((T *)a.o)[(int64_t)bh * D + d] = to16<T>(res);
}

}  // namespace

// Scratch of the allocation-free decode entry point: the decode workspace
// (partials, (m, d') pairs, first/last runs) in a file-scope device array.
// Each GPU the library runs on holds its own copy until the process ends.
// Host code must never pass `scratch` itself to a kernel (in host code the
// name is a host-side stand-in): decode_scratch() looks up its address on the
// current device once and caches it per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // the device is current: its copy of the array is the one resolved
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

int decode_runs(int hkv, int cus) {
    const int hb = heads_per_block(hkv);
    const int nb = (hkv + hb - 1) / hb;
    int runs = (cus > 0 ? cus : 1) / nb;
    if (runs < 1) runs = 1;
    if (runs > kDecodeMaxRuns) runs = kDecodeMaxRuns;
    return runs;
}

template <typename T>
hipError_t launch_decode_typed(const DecodeArgs &a, hipStream_t stream) {
    constexpr int D = 128;
    if (a.batch == 0) return hipSuccess;
    const int hb = heads_per_block(a.hkv);
    const int nb = (a.hkv + hb - 1) / hb;
    // one persistent workgroup per (run, head block)
    const int64_t grid = (int64_t)a.n_runs * nb;
    hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3((unsigned)grid), dim3(kDecThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.batch * a.hq)), dim3(D), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    return a.in_f16 ? launch_decode_typed<f16>(a, stream) : launch_decode_typed<bf16>(a, stream);
}

}  // namespace attn
