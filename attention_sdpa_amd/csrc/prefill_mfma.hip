// prefill_mfma.hip -- fused varlen causal prefill on the gfx950 matrix cores,
// for bf16 or fp16 inputs (the kernel is a template on the 16-bit type; P
// is rounded to the same type for the P V product).
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
// * Work units are (sequence, block of query positions, KV head g) with the
//   (up to 4) query heads of g's GQA group, so every K/V tile brought into
//   LDS serves 256 query rows; each wavefront owns one query head and 32
//   consecutive positions.  The kernel is persistent: one 8-wavefront
//   workgroup per CU walks its share of the units (heaviest first), and its
//   K/V tile stream runs on across unit boundaries, so that a unit costs no
//   launch, no pipeline fill and no exposed load latency.
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
// * Two groups of four wavefronts (one wave of each group per SIMD) run a
//   ping-pong: while one group runs its matrix phase (the next tile's S^T and
//   this tile's P V, MFMA after MFMA with LDS operand reads two steps
//   ahead), the other computes a softmax on the vector ALUs; a workgroup
//   barrier separates the half-steps.  The last 6 of a matrix phase's 16
//   P V MFMAs are issued at the start of the wave's next softmax phase,
//   when its partner on the SIMD is issuing its tile loads and the matrix
//   core would otherwise wait.
// * K/V tiles reach LDS by direct global->LDS loads (global_load_lds_dwordx4,
//   no register staging) into rings of three stages.  The group entering its
//   matrix phase issues them (one group all K tiles, the other all V tiles),
//   so the softmax group issues no memory instructions.  16-byte chunks are
//   XOR-swizzled (the swizzle is applied by choosing which global chunk each
//   lane fetches) so that the operand reads are free of bank conflicts.
// * Unit boundaries: the last step of a unit forms P V only (no S^T is
//   needed), and each group loads the next unit's Q rows right after it; the
//   group then writes its O in the half-step its softmax would have taken,
//   while the other group is in its matrix phase, and forms the next unit's
//   first S^T one half-step later.  The O stores are buffer stores against a
//   resource spanning the unit's valid rows (rows past the sequence end are
//   dropped), 8 per wave after one exchange of the lane halves, so the wait
//   counts that follow are exact.
// * Causal: tiles past the last visible key are never loaded; only tiles
//   that cross the diagonal (or the sequence end) are masked.  Work units are
//   dealt heaviest first (by K/V tile count) and the KV head is the
//   fastest-varying index, so that each XCD keeps reusing few heads' K/V in
//   its L2.
// * Exponentials in base 2 with c = s*log2(e): p = 2^(fma(x, c, -r*c)) for a
//   per-row reference r.  r follows the running maximum lazily: it is raised
//   (and o', d' rescaled by 2^(r_old*c - r_new*c), the same rounded
//   products) only when the scaled maximum exceeds the scaled reference by
//   more than 8 (x*c - r*c > 8), which keeps p <= 256 and leaves the result
//   unchanged in exact arithmetic.
// * Row sums are accumulated from the bf16-rounded P with v_dot2_f32_bf16,
//   i.e. from exactly the weights the P V product uses.
#include <type_traits>

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

// x = -inf when key offset c >= thr: one compare and one select per key.
// (Written as asm: the compiler otherwise turns the 16 compares of a block,
// whose constants increase, into a serial chain of scalar ORs.)
__device__ __forceinline__ float mask_key(float x, int thr, int c) {
    asm("v_cmp_le_i32 vcc, %1, %2\n\t"
        "v_cndmask_b32 %0, %0, %3, vcc"
        : "+v"(x)
        : "v"(thr), "i"(c), "v"(kNegInf)
        : "vcc");
    return x;
}

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
constexpr int kWaitVm12 = 0x007C;
constexpr int kWaitVm16 = 0x4070;   // vmcnt bits 5:4 live in bits 15:14
constexpr int kWaitVm20 = 0x4074;
constexpr int kWaitNone = 0xC07F;   // vmcnt 63: no memory wait (LDS and scalar: lgkmcnt 0)

// Buffer resource word 3 for raw (unformatted, unswizzled) buffer access.
constexpr int kBufferFlags = 0x00020000;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

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

// ---- work units and their schedule --------------------------------------
//
// A unit is (sequence b, query block qt, head chunk hc, KV head g): the
// pos_per_wg query positions from qt * pos_per_wg of the hpw query heads
// (chunk hc of g's GQA group) that read KV head g.  Its cost is its number
// of K/V tiles (under the causal mask it grows with qt, and with the
// sequence's cached prefix).  Units are sorted by cost, heaviest first: row
// r holds the units of cost nct-1-r, (sequence, query block) pairs in
// (b, qt) order, each with its head_chunks * hkv units, g fastest.  Unit u
// of that order goes to workgroup snake(u): round u / grid, position
// u % grid, reversed in odd rounds -- the greedy assignment for rounds of
// near-equal-cost units.  Every workgroup derives its own list from
// cu_seqlens_q/k at start ("listed" schedule).  Where the sizes exceed the tables below, workgroup i instead
// takes slots i, i + grid, ... of the padded (qt, b, hc, g) slot grid
// ("strided" schedule), which is correct for any size but less balanced.

constexpr int kMaxBatchListed = 1024;   // sequences
constexpr int kMaxRowsListed = 4096;    // query blocks per sequence; cost buckets
constexpr int kMaxUnitsListed = 2048;   // units per workgroup

struct Geo {
    int nqt;            // query-position blocks per sequence (upper bound)
    int nct;            // listed schedule: cost buckets (64-key tile counts 0 .. nct-1)
    int hpw;            // query heads per wave column
    int head_chunks;    // group / hpw
    int pos_per_wg;     // query positions per unit
    int lg, lhc, lb;    // strided schedule: log2 of G2, HC2, B2 (powers of
    int slots;          // two at or above hkv, head_chunks, batch); slot count
};

// Bounds of sequence b, clamped as the interface promises.
struct SeqMeta {
    int q0, Lq, k0, Lk;
};

__device__ __forceinline__ SeqMeta seq_meta(const VarlenArgs &a, int b) {
    SeqMeta m;
    if (a.pad_q) {   // padded batch: rows b * pad_q .., seqlens_q[b] of them
        const int L = ld_meta(a.seqlens_q, b);
        m.q0 = b * a.pad_q;
        m.Lq = L < 0 ? 0 : (L > a.pad_q ? a.pad_q : L);
    } else {
        int q0 = ld_meta(a.cu_q, b), q1 = ld_meta(a.cu_q, b + 1);
        q0 = q0 < 0 ? 0 : (q0 > a.total_q ? (int)a.total_q : q0);
        q1 = q1 < q0 ? q0 : (q1 > a.total_q ? (int)a.total_q : q1);
        m.q0 = q0;
        m.Lq = q1 - q0;
    }
    if (a.pad_q) {
        const int L = ld_meta(a.seqlens_k, b);
        m.k0 = b * a.pad_k;
        m.Lk = L < 0 ? 0 : (L > a.pad_k ? a.pad_k : L);
        return m;
    }
    int k0 = ld_meta(a.cu_k, b), k1 = ld_meta(a.cu_k, b + 1);
    if (a.block_table) {
        k1 = k1 < k0 ? k0 : k1;
        const int cap = a.max_blocks_per_seq * a.block_size;
        m.Lk = (k1 - k0) > cap ? cap : (k1 - k0);
        m.k0 = 0;
    } else {
        k0 = k0 < 0 ? 0 : (k0 > a.total_k ? (int)a.total_k : k0);
        k1 = k1 < k0 ? k0 : (k1 > a.total_k ? (int)a.total_k : k1);
        m.k0 = k0;
        m.Lk = k1 - k0;
    }
    return m;
}

// One work unit (wave-uniform values).
struct Unit {
    int k;              // position in this workgroup's schedule
    int valid;          // 0 once past the last unit
    int b, g, hc, qt;
    int q0, k0, Lq, Lk;
    int p0;             // first query position of the unit
    int kv_end;         // keys [0, kv_end) are visible to some row of the unit
    int n_tiles;        // ceil(kv_end / kBN)
};

__device__ __forceinline__ void unit_bounds(const VarlenArgs &a, const Geo &geo, Unit &u, const SeqMeta &m) {
    u.q0 = m.q0;
    u.Lq = m.Lq;
    u.k0 = m.k0;
    u.Lk = m.Lk;
    u.p0 = u.qt * geo.pos_per_wg;
    const int last = min(u.p0 + geo.pos_per_wg, u.Lq) - 1;
    u.kv_end = a.causal ? max(0, min(u.Lk, last + (u.Lk - u.Lq) + 1)) : u.Lk;
    u.n_tiles = (u.kv_end + kBN - 1) / kBN;
}

// Cost of the listed schedule's unit (query block qt of a sequence with Lq
// queries and Lk keys, P query positions per unit): its number of 64-key
// tiles, as unit_bounds counts them, with the per-sequence tile count
// clamped to nct - 1 (the histogram's range).  Under the end-aligned causal
// mask block qt < nq - 1 sees keys [0, P (qt + 1) + Lk - Lq), so its cost is
// s (qt + 1) + e clamped to [0, Tk] with s = P / 64, e = ceil((Lk - Lq) / 64),
// Tk = ceil(Lk / 64); the last block sees every key.
__device__ __forceinline__ int ceil_div_signed(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }

__device__ __forceinline__ int unit_cost(int causal, int Lq, int Lk, int qt, int P, int nct) {
    const int nq = (Lq + P - 1) / P;
    const int Tk = min((Lk + kBN - 1) / kBN, nct - 1);
    if (!causal || qt == nq - 1) return Tk;
    const int v = (P / kBN) * (qt + 1) + ceil_div_signed(Lk - Lq, kBN);
    return v < 0 ? 0 : (v > Tk ? Tk : v);
}

// The query blocks of one sequence whose unit_cost is c: cnt of them,
// starting at block first (they are contiguous).
__device__ __forceinline__ void unit_cost_range(int causal, int Lq, int Lk, int c, int P, int nct, int &cnt,
                                                int &first) {
    cnt = 0;
    first = 0;
    const int nq = (Lq + P - 1) / P;
    if (nq <= 0) return;
    const int Tk = min((Lk + kBN - 1) / kBN, nct - 1);
    if (!causal || Tk == 0) {
        if (c == Tk) cnt = nq;
        return;
    }
    const int s = P / kBN, e = ceil_div_signed(Lk - Lq, kBN);
    if (c == Tk) {
        int qT = ceil_div_signed(Tk - e, s) - 1;
        qT = qT < 0 ? 0 : (qT > nq - 1 ? nq - 1 : qT);
        cnt = nq - qT;
        first = qT;
    } else if (c == 0) {
        int n0 = e <= 0 ? (-e) / s : 0;
        cnt = n0 > nq - 1 ? nq - 1 : n0;
    } else if (c > 0 && c < Tk && (c - e) % s == 0) {
        const int qt = (c - e) / s - 1;
        if (qt >= 0 && qt <= nq - 2) {
            cnt = 1;
            first = qt;
        }
    }
}

// Strided schedule: the first unit at or after slot counter k (with rows;
// with tiles too if need_tiles).
__device__ __forceinline__ Unit find_unit_strided(const VarlenArgs &a, const Geo &geo, int k, bool need_tiles) {
    Unit u;
    for (;; ++k) {
        const int slot = (int)blockIdx.x + k * (int)gridDim.x;
        u.k = k;
        if (slot >= geo.slots) {
            u.valid = 0;
            u.n_tiles = 0;
            return u;
        }
        u.g = slot & ((1 << geo.lg) - 1);
        u.hc = (slot >> geo.lg) & ((1 << geo.lhc) - 1);
        u.b = (slot >> (geo.lg + geo.lhc)) & ((1 << geo.lb) - 1);
        u.qt = geo.nqt - 1 - (slot >> (geo.lg + geo.lhc + geo.lb));
        if (u.g >= a.hkv || u.hc >= geo.head_chunks || u.b >= a.batch) continue;   // padding
        const SeqMeta m = seq_meta(a, u.b);
        if (u.qt * geo.pos_per_wg >= m.Lq) continue;     // no query rows here
        unit_bounds(a, geo, u, m);
        if (need_tiles && u.n_tiles == 0) continue;
        u.valid = 1;
        return u;
    }
}

// Listed schedule: the first list entry at or after k (with tiles if
// need_tiles).  Entries: (b, qt << 16 | hc << 8 | g); meta: (q0, Lq, k0, Lk).
__device__ __forceinline__ Unit find_unit_listed(const VarlenArgs &a, const Geo &geo, const int2 *list,
                                                 const int4 *meta, int n_mine, int k, bool need_tiles) {
    Unit u;
    for (;; ++k) {
        u.k = k;
        if (k >= n_mine) {
            u.valid = 0;
            u.n_tiles = 0;
            return u;
        }
        const int2 e = list[k];
        u.b = __builtin_amdgcn_readfirstlane(e.x);
        const int pk = __builtin_amdgcn_readfirstlane(e.y);
        u.qt = pk >> 16;
        u.hc = (pk >> 8) & 255;
        u.g = pk & 255;
        const int4 mm = meta[u.b];
        SeqMeta m;
        m.q0 = __builtin_amdgcn_readfirstlane(mm.x);
        m.Lq = __builtin_amdgcn_readfirstlane(mm.y);
        m.k0 = __builtin_amdgcn_readfirstlane(mm.z);
        m.Lk = __builtin_amdgcn_readfirstlane(mm.w);
        unit_bounds(a, geo, u, m);
        if (need_tiles && u.n_tiles == 0) continue;
        u.valid = 1;
        return u;
    }
}

// The K/V load cursor: the next tile of the tile stream to be loaded.
struct KvCursor {
    int k, valid;
    int t, n_tiles, kv_end, g;
    int tok;            // contiguous K/V: key row of the tile's first key
    int bt_row;         // paged: b * max_blocks_per_seq
    int bt_i;           // paged: block-table index of the tile
    int in_blk;         // paged: the tile's offset inside its block
    int blk;            // paged: the tile's block id (validated)
    const bf16 *src;    // this wave's tensor at the tile's first key, head g
};

// Per-wave view of a unit: the query head, this lane's query position and
// its visible-key limit, and the tile counts of this wave's rows.
struct WaveView {
    int head;        // query head of this wave
    int pos;         // this lane's query position in the sequence
    int lim;         // keys j < lim are visible to this lane's row (0: none)
    int w_kv_full;   // every row of the wave sees all keys below this
    int nw;          // tiles with at least one visible key for the wave
    bool row_valid;
};

template <typename T, bool kListed, bool kPaged>
__global__ void __launch_bounds__(kThreads, 1)
prefill_mfma_kernel(VarlenArgs a, Geo geo) {
    typedef typename Vec16<T>::x2 T2;
    typedef typename Vec16<T>::x4 T4;
    typedef typename Vec16<T>::x8 T8;
    constexpr int KK = kD / 16;         // MFMA k-steps over head_dim
    constexpr int DB = kD / 32;         // 32-row blocks of d in O^T
    constexpr int kStageBytes = kTileElems * 2;
    // three-stage rings: stage i of K is sK[i], of V is sV[i]
    __shared__ __align__(16) bf16 sK[3][kTileElems];
    __shared__ __align__(16) bf16 sV[3][kTileElems];
    // listed schedule: per-sequence bounds, row prefix counts, unit list
    __shared__ int4 sMeta[kListed ? kMaxBatchListed : 1];
    __shared__ int sRows[kListed ? kMaxRowsListed : 1];
    __shared__ int2 sList[kListed ? kMaxUnitsListed : 1];
    __shared__ int sWaveSum[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // group A opens each step with its matrix phase.  Waves w and w + 4
    // share a SIMD and the older wave wins issue ties, so the younger waves
    // lead: measured, that order costs the pair less.
    const bool grpA = w >= 4;
    const int group = a.hq / a.hkv;
    const int n = lane & 31;                           // this lane's query
    const int hf = lane >> 5;                          // lane half
    const float cl = a.scale_log2;
    const int dr = lane >> 4, dc = lane & 15;
    constexpr bool paged = kPaged;                         // K/V through the block table

    // ---- listed schedule: this workgroup's units --------------------------
    // Units are sorted by cost (their K/V tile count), heaviest first, and
    // dealt to workgroups in a snake.  The cost of (sequence b, query block
    // qt) is closed-form (see unit_cost); within one sequence the blocks of
    // a given cost form a contiguous range (unit_cost_range), so the sort is
    // a counting sort: a histogram over cost, two scans, and a closed-form
    // lookup of each unit.  Row r of the histogram holds cost nct - 1 - r.
    int n_mine = 0;
    if constexpr (kListed) {
        const int nqt = geo.nqt, P = geo.pos_per_wg, nct = geo.nct;
        const int hcg = geo.head_chunks * a.hkv;
        for (int b = tid; b < a.batch; b += kThreads) {
            const SeqMeta m = seq_meta(a, b);
            sMeta[b] = make_int4(m.q0, m.Lq, m.k0, m.Lk);
        }
        for (int r = tid; r < nct; r += kThreads) sRows[r] = 0;
        __syncthreads();
        // histogram of pair costs: pairs (qt, b) flattened, b fastest
        for (int i = tid; i < nqt * a.batch; i += kThreads) {
            const int qt = i / a.batch, b = i - qt * a.batch;
            const int4 mm = sMeta[b];
            if (qt * P < mm.y) atomicAdd(&sRows[nct - 1 - unit_cost(a.causal, mm.y, mm.w, qt, P, nct)], 1);
        }
        __syncthreads();
        // one inclusive scan: pairs in rows <= r
        constexpr int kPer = kMaxRowsListed / kThreads;
        {
            int v[kPer];
            int sum = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int r = tid * kPer + i;
                sum += (r < nct) ? sRows[r] : 0;
                v[i] = sum;
            }
            int x = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            if (lane == 63) sWaveSum[w] = x;
            __syncthreads();
            int excl = x - sum;
            for (int j = 0; j < w; ++j) excl += sWaveSum[j];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int r = tid * kPer + i;
                if (r < nct) sRows[r] = v[i] + excl;
            }
            __syncthreads();
        }
        // units in rows < r: hcg * sRows[r - 1]
        const int grid = (int)gridDim.x, wg = (int)blockIdx.x;
        const int u_total = hcg * sRows[nct - 1];
        const int rounds = u_total / grid, rem = u_total - rounds * grid;
        n_mine = rounds + ((((rounds & 1) ? grid - 1 - wg : wg) < rem) ? 1 : 0);
        // the launch bounds the unit count so that the list fits; never write past it
        n_mine = min(n_mine, kMaxUnitsListed);
        for (int k = w; k < n_mine; k += kWaves) {
            const int u = k * grid + ((k & 1) ? grid - 1 - wg : wg);
            int lo = 0, hi = nct - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (hcg * __builtin_amdgcn_readfirstlane(sRows[mid - 1]) <= u) lo = mid;
                else hi = mid - 1;
            }
            const int j = u - (lo ? hcg * __builtin_amdgcn_readfirstlane(sRows[lo - 1]) : 0);
            const int bi = j / hcg, rm = j - bi * hcg;
            const int c = nct - 1 - lo;
            // the bi-th pair of cost c, in (b, qt) order
            int seen = 0, bsel = 0, qsel = 0;
            for (int b0 = 0; b0 < a.batch; b0 += 64) {
                const int b = b0 + lane;
                int cnt = 0, first = 0;
                if (b < a.batch) {
                    const int4 mm = sMeta[b];
                    unit_cost_range(a.causal, mm.y, mm.w, c, P, nct, cnt, first);
                }
                int x = cnt;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int y = __shfl_up(x, off, 64);
                    if (lane >= off) x += y;
                }
                const int tot = __shfl(x, 63, 64);
                if (bi < seen + tot) {
                    const uint64_t hit = __builtin_amdgcn_ballot_w64(seen + x > bi);
                    const int l = (int)__builtin_ctzll(hit);
                    bsel = b0 + l;
                    qsel = __shfl(first, l, 64) + (bi - seen - (__shfl(x, l, 64) - __shfl(cnt, l, 64)));
                    break;
                }
                seen += tot;
            }
            const int g = rm % a.hkv, hc = rm / a.hkv;
            if (lane == 0) sList[k] = make_int2(bsel, (qsel << 16) | (hc << 8) | g);
        }
        __syncthreads();
    }
    auto find_unit = [&](int k, bool need_tiles) ATTN_INLINE {
        if constexpr (kListed) return find_unit_listed(a, geo, sList, sMeta, n_mine, k, need_tiles);
        else return find_unit_strided(a, geo, k, need_tiles);
    };

    auto wave_view = [&](const Unit &u) ATTN_INLINE {
        WaveView v;
        v.head = u.g * group + u.hc * geo.hpw + (w % geo.hpw);
        const int wp0 = u.p0 + kRowsPerWave * (w / geo.hpw);
        v.pos = wp0 + n;
        v.row_valid = v.pos < u.Lq;
        const int off = u.Lk - u.Lq;
        const int wlast = min(wp0 + kRowsPerWave, u.Lq) - 1;
        const int w_kv_end = (wp0 < u.Lq) ? (a.causal ? max(0, min(u.Lk, wlast + off + 1)) : u.Lk) : 0;
        v.w_kv_full = a.causal ? max(0, min(u.Lk, wp0 + off + 1)) : u.Lk;
        v.lim = v.row_valid ? (a.causal ? min(u.Lk, v.pos + off + 1) : u.Lk) : 0;
        v.nw = (w_kv_end + kBN - 1) / kBN;
        return v;
    };

    // ---- direct global -> LDS loads of the K and V tiles --------------------
    // Group B loads every K tile and group A every V tile, each during its
    // own matrix phase, so the group busy with the softmax issues no memory
    // instructions.  Wave w' = w mod 4 of a group fills tile rows 16w' ..
    // 16w'+15 with four 1 KiB loads; lane l lands at physical chunk (l & 15)
    // of row 16w' + 4i + (l >> 4) and fetches the logical chunk that the
    // tensor's swizzle puts there.  Rows past the unit's last needed key
    // repeat that key (finite data; those keys are masked).
    const int wq = w & 3;
    const bf16 *my_src = grpA ? (const bf16 *)a.v : (const bf16 *)a.k;
    const uint32_t my_lds0 = (grpA ? lds_addr(&sV[0][0]) : lds_addr(&sK[0][0])) + 16 * wq * kD * 2;
    const uint32_t row_bytes = (uint32_t)a.hkv * kD * 2;
    const int rr0 = 16 * wq + dr;                          // this lane's rows: rr0 + 4i
    uint32_t chk[4], full[4];                              // chunk offsets; full-tile offsets
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rr0 + 4 * i;
        chk[i] = (dc ^ (grpA ? swz_v(r) : swz_k(r))) * 16;
        full[i] = r * row_bytes + chk[i];
    }

    // ---- the K/V tile stream ----------------------------------------------
    // Stream position s runs over the tiles of this workgroup's units one
    // after another; its ring stage is s mod 3.  In the ping-pong schedule
    // below, step s holds the matrix half-steps that read V(s) and K(s+1)
    // (group A's after the even barrier E_s, group B's after the odd
    // barrier O_s).  Group A loads V(s+2) in its matrix phase of step s and
    // group B loads K(s+3) in its matrix phase of step s: the stages they
    // overwrite were last read in step s-1.  Each group waits for its own
    // loads at even barriers only: at E_s, A for V(s) and B for K(s+1).
    Unit C = find_unit(0, false);                          // compute cursor
    auto skip_empty = [&](Unit &C) ATTN_INLINE {           // units with rows but no key: zeros
        while (C.valid && C.n_tiles == 0) {
            const WaveView v = wave_view(C);
            if (v.row_valid) {
                const int64_t obase = (((int64_t)C.q0 + v.pos) * a.hq + v.head) * (int64_t)kD + 4 * hf;
#pragma unroll
                for (int c = 0; c < kD; c += 8) {
                    if (a.out_f32) *reinterpret_cast<float4 *>((float *)a.o + obase + c) = make_float4(0.f, 0.f, 0.f, 0.f);
                    else *reinterpret_cast<uint2 *>((bf16 *)a.o + obase + c) = make_uint2(0u, 0u);
                }
            }
            C = find_unit(C.k + 1, false);
        }
    };
    skip_empty(C);
    if (!C.valid) return;

    auto load_blk = [&](int idx) ATTN_INLINE {
        const int blk = ld_meta(a.block_table, idx);
        return (blk >= 0 && blk < a.num_blocks) ? blk : 0;   // bad id: stay in bounds
    };
    KvCursor KU;                                           // this wave's load cursor
    auto set_src = [&]() ATTN_INLINE {
        const int tok = paged ? KU.blk * a.block_size + KU.in_blk : KU.tok;
        KU.src = my_src + ((int64_t)tok * a.hkv + KU.g) * (int64_t)kD;
    };
    const int64_t tile_stride = (int64_t)kBN * a.hkv * kD;   // elements between consecutive tiles
    auto cursor_to = [&](const Unit &u) ATTN_INLINE {
        KU.k = u.k;
        KU.valid = u.valid;
        KU.t = 0;
        KU.n_tiles = u.n_tiles;
        KU.kv_end = u.kv_end;
        KU.g = u.g;
        KU.tok = u.k0;
        if (paged && u.valid) {
            KU.bt_row = u.b * a.max_blocks_per_seq;
            KU.bt_i = 0;
            KU.in_blk = 0;
            KU.blk = load_blk(KU.bt_row);
        }
        if (u.valid) set_src();
    };
    cursor_to(C);
    auto advance = [&]() ATTN_INLINE {
        if (++KU.t >= KU.n_tiles) {
            cursor_to(find_unit(KU.k + 1, true));
        } else {
            KU.tok += kBN;
            KU.src += tile_stride;            // the next rows of the same block, or of k/v
            if (paged) {
                KU.in_blk += kBN;
                if (KU.in_blk >= a.block_size) {
                    KU.in_blk = 0;
                    ++KU.bt_i;
                    KU.blk = load_blk(KU.bt_row + KU.bt_i);
                    set_src();
                }
            }
        }
    };
    // Vector-memory operations this wave may leave outstanding at its next
    // waiting barrier: its latest K/V batch, plus any O stores issued after
    // it (the counter retires in issue order).
    int vm_allow = 0;
    int my_stage = 0;                                      // ring stage of this wave's next load
    int last_n = 0;                                        // loads in this wave's latest batch
    auto issue = [&]() ATTN_INLINE {
        last_n = 0;
        if (KU.valid) {
            const int lim = min(kBN - 1, KU.kv_end - 1 - KU.t * kBN);
            const uint32_t lds = my_lds0 + my_stage * kStageBytes;
            if (lim == kBN - 1) {
                lds_dma16x4<4 * kD * 2>(KU.src, full[0], full[1], full[2], full[3], lds);
            } else {
                uint32_t off[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) off[i] = (uint32_t)min(rr0 + 4 * i, lim) * row_bytes + chk[i];
                lds_dma16x4<4 * kD * 2>(KU.src, off[0], off[1], off[2], off[3], lds);
            }
            advance();
            last_n = 4;
        }
        vm_allow = last_n;
        my_stage = (my_stage == 2) ? 0 : my_stage + 1;
    };
    // The wait of this wave's next waiting barrier: the vector-memory
    // operations (vm_allow, below) it may leave outstanding.
    auto wait_barrier = [&]() ATTN_INLINE {
        if (vm_allow == 4) {                               // the steady state: one batch in flight
            stage_barrier<kWaitVm4>();
            return;
        }
        switch (vm_allow) {
            case 4: stage_barrier<kWaitVm4>(); break;
            case 8: stage_barrier<kWaitVm8>(); break;
            case 12: stage_barrier<kWaitVm12>(); break;
            case 16: stage_barrier<kWaitVm16>(); break;
            case 20: stage_barrier<kWaitVm20>(); break;
            default: stage_barrier<kWaitVm0>(); break;
        }
    };
    auto even_barrier = [&]() ATTN_INLINE { wait_barrier(); };
    auto odd_barrier = [&]() ATTN_INLINE { stage_barrier<kWaitNone>(); };
    // stream prologue: group A loads V0, V1; group B loads K0, K1, K2
    issue();
    issue();
    if (!grpA) issue();

    int st = 0;                                            // ring stage of the unit's first tile
    T8 qf[KK];
    f32x16 o[DB];
    float m_ref, mc_ref, l_run;
    f32x16 sacc[2];
    T8 pb[4];
    // P V MFMAs of a step moved into the following softmax phase (measured
    // best of 4..12: the partner wave's load issue leaves the matrix core
    // idle for about that long), their V operands kept in registers
    constexpr int kDefer = 6;
    T8 vkeep[kDefer];
    // Q rows of unit u into qf.  A row past the sequence end reads the
    // sequence's first row instead: finite values confined to its own lane
    // pair, whose output is dropped.
    auto load_q = [&](const Unit &u) ATTN_INLINE {
        const WaveView qv = wave_view(u);
        const bf16 *qp = (const bf16 *)a.q + (((int64_t)u.q0 + (qv.row_valid ? qv.pos : 0)) * a.hq + qv.head) * (int64_t)kD + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 tq = ld16(qp + 16 * kk);
            qf[kk] = *reinterpret_cast<T8 *>(&tq);
        }
    };
    // O = o' / d' of unit u.  Buffer stores against a resource that spans
    // the unit's valid rows: stores of rows past the sequence end fall
    // outside it and are dropped, so every wave issues exactly 8 (bf16) or
    // 16 (fp32) stores.
    auto store_o = [&](const Unit &u, const WaveView &v) ATTN_INLINE {
        float l_tot;
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
            l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int esz = a.out_f32 ? 4 : 2;
        const int rows = min(geo.pos_per_wg, u.Lq - u.p0);
        char *ob = (char *)a.o + ((int64_t)(u.q0 + u.p0) * a.hq) * (int64_t)(kD * esz);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ob, (short)0, rows * a.hq * kD * esz, kBufferFlags);
        const int voff = ((v.pos - u.p0) * a.hq + v.head) * kD * esz;
        if (a.out_f32) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = 32 * db + 8 * a4 + 4 * hf;
                    const u32x4 r = {__float_as_uint(o[db][4 * a4] * inv), __float_as_uint(o[db][4 * a4 + 1] * inv),
                                     __float_as_uint(o[db][4 * a4 + 2] * inv), __float_as_uint(o[db][4 * a4 + 3] * inv)};
                    __builtin_amdgcn_raw_buffer_store_b128(r, rs, voff + 4 * d0, 0, 0);
                }
        } else {
            // lane n holds d = 8m + 0..3 of its row and lane n + 32 holds
            // d = 8m + 4..7; one exchange of the two halves gives each lane 8
            // consecutive d values, so a store covers 32 bytes of each row
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    T4 y, x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        y[e] = to16<T>(o[db][8 * pr + e] * inv);
                        x[e] = to16<T>(o[db][8 * pr + 4 + e] * inv);
                    }
                    const u32x2 yu = *reinterpret_cast<u32x2 *>(&y), xu = *reinterpret_cast<u32x2 *>(&x);
                    const auto s0 = __builtin_amdgcn_permlane32_swap(yu[0], xu[0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(yu[1], xu[1], false, false);
                    const u32x4 r = {s0[0], s1[0], s0[1], s1[1]};
                    __builtin_amdgcn_raw_buffer_store_b128(r, rs, voff + 2 * (32 * db + 16 * pr + 8 * hf), 0, 0);
                }
        }
    };
    load_q(C);
    bool first = true;
    Unit Cn;
    for (;;) {
        // ---- one unit: the ping-pong program on its tiles ----------------
        const WaveView V = wave_view(C);
        const int ntl = C.n_tiles;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] = f32x16{};
        m_ref = kNegInf; mc_ref = 0.f; l_run = 0.f;
        const T2 ones2 = {(T)1.f, (T)1.f};
        const int k_row = perm23(n);
        const int gq = lane >> 4, s16 = lane & 15;
        const int v_row_part = 8 * (gq >> 1) + (s16 >> 2);
        const int v_col_elem = 16 * (gq & 1) + 4 * (s16 & 3);

        // S^T = K Q^T for a 64-key tile (two 32-key blocks) from K stage ks
        auto qk = [&](int ks) ATTN_INLINE {
            const bf16 *Kt = &sK[0][0] + ks * kTileElems;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
                const bf16 *krow = Kt + (32 * kb + k_row) * kD;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int ch = (2 * kk + hf) ^ (lane & 15);
                    const T8 kf = *reinterpret_cast<const T8 *>(krow + ch * 8);
                    sacc[kb] = mfma_32x32x16(kf, qf[kk], sacc[kb]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        };
        // One matrix phase: the next tile's S^T = K Q^T from K stage ks and
        // O^T += V^T P^T for the tile in V stage vs, with the row sums from
        // the same bf16 weights.  The two products alternate MFMA by MFMA;
        // the operands of step i + kAhead are read from LDS during step i.
        // With defer, the last kDefer P V MFMAs only keep their V operands;
        // the step loop issues them after the next barrier.
        auto mma = [&](int ks, int vs, auto with_qk, auto defer) ATTN_INLINE {
            constexpr bool kQK = decltype(with_qk)::value;
            constexpr bool kDef = decltype(defer)::value;
            constexpr int kAhead = 2;   // measured best of 1..5
            const bf16 *Kt = &sK[0][0] + ks * kTileElems;
            const bf16 *Vt = &sV[0][0] + vs * kTileElems;
            T8 kbuf[16], vbuf[16];
            auto read_k = [&](int i) ATTN_INLINE {
                const int kb = i >> 3, kk = i & 7;
                const bf16 *krow = Kt + (32 * kb + k_row) * kD;
                const int ch = (2 * kk + hf) ^ (lane & 15);
                kbuf[i] = *reinterpret_cast<const T8 *>(krow + ch * 8);
            };
            auto read_v = [&](int i) ATTN_INLINE {
                const int jj = i >> 2, db = i & 3;
                const int r = 16 * jj + v_row_part;
                const int col = 32 * db + v_col_elem;
                const int ch0 = col >> 3, sub = col & 7;
                const bf16 *p0r = Vt + r * kD + ((ch0 ^ swz_v(r)) * 8) + sub;
                const bf16 *p1r = Vt + (r + 4) * kD + ((ch0 ^ swz_v(r + 4)) * 8) + sub;
                const T4 lo = ds_read_tr4<T>(p0r);
                const T4 hi = ds_read_tr4<T>(p1r);
                vbuf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
                if constexpr (kQK) read_k(i);
                read_v(i);
            }
            if constexpr (kQK) {
                sacc[0] = f32x16{};
                sacc[1] = f32x16{};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (kQK) {
                    sacc[i >> 3] = mfma_32x32x16(kbuf[i], qf[i & 7], sacc[i >> 3]);
                    if (i + kAhead < 16) read_k(i + kAhead);
                }
                const int jj = i >> 2, db = i & 3;
                if (kDef && i >= 16 - kDefer) vkeep[i - (16 - kDefer)] = vbuf[i];
                else o[db] = mfma_32x32x16(vbuf[i], pb[jj], o[db]);
                if (i + kAhead < 16) read_v(i + kAhead);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // softmax of tile t: mask (diagonal/end tiles only), row max, lazy
        // reference update (rescaling o', d' if it moves), P = 2^(S c - r c)
        // in bf16 -- the B operand of the next P V
        auto softmax = [&](int t) ATTN_INLINE {
            const int t0 = t * kBN;
            if (t0 + kBN > V.w_kv_full) {
                // register i of block kb holds key t0 + 32 kb + 8 hf + c_i,
                // c_i = i (i < 8) or i + 8; it is masked when key >= lim
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int thr = V.lim - t0 - 32 * kb - 8 * hf;
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[kb][i] = mask_key(sacc[kb][i], thr, i < 8 ? i : i + 8);
                }
            }
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            // straight-line (no short-circuit, so no exec-mask branches)
            const bool need = (mx > m_ref) & ((m_ref == kNegInf) | (mx * cl > mc_ref + kRescaleLog2));
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
                    pb[2 * kb + (i >> 3)][i & 7] = to16<T>(fast_exp2(fmaf(sacc[kb][i], cl, -mc_ref)));
        };

        // d' += the row sums of the weights the last P V used (the bf16-rounded
        // ones), at the start of the following softmax phase: there they fill
        // the wait for the matrix phase's last results (measured: 6 % faster
        // than beside the MFMAs, 8 % faster than after the exponentials)
        auto sum_p = [&]() ATTN_INLINE {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    T2 pr;
                    pr[0] = pb[jj][2 * e];
                    pr[1] = pb[jj][2 * e + 1];
                    l_run = dot2_acc(pr, ones2, l_run);
                }
        };
        auto zero_p = [&]() ATTN_INLINE {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) pb[jj] = T8{};
        };

        // ---- prologue: S^T and P of the unit's first tile ------------------
        // The first time, K(s0) and the Q rows are waited for outright.
        // Later units follow their predecessor's last steps directly: each
        // group forms its first S^T in the half-step after its own O stores
        // (the two groups one half-step apart, as in the step loop).
        if (first) {
            stage_barrier<kWaitVm0>();
            if (grpA) qk(st);
            stage_barrier<kWaitNone>();
            if (!grpA) {
                qk(st);
                stage_barrier<kWaitNone>();
            }
        } else {
            // this wave's Q rows, and the K/V batch issued after them, have
            // landed: only the O stores may still be in flight (measured:
            // waiting for the batch here as well, rather than only for the Q
            // rows, is 1.5-2 % faster on the varlen and 32K workloads)
            if (a.out_f32) stage_barrier<kWaitVm16>();
            else stage_barrier<kWaitVm8>();
            qk(st);
            stage_barrier<kWaitNone>();
        }
        // The Q rows have landed (the barriers above waited for them), but the
        // compiler cannot know: its wait tracking counts the Q loads and not
        // the direct-to-LDS K/V loads, which the hardware counter also counts,
        // so it would wait for the Q loads again before the S^T MFMAs of every
        // step -- and in hardware that wait also covers the step's own tile
        // loads, stalling each matrix phase until they land.  Passing the
        // fragments through an empty asm statement ends that tracking.
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qf[kk]));
        if (V.nw > 0) softmax(0);
        else zero_p();
        // ---- all steps but the last ----------------------------------------
        for (int t = 0; t + 1 < ntl; ++t) {
            const int st1 = (st == 2) ? 0 : st + 1;
            if (grpA) even_barrier();
            else odd_barrier();
            __builtin_amdgcn_s_setprio(1);
            // this step's K/V batch first: the stage it refills was last read
            // in the previous step, before the barrier just passed
            issue();
            // every wave runs every step: past its last visible tile its P is
            // zero (adding exactly 0)
            mma(st1, st, std::true_type{}, std::true_type{});
            __builtin_amdgcn_s_setprio(0);
            if (grpA) odd_barrier();
            else even_barrier();
            // the deferred P V MFMAs (same operands, same order per
            // accumulator: the same result bits), while the partner wavefront
            // issues its loads, interleaved with the row sums of the same
            // weights; both precede the softmax that overwrites pb and may
            // rescale o
#pragma unroll
            for (int x = 0; x < kDefer; ++x) {
                const int i = 16 - kDefer + x, jj = i >> 2, db = i & 3;
                o[db] = mfma_32x32x16(vkeep[x], pb[jj], o[db]);
            }
            sum_p();
#pragma unroll
            for (int x = 0; x < kDefer; ++x) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 16 / kDefer, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < V.nw) softmax(t + 1);
            else zero_p();
            st = st1;
        }
        // ---- the last step: P V only, then the next unit's Q rows ----------
        {
            const int st1 = (st == 2) ? 0 : st + 1;
            if (grpA) even_barrier();
            else odd_barrier();
            __builtin_amdgcn_s_setprio(1);
            mma(st1, st, std::false_type{}, std::false_type{});   // nothing deferred: O is stored next
            __builtin_amdgcn_s_setprio(0);
            sum_p();
            Cn = find_unit(C.k + 1, false);
            skip_empty(Cn);
            if (Cn.valid) load_q(Cn);                      // before the batch: the next wait covers it
            issue();
            if (grpA) odd_barrier();
            else even_barrier();
            st = st1;
        }
        // ---- O of this unit, in the half-step its softmax would take --------
        store_o(C, V);
        vm_allow = last_n + (a.out_f32 ? 16 : 8);
        C = Cn;
        if (!C.valid) break;
        first = false;
    }
    if (grpA) stage_barrier<kWaitNone>();                  // B's last half-step
    // no direct-to-LDS load may outlive the workgroup's LDS allocation
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

}  // namespace

template <typename T>
hipError_t launch_prefill_typed(const VarlenArgs &a, hipStream_t stream) {
    const int group = a.hq / a.hkv;
    Geo geo;
    geo.hpw = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
    geo.head_chunks = group / geo.hpw;
    geo.pos_per_wg = kRowsPerWave * (kWaves / geo.hpw);
    geo.nqt = (a.max_seqlen_q + geo.pos_per_wg - 1) / geo.pos_per_wg;
    {
        const int64_t nct = ((int64_t)a.max_seqlen_k + kBN - 1) / kBN + 1;
        geo.nct = (int)(nct < kMaxRowsListed ? nct : kMaxRowsListed);
    }
    auto lg2 = [](int x) { int l = 0; while ((1 << l) < x) ++l; return l; };
    geo.lg = lg2(a.hkv);
    geo.lhc = lg2(geo.head_chunks);
    geo.lb = lg2(a.batch);
    const int64_t slots = (int64_t)geo.nqt << (geo.lg + geo.lhc + geo.lb);
    if (slots == 0) return hipSuccess;
    if (slots > (1LL << 30) || a.total_q > 0x7fffffffLL || a.total_k > 0x7fffffffLL) return hipErrorInvalidValue;
    geo.slots = (int)slots;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus < 1) cus = 1;
    // upper bound of the unit count (every sequence at max_seqlen_q)
    const int64_t units_max = (int64_t)geo.nqt * a.batch * geo.head_chunks * a.hkv;
    const int64_t grid_l = units_max < cus ? units_max : cus;
    const bool listed = a.batch <= kMaxBatchListed && geo.nqt <= kMaxRowsListed && a.hkv <= 256 &&
                        geo.head_chunks <= 256 && (units_max + grid_l - 1) / grid_l <= kMaxUnitsListed;
    const bool paged = a.block_table != nullptr;
    if (listed) {
        if (paged)
            hipLaunchKernelGGL((prefill_mfma_kernel<T, true, true>), dim3((unsigned)grid_l), dim3(kThreads), 0, stream, a, geo);
        else
            hipLaunchKernelGGL((prefill_mfma_kernel<T, true, false>), dim3((unsigned)grid_l), dim3(kThreads), 0, stream, a, geo);
    } else {
        // a multiple of the padded KV-head count keeps each workgroup on one head
        int64_t grid = geo.slots < (int64_t)cus ? geo.slots : (int64_t)cus;
        const int g2 = 1 << geo.lg;
        if (grid > g2) grid -= grid % g2;
        if (paged)
            hipLaunchKernelGGL((prefill_mfma_kernel<T, false, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, geo);
        else
            hipLaunchKernelGGL((prefill_mfma_kernel<T, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a, geo);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_mfma(const VarlenArgs &a, hipStream_t stream) {
    return a.in_f16 ? launch_prefill_typed<f16>(a, stream) : launch_prefill_typed<bf16>(a, stream);
}

}  // namespace attn
