// Block selector of QSA (cuDNN Frontend QSA page, "Finding QSA attention and
// its indexer"): every complete compressed block before a query's own block
// scores scale * sum_h relu(qi[t, h] . kbar[block]); each query keeps its top_k
// blocks, which are expanded into the route rows that the attention entry
// points take (NeMo AutoModel QSA page: four-token groups of complete blocks,
// -1 padding, then the query's incomplete causal tail).
//
// Two kernels:
//  * k_select_scores, a dense contraction on the matrix cores: the A operand
//    is 16 heads of one query (the indexer rows stay in registers for the whole
//    pass), the B operand 16 kbar rows staged through LDS. Each MFMA output is
//    one head's dot with one block; relu and the head sum happen in registers,
//    then a reduce-scatter over the four lane quads leaves one score per lane.
//  * k_select_topk, one work group per query row: the row's scores become
//    order-preserving 32-bit keys held in registers, a three-pass radix select
//    (11, 11 and 10 bits, histograms in LDS) finds the top_k-th key, and
//    ballots place the chosen blocks in ascending order in the outputs.
#include "common.h"

namespace qsa {
namespace {

constexpr int kSelRow = kSelD * 2;                    // bytes per indexer row (bf16)
constexpr int kSelWaves = 8;                          // waves per scoring work group
constexpr int kSelTileRows = 64;                      // kbar rows per staged tile
constexpr int kSelTileBytes = kSelTileRows * kSelRow;  // 16 KB

// Position data of query t of batch row b: its document start s, the kbar row
// base of its document and the visible kbar rows [r0, r1). A query whose
// document starts after it or at a negative position is padding (c = -1).
struct QueryRange {
    int64_t s, base, c, r0, r1;
};

__device__ __forceinline__ QueryRange query_range(const SelectProblem &a, int64_t b, int64_t t)
{
    QueryRange q;
    const int64_t p = a.q_offset + t;
    q.s = a.doc_start ? (int64_t)a.doc_start[b * a.Sq + t] : 0;
    q.base = a.blk_base ? (int64_t)a.blk_base[b * a.Sq + t] : 0;
    if (q.s < 0 || q.s > p) {
        q.c = -1;
        q.r0 = q.r1 = 0;
        return q;
    }
    q.c = (p - q.s) >> 2;
    q.r0 = q.base > 0 ? q.base : 0;
    q.r1 = q.base + q.c < a.NB ? q.base + q.c : a.NB;
    if (q.r1 < q.r0) q.r1 = q.r0;
    return q;
}

__device__ __forceinline__ int64_t wave_min(int64_t x)
{
    for (int o = 32; o; o >>= 1) {
        const int64_t y = __shfl_xor(x, o);
        x = y < x ? y : x;
    }
    return x;
}

__device__ __forceinline__ int64_t wave_max(int64_t x)
{
    for (int o = 32; o; o >>= 1) {
        const int64_t y = __shfl_xor(x, o);
        x = y > x ? y : x;
    }
    return x;
}

// Work group: kSelWaves waves x QW queries; wave w takes queries t0 + w QW ..
// t0 + w QW + QW - 1 and the kbar rows of the union of their visible ranges,
// tile by tile. HG groups of 16 heads (heads past H read as zero and add zero).
template <int HG, int QW>
__global__ __launch_bounds__(64 * kSelWaves) void k_select_scores(SelectProblem a)
{
    constexpr int QT = kSelWaves * QW;
    __shared__ __attribute__((aligned(16))) char tiles[2 * kSelTileBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    const int64_t ntiles_b = (a.Sq + QT - 1) / QT;
    // The last query tiles see the most blocks: they go first.
    const int64_t b = (int64_t)blockIdx.x % a.B;
    const int64_t t0 = (ntiles_b - 1 - (int64_t)blockIdx.x / a.B) * QT;

    // Union of the work group's visible rows (every wave computes it).
    int64_t lo = INT64_MAX, hi = INT64_MIN;
    if (lane < QT && t0 + lane < a.Sq) {
        const QueryRange r = query_range(a, b, t0 + lane);
        if (r.r1 > r.r0) {
            lo = r.r0;
            hi = r.r1;
        }
    }
    const int64_t R_lo = wave_min(lo), R_hi = wave_max(hi);
    if (R_lo >= R_hi) return;  // uniform over the work group

    // This wave's queries and their ranges.
    int64_t qr0[QW], qr1[QW];
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
        const int64_t t = t0 + wave * QW + qi;
        qr0[qi] = qr1[qi] = 0;
        if (t < a.Sq) {
            const QueryRange r = query_range(a, b, t);
            qr0[qi] = r.r0;
            qr1[qi] = r.r1;
        }
    }

    // A operands: lane (head col of group g, quad) holds elements 32 k + 8 quad
    // .. +7 of that head's row, for the four K steps k.
    const int64_t nq = a.Sq - t0 < QT ? a.Sq - t0 : QT;
    const rsrc_t qr = make_rsrc(a.q + (b * a.Sq + t0) * a.H * kSelD,
                                (uint32_t)(nq * a.H * kSelRow));
    bf16x8 A[QW][HG][4];
#pragma unroll
    for (int qi = 0; qi < QW; ++qi)
#pragma unroll
        for (int g = 0; g < HG; ++g) {
            const int h = 16 * g + col;
            const uint32_t row = (uint32_t)((wave * QW + qi) * a.H + h);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t off = h < a.H ? row * kSelRow + k * 64 + quad * 16 : kOutOfRange;
                A[qi][g][k] = as_bf16x8(buf_load16(qr, off));
            }
        }

    // kbar tiles: row rr of a tile at byte rr * 256, its 16-byte chunk c at
    // slot c ^ (rr & 15), so that 16 lanes reading one chunk of 16 rows touch
    // every bank once. Rows past NB read as zero.
    const i32x4 kr = rsrc_words(a.kbar + b * a.NB * kSelD, (uint32_t)(a.NB * kSelRow));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)tiles;
    auto stage = [&](int64_t row0, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ins = 2 * wave + i;             // 16 instructions of 4 rows each
            const int rr = 4 * ins + (lane >> 4);
            const uint32_t off = (uint32_t)(row0 + rr) * kSelRow +
                                 (uint32_t)(((lane & 15) ^ (rr & 15)) << 4);
            dma16_asm(kr, lds0 + buf * kSelTileBytes + ins * 1024, off);
        }
    };

    const int64_t ntile = (R_hi - R_lo + kSelTileRows - 1) / kSelTileRows;
    stage(R_lo, 0);
    QSA_WAIT_VM(0);
    __syncthreads();
    float *const srow = a.scores + (b * a.Sq + t0 + wave * QW) * a.NB;
    for (int64_t n = 0; n < ntile; ++n) {
        const int buf = (int)(n & 1);
        const int64_t row0 = R_lo + n * kSelTileRows;
        if (n + 1 < ntile) stage(row0 + kSelTileRows, buf ^ 1);
        const lds_char *tile = (const lds_char *)tiles + buf * kSelTileBytes;
        float part[QW][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 Bv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                Bv[k] = lds_read16(tile + (16 * s + col) * kSelRow + (((4 * k + quad) ^ col) << 4));
#pragma unroll
            for (int qi = 0; qi < QW; ++qi) {
                float acc = 0.0f;
#pragma unroll
                for (int g = 0; g < HG; ++g) {
                    f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < 4; ++k) c = mfma_16x16x32(A[qi][g][k], as_bf16x8(Bv[k]), c);
                    acc += (fmaxf(c[0], 0.0f) + fmaxf(c[1], 0.0f)) +
                           (fmaxf(c[2], 0.0f) + fmaxf(c[3], 0.0f));
                }
                part[qi][s] = acc;
            }
        }
        // Reduce-scatter over the quads: lane (col, quad) ends with the sum over
        // all heads for row row0 + 16 quad + col.
        const bool upper = (quad & 2) != 0, odd = (quad & 1) != 0;
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) {
            const float s0 = upper ? part[qi][0] : part[qi][2];
            const float s1 = upper ? part[qi][1] : part[qi][3];
            const float w0 = (upper ? part[qi][2] : part[qi][0]) + __shfl_xor(s0, 32);
            const float w1 = (upper ? part[qi][3] : part[qi][1]) + __shfl_xor(s1, 32);
            const float sum = (odd ? w1 : w0) + __shfl_xor(odd ? w0 : w1, 16);
            const int64_t r = row0 + 16 * quad + col;
            if (r >= qr0[qi] && r < qr1[qi]) srow[qi * a.NB + r] = a.scale * sum + 0.0f;
        }
        QSA_WAIT_VM(0);
        __syncthreads();
    }
}

template <int HG>
hipError_t launch_scores_hg(const SelectProblem &a, hipStream_t s)
{
    constexpr int QW = HG <= 2 ? 4 : 2;
    constexpr int QT = kSelWaves * QW;
    const int64_t blocks = a.B * ((a.Sq + QT - 1) / QT);
    hipLaunchKernelGGL((k_select_scores<HG, QW>), dim3((unsigned)blocks), dim3(64 * kSelWaves), 0,
                       s, a);
    return hipGetLastError();
}

__global__ void k_fill_f32(float *p, int64_t n, float v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ---- top-k ----

constexpr int kTopThreads = 256;

// Exclusive prefix of v over the work group's threads in order; total in tot.
// Ends with a barrier, so the scratch can be reused at once.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *wsum, uint32_t &tot)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint32_t pre = 0, t = 0;
#pragma unroll
    for (int i = 0; i < kTopThreads / 64; ++i) {
        const uint32_t x = wsum[i];
        pre += i < w ? x : 0u;
        t += x;
    }
    __syncthreads();
    tot = t;
    return pre + incl - v;
}

// Order-preserving key of a score: larger score, larger key; -0 and +0 alike.
__device__ __forceinline__ uint32_t score_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Writes -1 into out[from .. to) (int32 words), the work group together.
__device__ __forceinline__ void fill_minus1(int32_t *out, int64_t from, int64_t to)
{
    for (int64_t i = from + threadIdx.x; i < to; i += kTopThreads) out[i] = -1;
}

// One work group per query row. Thread (wave w, lane l) holds the rows
// r0 + 256 m + 64 w + l for m < KPT, so chunk m covers 256 consecutive rows
// in thread order and ballots give each thread its place in row order.
template <int KPT>
__global__ __launch_bounds__(kTopThreads) void k_select_topk(SelectProblem a)
{
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t cnt[KPT * 4];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t pick[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int64_t b = row / a.Sq, t = row % a.Sq;
    const int k = a.top_k;
    const int64_t W = 4 * (int64_t)k + 4;
    int32_t *bo = a.blocks ? a.blocks + row * k : nullptr;
    int32_t *ro = a.routes ? a.routes + row * W : nullptr;
    const QueryRange q = query_range(a, b, t);
    if (q.c < 0) {  // padding: nothing selected, no tail
        if (bo) fill_minus1(bo, 0, k);
        if (ro) fill_minus1(ro, 0, W);
        return;
    }
    const int64_t n = q.r1 - q.r0;
    const int nsel = n < k ? (int)n : k;
    const float *sr = a.scores + row * a.NB;

    uint32_t key[KPT];
    bool valid[KPT];
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const int64_t r = q.r0 + 256 * m + threadIdx.x;
        valid[m] = r < q.r1;
        key[m] = valid[m] ? score_key(sr[r]) : 0u;
    }

    // Radix select of the nsel-th largest key (skipped when every visible
    // block is kept). need = how many of the keys that match the prefix so far
    // are still to be taken.
    bool all = n <= k;      // take every valid key
    bool ge_only = false;   // take the keys >= prefix
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)k, eq_cnt = 0;
    if (!all) {
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
            const uint32_t nb = pass < 2 ? 2048u : 1024u;
            for (int i = threadIdx.x; i < (int)nb; i += kTopThreads) hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < KPT; ++m)
                if (valid[m] && (key[m] & pmask) == prefix)
                    atomicAdd(&hist[(key[m] >> shift) & (nb - 1)], 1u);
            __syncthreads();
            // Thread i sums bins [per i, per i + per); the bins of higher threads
            // hold larger keys.
            const int per = (int)nb / kTopThreads;
            uint32_t mine = 0;
            for (int j = 0; j < per; ++j) mine += hist[per * threadIdx.x + j];
            uint32_t tot;
            const uint32_t below = block_scan(mine, wsum, tot);
            const uint32_t above = tot - below - mine;  // counts in higher threads' bins
            if (above < need && above + mine >= need) {
                uint32_t acc = above;
                for (int j = per - 1; j >= 0; --j) {
                    const uint32_t h = hist[per * threadIdx.x + j];
                    if (acc + h >= need) {
                        pick[0] = (uint32_t)(per * threadIdx.x + j);
                        pick[1] = acc;
                        pick[2] = h;
                        break;
                    }
                    acc += h;
                }
            }
            __syncthreads();
            const uint32_t bin = pick[0];
            need -= pick[1];
            eq_cnt = pick[2];
            prefix |= bin << shift;
            pmask |= (nb - 1) << shift;
            __syncthreads();  // pick is rewritten by the next pass
            if (eq_cnt == need) {
                ge_only = true;
                break;
            }
        }
    }

    // Which keys are taken; among keys equal to the final prefix (ties on the
    // full key) only the first `need` in row order.
    bool take[KPT];
    const bool ties = !all && !ge_only;
    if (ties) {
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const uint64_t e = __ballot(valid[m] && key[m] == prefix);
            if (lane == 0) cnt[4 * m + w] = (uint32_t)__builtin_popcountll(e);
        }
        __syncthreads();
        // exclusive scan of cnt[] in (m, wave) order
        const int per = (KPT * 4 + kTopThreads - 1) / kTopThreads;
        uint32_t mine = 0;
        for (int j = 0; j < per; ++j) {
            const int i = per * threadIdx.x + j;
            mine += i < KPT * 4 ? cnt[i] : 0u;
        }
        uint32_t tot;
        uint32_t run = block_scan(mine, wsum, tot);
        for (int j = 0; j < per; ++j) {
            const int i = per * threadIdx.x + j;
            if (i < KPT * 4) {
                const uint32_t x = cnt[i];
                cnt[i] = run;
                run += x;
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const bool eq = valid[m] && key[m] == prefix;
            const uint64_t e = __ballot(eq);
            const uint32_t rank = cnt[4 * m + w] + lanes_below(e);
            take[m] = valid[m] && (key[m] > prefix || (eq && rank < need));
        }
        __syncthreads();  // cnt is reused below
    } else {
#pragma unroll
        for (int m = 0; m < KPT; ++m) take[m] = valid[m] && (all || key[m] >= prefix);
    }

    // Output positions in row order.
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const uint64_t e = __ballot(take[m]);
        if (lane == 0) cnt[4 * m + w] = (uint32_t)__builtin_popcountll(e);
    }
    __syncthreads();
    {
        const int per = (KPT * 4 + kTopThreads - 1) / kTopThreads;
        uint32_t mine = 0;
        for (int j = 0; j < per; ++j) {
            const int i = per * threadIdx.x + j;
            mine += i < KPT * 4 ? cnt[i] : 0u;
        }
        uint32_t tot;
        uint32_t run = block_scan(mine, wsum, tot);
        for (int j = 0; j < per; ++j) {
            const int i = per * threadIdx.x + j;
            if (i < KPT * 4) {
                const uint32_t x = cnt[i];
                cnt[i] = run;
                run += x;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const uint64_t e = __ballot(take[m]);
        if (take[m]) {
            const uint32_t pos = cnt[4 * m + w] + lanes_below(e);
            const int64_t j = q.r0 + 256 * m + threadIdx.x - q.base;
            if (bo) bo[pos] = (int32_t)j;
            if (ro) {
                const int32_t id = (int32_t)(q.s + 4 * j);
                *reinterpret_cast<int4 *>(ro + 4 * (int64_t)pos) = make_int4(id, id + 1, id + 2, id + 3);
            }
        }
    }
    if (bo) fill_minus1(bo, nsel, k);
    if (ro) {
        fill_minus1(ro, 4 * (int64_t)nsel, 4 * (int64_t)k);
        if (threadIdx.x < 4) {
            const int64_t p = a.q_offset + t;
            const int64_t id = q.s + 4 * q.c + threadIdx.x;
            ro[4 * (int64_t)k + threadIdx.x] = id <= p ? (int32_t)id : -1;
        }
    }
}

template <int KPT>
hipError_t launch_topk_kpt(const SelectProblem &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_select_topk<KPT>, dim3((unsigned)(a.B * a.Sq)), dim3(kTopThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select_fill(const SelectProblem &a, hipStream_t s)
{
    const int64_t n = a.B * a.Sq * a.NB;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, s, a.scores, n,
                       -INFINITY);
    return hipGetLastError();
}

hipError_t launch_select_scores(const SelectProblem &a, hipStream_t s)
{
    switch ((a.H + 15) / 16) {
    case 1: return launch_scores_hg<1>(a, s);
    case 2: return launch_scores_hg<2>(a, s);
    case 3: return launch_scores_hg<3>(a, s);
    default: return launch_scores_hg<4>(a, s);
    }
}

hipError_t launch_select_topk(const SelectProblem &a, hipStream_t s)
{
    const int64_t kpt = (a.NB + kTopThreads - 1) / kTopThreads;
    if (kpt <= 4) return launch_topk_kpt<4>(a, s);
    if (kpt <= 8) return launch_topk_kpt<8>(a, s);
    if (kpt <= 16) return launch_topk_kpt<16>(a, s);
    if (kpt <= 32) return launch_topk_kpt<32>(a, s);
    if (kpt <= 64) return launch_topk_kpt<64>(a, s);
    return launch_topk_kpt<128>(a, s);
}

}  // namespace qsa
