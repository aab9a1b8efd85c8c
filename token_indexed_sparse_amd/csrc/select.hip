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
//    order-preserving 32-bit keys held in registers; a radix search over the
//    keys relative to the row's smallest (11 bits a step from the highest bit
//    the row's range needs, histograms in LDS) narrows the top_k-th key to one
//    bin, whose keys are ranked directly when there are few; ballots place
//    the chosen blocks in ascending order, and the block list and route rows
//    leave in coalesced stores.
#include "common.h"

namespace qsa {
namespace {

constexpr int kSelRow = kSelD * 2;                    // bytes per indexer row (bf16)
constexpr int kSelWaves = 4;                          // waves per scoring work group
constexpr int kSelTileRows = 128;                     // kbar rows per staged tile
constexpr int kSelTileBytes = kSelTileRows * kSelRow;  // 32 KB per buffer, two buffers

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
        for (int i = 0; i < 32 / kSelWaves; ++i) {
            const int ins = (32 / kSelWaves) * wave + i;  // 32 loads of 4 rows each
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
        // Two halves of 64 rows, four slabs of 16 rows each.
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            float part[QW][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 Bv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    Bv[k] = lds_read16(tile + (64 * hs + 16 * s + col) * kSelRow +
                                       (((4 * k + quad) ^ col) << 4));
#pragma unroll
                for (int qi = 0; qi < QW; ++qi) {
                    float acc = 0.0f;
#pragma unroll
                    for (int g = 0; g < HG; ++g) {
                        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            c = mfma_16x16x32(A[qi][g][k], as_bf16x8(Bv[k]), c);
                        acc += (fmaxf(c[0], 0.0f) + fmaxf(c[1], 0.0f)) +
                               (fmaxf(c[2], 0.0f) + fmaxf(c[3], 0.0f));
                    }
                    part[qi][s] = acc;
                }
            }
            // Reduce-scatter over the quads: lane (col, quad) ends with the sum
            // over all heads for row row0 + 64 hs + 16 quad + col.
            const bool upper = (quad & 2) != 0, odd = (quad & 1) != 0;
#pragma unroll
            for (int qi = 0; qi < QW; ++qi) {
                const float s0 = upper ? part[qi][0] : part[qi][2];
                const float s1 = upper ? part[qi][1] : part[qi][3];
                const float w0 = (upper ? part[qi][2] : part[qi][0]) + __shfl_xor(s0, 32);
                const float w1 = (upper ? part[qi][3] : part[qi][1]) + __shfl_xor(s1, 32);
                const float sum = (odd ? w1 : w0) + __shfl_xor(odd ? w0 : w1, 16);
                const int64_t r = row0 + 64 * hs + 16 * quad + col;
                if (r >= qr0[qi] && r < qr1[qi]) srow[qi * a.NB + r] = a.scale * sum + 0.0f;
            }
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

constexpr int kBins = 2048;      // radix digit of 11 bits
constexpr int kMaxCand = 64;     // boundary bins this small are ranked directly
// Bin b lives at word b + b / 32: lane l of the bin search reads its 32 bins
// at 33 l + j, 64 distinct banks for every j.
constexpr int kHistWords = kBins + kBins / 32;
__device__ __forceinline__ int hslot(uint32_t b) { return (int)(b + (b >> 5)); }

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

// Exclusive prefix sums of arr[0 .. n) in place, by one wave (lane l takes a
// contiguous run of the entries).
__device__ __forceinline__ void wave_scan_lds(uint32_t *arr, int n)
{
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) >> 6;
    uint32_t mine = 0;
    for (int j = 0; j < per; ++j) {
        const int i = per * lane + j;
        mine += i < n ? arr[i] : 0u;
    }
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    uint32_t run = incl - mine;
    for (int j = 0; j < per; ++j) {
        const int i = per * lane + j;
        if (i < n) {
            const uint32_t x = arr[i];
            arr[i] = run;
            run += x;
        }
    }
}

// Writes -1 into out[from .. to) (int32 words), the work group together.
__device__ __forceinline__ void fill_minus1(int32_t *out, int64_t from, int64_t to, int nt)
{
    for (int64_t i = from + threadIdx.x; i < to; i += nt) out[i] = -1;
}

// One work group of NT threads per query row. Thread (wave w, lane l) holds
// the rows r0 + NT m + 64 w + l for m < KPT: chunk m covers NT consecutive
// rows in thread order, so ballots give each thread its place in row order. A
// key of 0 marks a row past the visible ones (real keys are at least 1).
//
// Selection: with n visible blocks and n > top_k, the keys are rebased to
// rel = key - (smallest key) + 1 and a radix search runs over rel, 11 bits at
// a time from the highest bit the row's range needs, so the first histogram
// already spreads over the row's values. need = how many keys that match the
// current prefix are still to be taken. The search ends when the bin holding
// the boundary is taken whole (its count equals need), or when it holds at
// most kMaxCand keys: those are ranked directly (larger key first, then lower
// row), which fixes the boundary key and row. When the digits run out, every
// key of the bin is the same and the first `need` of them in row order are
// taken. Every case ends as one rule: take key > tau, and of the keys equal
// to tau those at rows <= tie_row.
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void k_select_topk(SelectProblem a)
{
    constexpr int NW = NT / 64;  // waves per row
    __shared__ uint32_t hist[2][kHistWords];
    __shared__ uint32_t cnt[KPT * NW];
    __shared__ uint32_t red[2 * NW];
    __shared__ uint32_t cand_key[kMaxCand], cand_row[kMaxCand];
    __shared__ uint32_t ncand;
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
        if (bo) fill_minus1(bo, 0, k, NT);
        if (ro) fill_minus1(ro, 0, W, NT);
        return;
    }
    const int n = (int)(q.r1 - q.r0);
    const int nsel = n < k ? n : k;
    const float *sr = a.scores + row * a.NB;

    // One buffer descriptor over the visible scores; chunk m at a scalar offset.
    const rsrc_t srs = make_rsrc(sr + q.r0, (uint32_t)n * 4u);
    uint32_t key[KPT];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
        const bool in = (int)threadIdx.x < n - NT * m;
        const float f = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(srs, 4 * (int)threadIdx.x, 4 * NT * m, 0));
        const uint32_t kv = score_key(f);
        key[m] = in ? (kv > 1u ? kv : 1u) : 0u;
        if (in) {
            kmin = key[m] < kmin ? key[m] : kmin;
            kmax = key[m] > kmax ? key[m] : kmax;
        }
    }

    uint32_t tau = 0, tie_row = 0;  // with n <= top_k: every key >= 1
    if (n > k) {
        uint32_t need = (uint32_t)k;
        for (int i = threadIdx.x; i < kHistWords; i += NT) hist[0][i] = 0;
        if (threadIdx.x == 0) ncand = 0;
#pragma unroll
        for (int o = 32; o; o >>= 1) {
            const uint32_t x = __shfl_xor(kmin, o), y = __shfl_xor(kmax, o);
            kmin = x < kmin ? x : kmin;
            kmax = y > kmax ? y : kmax;
        }
        if (lane == 0) {
            red[w] = kmin;
            red[NW + w] = kmax;
        }
        __syncthreads();
        kmin = red[0];
        kmax = red[NW];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
            kmin = red[i] < kmin ? red[i] : kmin;
            kmax = red[NW + i] > kmax ? red[NW + i] : kmax;
        }
#pragma unroll
        for (int m = 0; m < KPT; ++m) key[m] = key[m] ? key[m] - kmin + 1u : 0u;
        const uint32_t range = kmax - kmin + 1u;  // largest rel
        // Keys in play: (rel >> hi_sh) == prefix; the digit is rel >> sh
        // (hi_sh - sh <= 11 bits).
        int sh = range >> 11 ? 32 - __builtin_clz(range) - 11 : 0;
        int hi_sh = sh + 11;
        uint32_t prefix = 0;
        int mode = 0;
#pragma unroll 1
        for (int pass = 0;; ++pass) {
            uint32_t *h = hist[pass & 1];
            // Clear the other buffer for the next pass (its last reads were
            // before the previous pass's pick barrier).
            for (int i = threadIdx.x; i < kHistWords; i += NT) hist[(pass + 1) & 1][i] = 0;
            const uint32_t dmask = (1u << (hi_sh - sh)) - 1u;
            const bool all_in = hi_sh >= 32;
            const int hs = all_in ? 31 : hi_sh;  // no shift by 32 (all_in decides then)
            // Rows past the visible ones (key 0) stay out; the zero is hidden
            // from the compiler so that it recomputes this test each pass
            // instead of keeping a mask per key alive.
            uint32_t zero_h = 0;
            asm volatile("" : "+s"(zero_h));
#pragma unroll
            for (int m = 0; m < KPT; ++m)
                if (key[m] > zero_h && (all_in || (key[m] >> hs) == prefix))
                    atomicAdd(&h[hslot((key[m] >> sh) & dmask)], 1u);
            __syncthreads();
            if (w == 0) {
                // Bin of the boundary: lane l sums bins [32 l, 32 l + 32); the
                // counts of higher lanes' bins come from a suffix scan.
                uint32_t mine = 0;
#pragma unroll 8
                for (int j = 0; j < 32; ++j) mine += h[33 * lane + j];
                uint32_t incl = mine;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = __shfl_down(incl, o);
                    if (lane + o < 64) incl += y;
                }
                uint32_t above = incl - mine;
                if (above < need && incl >= need) {
                    for (int j = 31; j >= 0; --j) {
                        const uint32_t x = h[33 * lane + j];
                        if (above + x >= need) {
                            pick[0] = (uint32_t)(32 * lane + j);
                            pick[1] = above;
                            pick[2] = x;
                            break;
                        }
                        above += x;
                    }
                }
            }
            __syncthreads();
            const uint32_t cbin = pick[2];
            prefix = (prefix << (hi_sh - sh)) | pick[0];  // rel >> sh of the bin
            need -= pick[1];
            if (cbin == need) {  // the whole bin is taken: rel >= prefix << sh (>= 1)
                tau = prefix << sh;
                tie_row = 0xffffffffu;
                break;
            }
            if (sh == 0) {  // every key of the bin equals prefix (>= 1)
                tau = prefix;
                mode = 3;
                break;
            }
            if (cbin <= (uint32_t)kMaxCand) {
                // Rank the bin's keys directly: larger key first, then lower row.
                uint32_t zero_c = 0;  // a second hidden zero: no masks kept from above
                asm volatile("" : "+s"(zero_c));
#pragma unroll
                for (int m = 0; m < KPT; ++m) {
                    if (key[m] > zero_c && (key[m] >> sh) == prefix) {
                        const uint32_t slot = atomicAdd(&ncand, 1u);
                        cand_key[slot] = key[m];
                        cand_row[slot] = (uint32_t)(NT * m + threadIdx.x);
                    }
                }
                __syncthreads();
                if (w == 0 && lane < (int)cbin) {
                    const uint32_t ck = cand_key[lane], cr = cand_row[lane];
                    uint32_t rank = 0;
                    for (int j = 0; j < (int)cbin; ++j) {
                        const uint32_t ok = cand_key[j], orow = cand_row[j];
                        rank += (ok > ck || (ok == ck && orow < cr)) ? 1u : 0u;
                    }
                    if (rank == need - 1) {
                        pick[0] = ck;
                        pick[1] = cr;
                    }
                }
                __syncthreads();
                tau = pick[0];
                tie_row = pick[1];
                break;
            }
            hi_sh = sh;
            sh = sh >= 11 ? sh - 11 : 0;
            __syncthreads();  // pick is rewritten by the next pass
        }
        if (mode == 3) {
            // tie_row: the row of the need-th key equal to tau in row order
#pragma unroll
            for (int m = 0; m < KPT; ++m) {
                const uint64_t e = __ballot(key[m] == tau);
                if (lane == 0) cnt[NW * m + w] = (uint32_t)__builtin_popcountll(e);
            }
            __syncthreads();
            if (w == 0) wave_scan_lds(cnt, KPT * NW);
            __syncthreads();
#pragma unroll
            for (int m = 0; m < KPT; ++m) {
                const bool eq = key[m] == tau;
                const uint32_t rank = cnt[NW * m + w] + lanes_below(__ballot(eq));
                if (eq && rank == need - 1) pick[3] = (uint32_t)(NT * m + threadIdx.x);
            }
            __syncthreads();
            tie_row = pick[3];
        }
    }
    // Row NT m + tid <= tie_row, compared as (chunk, thread) pairs.
    const int tie_m = (int)(tie_row / NT);
    const bool tid_le = threadIdx.x <= tie_row % NT;
    auto take = [&](int m) {
        return key[m] > tau || (key[m] == tau && (m < tie_m || (m == tie_m && tid_le)));
    };

    // Output positions in row order. The kept block numbers are compacted
    // into LDS (the histogram space, free by now: top_k <= 4096 words), then
    // the block list and the route rows leave in coalesced stores.
    int32_t *sel = reinterpret_cast<int32_t *>(&hist[0][0]);
    if (nsel > 0) {
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const uint64_t e = __ballot(take(m));
            if (lane == 0) cnt[NW * m + w] = (uint32_t)__builtin_popcountll(e);
        }
        __syncthreads();
        if (w == 0) wave_scan_lds(cnt, KPT * NW);
        __syncthreads();
        // Recompute the rule rather than keep KPT ballot masks across the scan.
        asm volatile("" : "+v"(tau));
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
            const bool tk = take(m);
            const uint64_t e = __ballot(tk);
            if (tk)
                sel[cnt[NW * m + w] + lanes_below(e)] =
                    (int32_t)(q.r0 + NT * m + threadIdx.x - q.base);
        }
        __syncthreads();
    }
    if (bo)
        for (int i = threadIdx.x; i < k; i += NT) bo[i] = i < nsel ? sel[i] : -1;
    if (ro) {
        // route row: slot group g < nsel holds block sel[g], then -1 groups,
        // and group k the query's own incomplete block
        int4 *r4 = reinterpret_cast<int4 *>(ro);
        const int64_t p = a.q_offset + t;
        for (int g = threadIdx.x; g <= k; g += NT) {
            int4 v = make_int4(-1, -1, -1, -1);
            if (g < nsel) {
                const int32_t id = (int32_t)(q.s + 4 * (int64_t)sel[g]);
                v = make_int4(id, id + 1, id + 2, id + 3);
            } else if (g == k) {
                const int64_t id = q.s + 4 * q.c;
                v = make_int4((int32_t)id, id + 1 <= p ? (int32_t)(id + 1) : -1,
                              id + 2 <= p ? (int32_t)(id + 2) : -1,
                              id + 3 <= p ? (int32_t)(id + 3) : -1);
            }
            r4[g] = v;
        }
    }
}

template <int KPT, int NT>
hipError_t launch_topk_kpt(const SelectProblem &a, hipStream_t s)
{
    hipLaunchKernelGGL((k_select_topk<KPT, NT>), dim3((unsigned)(a.B * a.Sq)), dim3(NT), 0, s, a);
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
    // Up to 2048 blocks a row: 256 threads, at most 8 keys each; longer rows:
    // 512 threads (16 keys each at 8192 blocks), measured 7 % faster there
    // than 256 threads with 32 keys each (1024 threads were 40 % slower).
    if (a.NB <= 1024) return launch_topk_kpt<4, 256>(a, s);
    if (a.NB <= 2048) return launch_topk_kpt<8, 256>(a, s);
    if (a.NB <= 4096) return launch_topk_kpt<8, 512>(a, s);
    if (a.NB <= 8192) return launch_topk_kpt<16, 512>(a, s);
    if (a.NB <= 16384) return launch_topk_kpt<32, 512>(a, s);
    return launch_topk_kpt<64, 512>(a, s);
}

}  // namespace qsa
