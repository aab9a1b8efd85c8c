// Route preprocessing on the device: membership table, per-row sorted key
// lists, 128 x 128 tile kinds and the forward / reverse tile lists.
//
// Definitions: "nemo_automodel ... flex_qsa" page (`_routes_to_membership`,
// `_block_mask_from_membership`, `_dense_blocks_to_ordered`) and "... fa4_qsa"
// page (`_preprocess`, `_block_kinds`, `_compact_blocks`). Everything stays on
// the device; the host never reads a count.
//
// gfx950 design: one workgroup per query row scatters the row's routes into an
// on-chip bitmap (one bit per key, LDS atomics dedupe for free), then writes
// the byte row of the table with 16-byte coalesced stores in a single pass
// (the table is never cleared and re-scattered in HBM), compacts the bitmap
// into the ascending key list with a workgroup prefix sum, and adds the row's
// per-tile popcounts into the tile counters with integer atomics (the result
// does not depend on their order). One wave per tile row / tile column then
// classifies and compacts with ballots.
#include "common.h"

namespace qsa {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kRouteUnroll = 8;  // route loads in flight per thread
constexpr int kFullWords = 256;

// LDS bytes of k_prep_rows without and with the staged key list; the list is
// staged when the whole fits in 64 KB.
__host__ __device__ inline size_t prep_lds_base(const Problem &p)
{
    return (size_t)(p.stride / 32) * 4 + (kPrepThreads + 1) * 4;
}
__host__ __device__ inline bool prep_stage_keys(const Problem &p)
{
    return prep_lds_base(p) + (size_t)p.W * 4 <= 65536;
}  // full-tile bits per tile row kept in LDS (8192 key tiles)

__global__ void k_fill_i32(int32_t *__restrict__ p, int64_t n, int32_t value)
{
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
         x += (int64_t)gridDim.x * blockDim.x)
        p[x] = value;
}

// Row `row`'s routes into its LDS bitmap (bm cleared, then one bit set per
// member key).
template <typename RouteT>
__device__ __forceinline__ void fill_from_routes(const Problem &p, uint32_t *bm, int64_t row,
                                                 int tid)
{
    // The loads of a round are all issued before its LDS atomics, so a row
    // waits for one or two memory latencies, not one per route.
    const RouteT *routes = static_cast<const RouteT *>(p.routes) + row * p.W;
    if (sizeof(RouteT) == 4 && (p.W & 3) == 0 && ((uintptr_t)p.routes & 15) == 0) {
        // Four consecutive slots per thread in one 16-byte load; the bits of
        // slots that fall in the same word are merged before the atomic, so
        // runs of consecutive keys cost one atomic per word and thread.
        const int4 *r4 = reinterpret_cast<const int4 *>(routes);
        const int64_t n4 = p.W >> 2;
        for (int64_t s0 = 0; s0 < n4; s0 += (int64_t)kPrepThreads * kRouteUnroll) {
            int4 r[kRouteUnroll];
#pragma unroll
            for (int u = 0; u < kRouteUnroll; ++u) {
                const int64_t s = s0 + u * kPrepThreads + tid;
                r[u] = s < n4 ? r4[s] : make_int4(-1, -1, -1, -1);
            }
#pragma unroll
            for (int u = 0; u < kRouteUnroll; ++u) {
                const int32_t v[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
                int32_t word = -1;
                uint32_t bits = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (v[e] < 0 || v[e] >= p.Skv) continue;
                    const int32_t wv = v[e] >> 5;
                    if (wv != word) {
                        if (bits) atomicOr(&bm[word], bits);
                        word = wv;
                        bits = 0u;
                    }
                    bits |= 1u << (v[e] & 31);
                }
                if (bits) atomicOr(&bm[word], bits);
            }
        }
    } else {
        for (int64_t s0 = 0; s0 < p.W; s0 += (int64_t)kPrepThreads * kRouteUnroll) {
            int64_t r[kRouteUnroll];
#pragma unroll
            for (int u = 0; u < kRouteUnroll; ++u) {
                const int64_t s = s0 + u * kPrepThreads + tid;
                r[u] = s < p.W ? (int64_t)routes[s] : -1;  // range test on the full width
            }
#pragma unroll
            for (int u = 0; u < kRouteUnroll; ++u)
                if (r[u] >= 0 && r[u] < p.Skv) atomicOr(&bm[r[u] >> 5], 1u << (r[u] & 31));
        }
    }
}

// floor(a / 4) for any sign (arithmetic shift).
__device__ __forceinline__ int64_t floor_div4(int64_t a) { return a >> 2; }

// Row t's block selection into its LDS bitmap (cuDNN Frontend QSA page,
// section "Selection and components"): key j is a member iff
// lo[t] <= j <= hi[t], 0 <= j < Skv, and its block
// b = blk_base[t] + floor((j - tok_base[t]) / 4) lies in [0, NB) with
// sel[t, b] != 0. Only the blocks that keys of [lo, hi] map to are read:
// block b holds the keys tok_base + 4 (b - blk_base) + 0..3.
__device__ __forceinline__ void fill_from_blocks(const Problem &p, uint32_t *bm, int64_t row,
                                                 int tid)
{
    const int64_t lo = max((int64_t)p.sel_lo[row], (int64_t)0);
    const int64_t hi = min((int64_t)p.sel_hi[row], p.Skv - 1);
    if (lo > hi) return;
    const int64_t bb = p.sel_blk_base[row], tb = p.sel_tok_base[row];
    const int64_t b0 = max(bb + floor_div4(lo - tb), (int64_t)0);
    const int64_t b1 = min(bb + floor_div4(hi - tb), p.NB - 1);
    const uint8_t *sel = p.sel + row * p.NB;
    constexpr int kUnroll = 8;
    for (int64_t c0 = b0; c0 <= b1; c0 += (int64_t)kPrepThreads * kUnroll) {
        uint8_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t bk = c0 + u * kPrepThreads + tid;
            v[u] = bk <= b1 ? sel[bk] : 0;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!v[u]) continue;
            const int64_t bk = c0 + u * kPrepThreads + tid;
            const int64_t first = tb + 4 * (bk - bb);
            const int64_t j0 = max(first, lo), j1 = min(first + 3, hi);
            // at most four keys, in at most two words
            for (int64_t j = j0; j <= j1;) {
                const int64_t w = j >> 5;
                const int64_t je = min(j1, 32 * w + 31);
                const uint32_t n = (uint32_t)(je - j + 1);
                atomicOr(&bm[w], ((1u << n) - 1u) << (j & 31));
                j = je + 1;
            }
        }
    }
}

// Row (b, i)'s document-causal selection into its LDS bitmap ("fa4" page,
// `document_causal_fa4_attention`): key j is a member iff the query's
// document id d is nonzero, kv_doc[b, j] == d and j <= q_global_start + i.
// Wave v takes the 64-key blocks v, v + 4, ... (four in flight): one ballot
// per block gives its two bitmap words, written without atomics.
__device__ __forceinline__ void fill_from_docs(const Problem &p, uint32_t *bm, int64_t row,
                                               int tid)
{
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int32_t d = p.q_doc[row];
    const int64_t hi = min(p.q_global_start + i, p.Skv - 1);
    if (d == 0 || hi < 0) return;
    const int lane = tid & 63, wave = tid >> 6;
    const int32_t *kd = p.kv_doc + b * p.Skv;
    constexpr int kU = 4;
    for (int64_t c0 = 64 * wave; c0 <= hi; c0 += 64 * 4 * kU) {
        int32_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = c0 + 64 * 4 * u + lane;
            v[u] = j <= hi ? kd[j] : 0;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j0 = c0 + 64 * 4 * u;
            const uint64_t ball = __ballot(j0 + lane <= hi && v[u] == d);
            if (j0 <= hi && lane == 0) {
                bm[j0 >> 5] = (uint32_t)ball;
                if ((j0 >> 5) + 1 < (p.stride >> 5)) bm[(j0 >> 5) + 1] = (uint32_t)(ball >> 32);
            }
        }
    }
}

// Everything after the row's bitmap is built: membership outputs, key list,
// count and tile counts.
__device__ __forceinline__ void finish_row(const Problem &p, uint32_t *bm, uint32_t *scan,
                                           int64_t row, int tid)
{
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int64_t nwords = p.stride >> 5;

    // Byte row of the membership table, 16 bytes per store.
    if (p.memb) {
        uint4 *dst = reinterpret_cast<uint4 *>(p.memb + row * p.stride);
        for (int64_t c = tid; c < (p.stride >> 4); c += kPrepThreads) {
            const uint32_t bits = (bm[c >> 1] >> ((c & 1) * 16)) & 0xffffu;
            uint32_t wv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t nib = (bits >> (4 * x)) & 0xfu;
                wv[x] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
            }
            dst[c] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }

    // Bit-packed copy of the row for the key-major backward scan.
    if (p.mbits) {
        uint32_t *dst = p.mbits + row * (p.stride >> 5);
        for (int64_t w = tid; w < nwords; w += kPrepThreads) dst[w] = bm[w];
    }

    // Ascending key list. Wave v owns a contiguous quarter of the words, and
    // inside it lane l owns words l, l + 64, ..., so a run of dense words (a
    // window of consecutive keys) spreads over the lanes instead of falling on
    // one thread. Positions: the words before the wave's quarter (wave totals
    // through LDS), then, inside the quarter, the earlier 64-word blocks and
    // the earlier lanes of the word's own block (wave scans). Calls that keep
    // only the bit-packed membership build their lists from it later
    // (k_row_lists); then there is no list and no count here.
    if (p.row_keys) {
        const int lane = tid & 63, wv = tid >> 6;
        const int64_t qw = (nwords + kPrepThreads / 64 - 1) / (kPrepThreads / 64);
        const int64_t wbeg = wv * qw, wend = (wbeg + qw < nwords) ? wbeg + qw : nwords;
        int mine = 0;
        for (int64_t w = wbeg + lane; w < wend; w += 64) mine += __popc(bm[w]);
        int wave_total = mine;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) wave_total += __shfl_xor(wave_total, off);
        if (lane == 0) scan[wv] = wave_total;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int v = 0; v < kPrepThreads / 64; ++v) {
            const int tv = scan[v];
            before += v < wv ? tv : 0;
            total += tv;
        }
        int32_t *keys = p.row_keys + row * p.W;
        const bool staged = prep_stage_keys(p);
        int32_t *sk = reinterpret_cast<int32_t *>(scan + kPrepThreads + 1);
        int run = before;  // keys before the current 64-word block
        for (int64_t w0 = wbeg; w0 < wend; w0 += 64) {
            const int64_t w = w0 + lane;
            uint32_t bits = w < wend ? bm[w] : 0u;
            const int c = __popc(bits);
            int inc = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(inc, off);
                if (lane >= off) inc += t;
            }
            int pos = run + inc - c;
            while (bits) {
                const int bit = __ffs(bits) - 1;
                bits &= bits - 1;
                const int32_t key = (int32_t)(w * 32 + bit);
                if (staged) sk[pos++] = key;  // through LDS: the list leaves in coalesced stores
                else keys[pos++] = key;
            }
            run += __shfl(inc, 63);
        }
        if (staged) {
            __syncthreads();
            for (int64_t s = tid; s < p.W; s += kPrepThreads) keys[s] = s < total ? sk[s] : -1;
        } else {
            for (int64_t s = total + tid; s < p.W; s += kPrepThreads) keys[s] = -1;
        }
        if (tid == 0) {
            p.row_cnt[row] = total;
            if (p.has_routes) p.has_routes[row] = total > 0 ? 1 : 0;
        }
    }

    // Tile counts: tile t covers words 4t .. 4t+3.
    int32_t *tc = p.tile_cnt + (b * p.nQT + (i >> 7)) * p.nKT;
    for (int64_t t = tid; t < p.nKT; t += kPrepThreads) {
        const int c = __popc(bm[4 * t]) + __popc(bm[4 * t + 1]) + __popc(bm[4 * t + 2]) +
                      __popc(bm[4 * t + 3]);
        if (c) atomicAdd(&tc[t], c);
    }
}

template <typename RouteT>
__global__ __launch_bounds__(kPrepThreads) void k_prep_rows(Problem p)
{
    extern __shared__ uint32_t lds[];
    const int64_t row = blockIdx.x;  // flat b * Sq + i
    const int tid = threadIdx.x;
    const int64_t nwords = p.stride >> 5;
    uint32_t *bm = lds;
    uint32_t *scan = lds + nwords;  // one total per wave
    for (int64_t w = tid; w < nwords; w += kPrepThreads) bm[w] = 0u;
    __syncthreads();
    fill_from_routes<RouteT>(p, bm, row, tid);
    __syncthreads();
    finish_row(p, bm, scan, row, tid);
}

__global__ __launch_bounds__(kPrepThreads) void k_prep_rows_docs(Problem p)
{
    extern __shared__ uint32_t lds[];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nwords = p.stride >> 5;
    uint32_t *bm = lds;
    uint32_t *scan = lds + nwords;
    for (int64_t w = tid; w < nwords; w += kPrepThreads) bm[w] = 0u;
    __syncthreads();
    fill_from_docs(p, bm, row, tid);
    __syncthreads();
    finish_row(p, bm, scan, row, tid);
}

__global__ __launch_bounds__(kPrepThreads) void k_prep_rows_blocks(Problem p)
{
    extern __shared__ uint32_t lds[];
    const int64_t row = blockIdx.x;  // packed token t
    const int tid = threadIdx.x;
    const int64_t nwords = p.stride >> 5;
    uint32_t *bm = lds;
    uint32_t *scan = lds + nwords;
    for (int64_t w = tid; w < nwords; w += kPrepThreads) bm[w] = 0u;
    __syncthreads();
    fill_from_blocks(p, bm, row, tid);
    __syncthreads();
    finish_row(p, bm, scan, row, tid);
}

__device__ __forceinline__ int32_t tile_kind(int32_t cnt)
{
    return cnt == 0 ? 0 : (cnt == kTile * kTile ? 2 : 1);
}

// One wave per (b, tile row): kinds and the forward lists.
__global__ __launch_bounds__(64) void k_lists_fwd(Problem p)
{
    const int64_t br = blockIdx.x;  // b * nQT + r
    const int lane = threadIdx.x;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t *tc = p.tile_cnt + br * p.nKT;
    int32_t *kd = p.kinds + br * p.nKT;
    int32_t *pi = p.fwd_p_idx + br * p.nKT;
    int32_t *fi = p.fwd_f_idx + br * p.nKT;
    int np_ = 0, nf = 0;
    for (int64_t t0 = 0; t0 < p.nKT; t0 += 64) {
        const int64_t t = t0 + lane;
        const bool in = t < p.nKT;
        const int32_t kind = in ? tile_kind(tc[t]) : 0;
        if (in) kd[t] = kind;
        const uint64_t mp = __ballot(in && kind == 1);
        const uint64_t mf = __ballot(in && kind == 2);
        if (kind == 1 && in) pi[np_ + __popcll(mp & below)] = (int32_t)t;
        if (kind == 2 && in) fi[nf + __popcll(mf & below)] = (int32_t)t;
        np_ += __popcll(mp);
        nf += __popcll(mf);
    }
    for (int64_t t = np_ + lane; t < p.nKT; t += 64) pi[t] = -1;
    for (int64_t t = nf + lane; t < p.nKT; t += 64) fi[t] = -1;
    if (lane == 0) {
        p.fwd_p_cnt[br] = np_;
        p.fwd_f_cnt[br] = nf;
    }
}

// One wave per (b, tile column): the reverse lists.
__global__ __launch_bounds__(64) void k_lists_rev(Problem p)
{
    const int64_t bt = blockIdx.x;  // b * nKT + t
    const int64_t b = bt / p.nKT, t = bt - b * p.nKT;
    const int lane = threadIdx.x;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t *pi = p.rev_p_idx + bt * p.nQT;
    int32_t *fi = p.rev_f_idx + bt * p.nQT;
    int np_ = 0, nf = 0;
    for (int64_t r0 = 0; r0 < p.nQT; r0 += 64) {
        const int64_t r = r0 + lane;
        const bool in = r < p.nQT;
        const int32_t kind = in ? tile_kind(p.tile_cnt[(b * p.nQT + r) * p.nKT + t]) : 0;
        const uint64_t mp = __ballot(in && kind == 1);
        const uint64_t mf = __ballot(in && kind == 2);
        if (kind == 1 && in) pi[np_ + __popcll(mp & below)] = (int32_t)r;
        if (kind == 2 && in) fi[nf + __popcll(mf & below)] = (int32_t)r;
        np_ += __popcll(mp);
        nf += __popcll(mf);
    }
    for (int64_t r = np_ + lane; r < p.nQT; r += 64) pi[r] = -1;
    for (int64_t r = nf + lane; r < p.nQT; r += 64) fi[r] = -1;
    if (lane == 0) {
        p.rev_p_cnt[bt] = np_;
        p.rev_f_cnt[bt] = nf;
    }
}

// One wave per row: the row's sorted key list without the keys of full tiles
// (order kept). Full tiles are computed densely; every other selected key
// stays on the gathered path.
__global__ __launch_bounds__(256) void k_partial_keys(Problem p)
{
    __shared__ uint32_t fullbits[4][kFullWords];
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.B * p.Sq) return;
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int32_t *kd = p.kinds + (b * p.nQT + (i >> 7)) * p.nKT;
    const int32_t *keys = p.row_keys + row * p.W;
    int32_t *out = p.pkeys + row * p.W;
    const int n = p.row_cnt[row];
    // Full-tile bits of the row's tile row in LDS (one bit per key tile), so
    // that a key's test needs no dependent load. Rows on tile rows longer than
    // the bit set test the kinds in memory.
    uint32_t *full = fullbits[threadIdx.x >> 6];
    const bool in_lds = p.nKT <= 32 * kFullWords;
    if (in_lds) {
        for (int64_t t0 = 0; t0 < p.nKT; t0 += 64) {
            const int64_t t = t0 + lane;
            const uint64_t f = __ballot(t < p.nKT && kd[t] == 2);
            if (lane == 0) {
                full[t0 >> 5] = (uint32_t)f;
                if ((t0 >> 5) + 1 < kFullWords) full[(t0 >> 5) + 1] = (uint32_t)(f >> 32);
            }
        }
    }
    wave_lds_sync();
    auto is_full = [&](int32_t key) {
        const int32_t t = key >> 7;
        return in_lds ? ((full[t >> 5] >> (t & 31)) & 1u) != 0u : kd[t] == 2;
    };
    int cnt = 0;
    // Eight 64-key groups per round, so that their loads are in flight together.
    for (int s0 = 0; s0 < n; s0 += 512) {
        int32_t key[8];
        bool keep[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + 64 * u + lane;
            key[u] = s < n ? keys[s] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) keep[u] = s0 + 64 * u + lane < n && !is_full(key[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint64_t ball = __ballot(keep[u]);
            if (keep[u]) out[cnt + __popcll(ball & below)] = key[u];
            cnt += __popcll(ball);
        }
    }
    if (lane == 0) p.pcnt[row] = cnt;
}


// A row's ascending key list and count from its bit-packed membership; with
// skip_full, without the keys of the full tiles of the row's tile row (the
// partial-tile list of the gathered passes, valid up to its count), else all
// keys with a -1 tail to the row width W. One wave per row: lane l takes words l, l + 64,
// ... four blocks of 64 words at a time (their loads in flight together);
// a word's keys go to positions from a wave prefix sum of the popcounts.
__global__ __launch_bounds__(256) void k_row_lists(Problem p, int32_t *out_keys,
                                                   int32_t *out_cnt, int skip_full)
{
    __shared__ uint32_t fullbits[4][kFullWords];
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.B * p.Sq) return;
    const int lane = threadIdx.x & 63;
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int64_t nwords = p.stride >> 5;
    const uint32_t *m = p.mbits + row * nwords;
    int32_t *out = out_keys + row * p.W;
    const int32_t *kd = p.kinds + (b * p.nQT + (i >> 7)) * p.nKT;
    uint32_t *full = fullbits[threadIdx.x >> 6];
    const bool in_lds = p.nKT <= 32 * kFullWords;
    if (skip_full && in_lds) {
        for (int64_t t0 = 0; t0 < p.nKT; t0 += 64) {
            const int64_t t = t0 + lane;
            const uint64_t f = __ballot(t < p.nKT && kd[t] == 2);
            if (lane == 0) {
                full[t0 >> 5] = (uint32_t)f;
                if ((t0 >> 5) + 1 < kFullWords) full[(t0 >> 5) + 1] = (uint32_t)(f >> 32);
            }
        }
    }
    wave_lds_sync();
    // word w lies in tile w / 4
    auto tile_full = [&](int64_t t) {
        return in_lds ? ((full[t >> 5] >> (t & 31)) & 1u) != 0u : kd[t] == 2;
    };
    constexpr int kR = 4;
    int base = 0;
    for (int64_t w0 = 0; w0 < nwords; w0 += 64 * kR) {
        uint32_t bits[kR];
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int64_t w = w0 + 64 * u + lane;
            bits[u] = w < nwords ? m[w] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int64_t w = w0 + 64 * u + lane;
            uint32_t x = bits[u];
            if (skip_full && x != 0u && tile_full(w >> 2)) x = 0u;
            const int c = __popc(x);
            int inc = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(inc, off);
                if (lane >= off) inc += t;
            }
            int pos = base + inc - c;
            while (x) {
                const int bit = __ffs(x) - 1;
                x &= x - 1;
                out[pos++] = (int32_t)(w * 32 + bit);
            }
            base += __shfl(inc, 63);
        }
    }
    // The full lists (for inspection) end in -1 up to W; the readers of the
    // partial-tile lists stop at the count, so those get no tail (a
    // document-causal plan of 32768 tokens has W = 32768: its tails were
    // 4.3 GB of stores).
    if (!skip_full)
        for (int64_t s2 = base + lane; s2 < p.W; s2 += 64) out[s2] = -1;
    if (lane == 0) out_cnt[row] = base;
}

}  // namespace

hipError_t launch_partial_keys(const Problem &p, hipStream_t s)
{
    const int64_t rows = p.B * p.Sq;
    if (p.row_keys)
        hipLaunchKernelGGL(k_partial_keys, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(k_row_lists, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p,
                           p.pkeys, p.pcnt, 1);
    return hipGetLastError();
}

hipError_t launch_row_keys(const Problem &p, int32_t *keys, int32_t *cnt, hipStream_t s)
{
    const int64_t rows = p.B * p.Sq;
    hipLaunchKernelGGL(k_row_lists, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p, keys,
                       cnt, 0);
    return hipGetLastError();
}

hipError_t launch_walk_reset(const Problem &p, hipStream_t s)
{
    // A fill kernel, not a memset: callers may capture these launches in a
    // graph.
    if (p.walk)
        hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(64), 0, s, reinterpret_cast<int32_t *>(p.walk),
                           (int64_t)16, 0);
    return hipGetLastError();
}

hipError_t launch_preprocess(const Problem &p, hipStream_t s)
{
    const int64_t ntiles = p.B * p.nQT * p.nKT;
    int blocks = (int)((ntiles + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_i32, dim3(blocks), dim3(256), 0, s, p.tile_cnt, ntiles, 0);
    const hipError_t e = launch_walk_reset(p, s);
    if (e != hipSuccess) return e;
    const size_t lds = prep_lds_base(p) + (prep_stage_keys(p) ? (size_t)p.W * 4 : 0);
    if (!p.routes && p.sel)
        hipLaunchKernelGGL(k_prep_rows_blocks, dim3((unsigned)(p.B * p.Sq)), dim3(kPrepThreads),
                           lds, s, p);
    else if (!p.routes)
        hipLaunchKernelGGL(k_prep_rows_docs, dim3((unsigned)(p.B * p.Sq)), dim3(kPrepThreads),
                           lds, s, p);
    else if (p.route_is_i64)
        hipLaunchKernelGGL(k_prep_rows<int64_t>, dim3((unsigned)(p.B * p.Sq)), dim3(kPrepThreads),
                           lds, s, p);
    else
        hipLaunchKernelGGL(k_prep_rows<int32_t>, dim3((unsigned)(p.B * p.Sq)), dim3(kPrepThreads),
                           lds, s, p);
    hipLaunchKernelGGL(k_lists_fwd, dim3((unsigned)(p.B * p.nQT)), dim3(64), 0, s, p);
    hipLaunchKernelGGL(k_lists_rev, dim3((unsigned)(p.B * p.nKT)), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
