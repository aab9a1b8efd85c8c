// Full 128 x 128 tiles of route-set grouped-query attention on gfx950.
//
// Definition: cuDNN Frontend "Query Sparse Attention (QSA)" page, section
// "Selection and components" (same scores, softmax and products as the
// gathered kernels) and its note that the kernel computes dense tiles where
// a tile of queries selects a whole key span and gathers only for the rest.
// A tile is full when all 128 query rows select all 128 keys of the key tile
// ("fa4_qsa" page, `_block_kinds`: count == 128 * 128); such pairs are
// exactly the keys the partial key lists leave out.
//
// Design (one work group of four waves per query tile, KV head and block of
// 64 (row, head) vectors; two work groups share a CU, so one's set-up and
// final stores overlap the other's products):
//  * Inside a full tile every (row, head) vector of the tile sees the same
//    keys, so the MFMA blocks take 16 consecutive vectors of the tile (rows
//    and heads mixed) instead of the 12 heads of one row: no padding lanes.
//    A wave owns one such block (16 vectors), a work group 64, and the 24
//    work groups of a query tile are consecutive blocks, which the XCD-aware
//    mapping keeps on one XCD so the key tiles they share stay in its L2.
//  * Keys come in chunks of 32 from the tile row's full key tiles. A chunk's
//    K and V rows are contiguous, staged once per work group into LDS by
//    direct-to-LDS loads (each wave issues a quarter) in the swizzled layout
//    of the gathered forward, into two chunk buffers: the next chunk flies
//    while one is computed. A wave waits (counted) for its own loads of the
//    chunk, then the work-group barrier makes every wave's loads visible and
//    frees the buffer of the previous chunk for the next load. With one work
//    group per CU (eight waves, four buffers) the set-up and the final
//    stores of every work group were exposed: 8-11 % slower.
//  * S^T = K Q^T and O^T = V^T P^T exactly as in the gathered forward (K in
//    the row layout, V through the transposing read, P^T straight from the
//    accumulators, P as bf16 high + low), per vector block.
//  * The forward starts from the state the gathered pass handed over
//    (unnormalised output, reference maximum, sum) and rescales only when a
//    chunk rises more than 2^64 above the reference, which random-scale
//    scores never do; it then writes out_fp32, out and lse.
#include "common.h"

namespace qsa {

namespace {

constexpr int kDenseWaves = 4;  // one wave per SIMD; two work groups share a CU
constexpr int kVecBlocks = 1;                                  // 16-vector blocks per wave
constexpr int kGroupVecs = kDenseWaves * 16 * kVecBlocks;      // vectors per work group
constexpr int kTileVecs = kTile * kGroup;                      // vectors of a query tile
constexpr int kVBlocks = kTileVecs / kGroupVecs;               // work groups per query tile
constexpr int kXcdTiles = 16;   // query tiles of one XCD group (xcd_group_block)
constexpr int kKeys = 32;                                      // keys per staged chunk
constexpr int kHalf = kKeys * 512;                             // K (or V) bytes of a chunk
constexpr int kBuf = 2 * kHalf;                                // K then V
constexpr int kRing = 2;        // chunk buffers: one chunk in flight ahead
constexpr int kStage = 16 / kDenseWaves;  // staging instructions per wave and tensor
constexpr int kChunkOps = 2 * kStage;     // direct-to-LDS loads a wave issues per chunk
constexpr float kSlack = 64.f;  // log2 of the largest unnormalised P
static_assert(kTileVecs % kGroupVecs == 0, "work groups must tile the query tile");
static_assert(kDenseWaves * kStage == 16, "the waves share the 16 row pairs of a chunk");

// This wave's loads of chunk ch have landed once at most the loads of the
// chunks issued after it (up to kRing - 2 of them) are in flight.
__device__ __forceinline__ void wait_chunk(int ch, int nch)
{
    static_assert(kRing == 2 || kRing == 4, "counted waits for one or three chunks in flight");
    if (kRing == 4 && ch + 2 < nch) QSA_WAIT_VM(2 * kChunkOps);
    else if (kRing == 4 && ch + 1 < nch) QSA_WAIT_VM(kChunkOps);
    else QSA_WAIT_VM(0);
}

struct DenseTile {
    int64_t b, r;
    int g, vb;
};

// Work group -> (batch, KV head, query tile, vector block); the vector blocks
// of one query tile are consecutive logical blocks, and runs of kXcdTiles
// query tiles go to the XCDs in turn. With one contiguous range per XCD, the
// XCDs that held the ends of long documents carried most of a
// document-causal call's full tiles (its step took 39.5 ms instead of 33).
__device__ __forceinline__ bool dense_tile(const Problem &p, DenseTile &t)
{
    const int64_t item = xcd_group_block(blockIdx.x, kXcdTiles * kVBlocks);
    const int64_t per_bg = p.nQT * kVBlocks;
    if (item >= p.B * p.Hkv * per_bg) return false;
    const int64_t bg = item / per_bg;
    const int64_t rem = item - bg * per_bg;
    t.b = bg / p.Hkv;
    t.g = (int)(bg - t.b * p.Hkv);
    t.r = rem / kVBlocks;
    t.vb = (int)(rem - t.r * kVBlocks);
    return true;
}

typedef volatile __attribute__((address_space(3))) uint32_t lds_flag;

__device__ __forceinline__ void forward_dense_item(const Problem &p, lds_char *buf,
                                                   lds_flag *redo_flag)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    DenseTile dt;
    if (!dense_tile(p, dt)) return;
    const int64_t b = dt.b, r = dt.r;
    const int g = dt.g;
    const int fcnt = p.fwd_f_cnt[b * p.nQT + r];
    if (fcnt == 0) return;
    // The tile list was written by an earlier launch: read it as constant
    // data, which gives scalar loads.
    const __attribute__((address_space(4))) int32_t *fidx =
        (const __attribute__((address_space(4))) int32_t *)(p.fwd_f_idx + (b * p.nQT + r) * p.nKT);

    // Vector 16x + col of the wave: (row i, head) of the tile. Full tiles are
    // never edge tiles, so every row exists.
    int64_t vrow[kVecBlocks], sidx[kVecBlocks];
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x) {
        const int v = dt.vb * kGroupVecs + wave * 16 * kVecBlocks + 16 * x + col;
        const int rt = v / kGroup, hd = v - kGroup * rt;
        const int64_t i = r * kTile + rt;
        const int head = g * kGroup + hd;
        vrow[x] = (b * p.Sq + i) * p.Hq + head;
        sidx[x] = (b * p.Hq + head) * p.Sq + i;
    }

    // Q as the B operand: lane (vector col, quad) holds columns 32t + 8quad ..
    // +7 for step t. The handed-over state: reference maximum and sum.
    bf16x8 qf[kVecBlocks][8];
    float m_hand[kVecBlocks], l_hand[kVecBlocks], m_ref[kVecBlocks];
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x) {
        const uint16_t *qr = p.q + vrow[x] * kD + 8 * quad;
#pragma unroll
        for (int t = 0; t < 8; ++t) qf[x][t] = as_bf16x8(*reinterpret_cast<const uint4 *>(qr + 32 * t));
        const float2 st = *reinterpret_cast<const float2 *>(p.fstate + 2 * sidx[x]);
        m_hand[x] = st.x;
        l_hand[x] = st.y;
        m_ref[x] = -INFINITY;
    }
    // Settle these loads before the staging starts: the compiler cannot count
    // the assembly loads, and the counted waits in the loop are then the only
    // vector memory waits there.
    QSA_WAIT_VM(0);
    f32x4 acc[kVecBlocks][16];
    float l_part[kVecBlocks];

    // Staging: instruction s (0..15) puts key slot s (lanes 0..31) and s + 16
    // (lanes 32..63) of a chunk at s * 1024, lane l taking chunk
    // (l & 31) ^ swz_mask(s) of its row; wave w issues s = 2w, 2w+1 for K
    // and for V. The chunk's first key goes into the descriptors, so the lane
    // offsets never change.
    const uint32_t row_bytes = (uint32_t)(p.Hkv * kD * 2);
    const uint16_t *kbase = p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    const uint16_t *vbase = p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    uint32_t loff[kStage];
#pragma unroll
    for (int y = 0; y < kStage; ++y) {
        const int s = kStage * wave + y;
        loff[y] = (uint32_t)(s + 16 * (lane >> 5)) * row_bytes +
                  ((uint32_t)((lane & 31) ^ swz_mask(s)) << 4);
    }
    const uint32_t base = lds_addr(buf);
    auto issue = [&](int c) {
        const int64_t key0 = (int64_t)fidx[c >> 2] * kTile + (c & 3) * kKeys;
        const i32x4 rk = rsrc_words(kbase + key0 * p.Hkv * kD, kKeys * row_bytes);
        const i32x4 rv = rsrc_words(vbase + key0 * p.Hkv * kD, kKeys * row_bytes);
        const uint32_t dst = base + (uint32_t)((c % kRing) * kBuf);
#pragma unroll
        for (int y = 0; y < kStage; ++y) {
            const uint32_t s = (uint32_t)(kStage * wave + y);
            dma16_asm(rk, dst + s * 1024, loff[y]);
            dma16_asm(rv, dst + kHalf + s * 1024, loff[y]);
        }
    };

    // Reads as in the gathered forward: K row layout, lane (key slot col,
    // quad) takes chunk 4t + quad of slot kb*16 + col; V transposed, lane i of
    // group quad names the 8-byte unit of slot kb*16 + 4*quad + i/4 holding
    // columns 16db + 4(i%4) .. +3.
    const int kmask = swz_mask(col);
    const int vkey = 4 * quad + (col >> 2);
    const int vm = swz_mask(vkey);
    const int vlane = vkey * 1024 + ((((col >> 1) & 1) ^ (vm & 1)) << 4) + (col & 1) * 8;
    const int vxor = vm >> 1;
    const float c = p.scale * 1.4426950408889634f;  // scores in log2 units

    auto compute = [&](uint32_t cb, bool first, lds_flag *flag, auto rescale_tag) {
        constexpr bool kRescale = decltype(rescale_tag)::value;
        const lds_char *ks = (const lds_char *)(uintptr_t)cb;
        const lds_char *vs = ks + kHalf;
        // S^T for both key blocks: all sixteen K reads are issued first, and
        // the two blocks' products alternate (two independent chains).
        f32x4 st[kVecBlocks][2];
        uint4 kr[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                kr[kb][t] = lds_read16(ks + col * 1024 + 512 * kb + (((4 * t + quad) ^ kmask) << 4));
        // keep the reads ahead of the products (the scheduler would otherwise
        // trade them for registers and keep two in flight)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < kVecBlocks; ++x) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                a0 = mfma_16x16x32(as_bf16x8(kr[0][t]), qf[x][t], a0);
                a1 = mfma_16x16x32(as_bf16x8(kr[1][t]), qf[x][t], a1);
            }
            st[x][0] = a0;
            st[x][1] = a1;
        }
        bf16x8 pb_hi[kVecBlocks], pb_lo[kVecBlocks];
#pragma unroll
        for (int x = 0; x < kVecBlocks; ++x) {
            // lane holds key slots kb*16 + 4*quad + e of vector col
            float tv[8];
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    tv[kb * 4 + e] = st[x][kb][e] * c;
                    mx = fmaxf(mx, tv[kb * 4 + e]);
                }
            // The column maximum (over the four lane groups) is needed only
            // to fix or raise the reference; the overflow test is a ballot of
            // the lanes' own maxima, the same answer without the exchange.
            auto column_max = [&](float v) {
                v = fmaxf(v, __shfl_xor(v, 16));
                return fmaxf(v, __shfl_xor(v, 32));
            };
            // The first chunk fixes the reference (the sums are still zero;
            // the hand-over is added at the end, scaled to the reference).
            if (first) m_ref[x] = fmaxf(m_hand[x], column_max(mx));
            if (__builtin_amdgcn_ballot_w64(mx > m_ref[x] + kSlack) != 0) {
                mx = column_max(mx);
                if constexpr (kRescale) {
                    const float mn = fmaxf(m_ref[x], mx);
                    const float f = __builtin_amdgcn_exp2f(m_ref[x] - mn);
#pragma unroll
                    for (int db = 0; db < 16; ++db) acc[x][db] *= f;
                    l_part[x] *= f;
                    m_ref[x] = mn;
                } else {
                    // Rare: raise the reference and have the work group redo
                    // the full tiles from the hand-over on the rescaling path
                    // (an empty hand-over has -inf). This pass's sums are
                    // discarded, so P may keep using the raised reference.
                    m_ref[x] = fmaxf(m_ref[x], mx);
                    if (lane == 0) *flag = 1;
                }
            }
            float pr[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = __builtin_amdgcn_exp2f(tv[k] - m_ref[x]);
                l_part[x] += pr[k];
            }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split_bf16x2(pr[2 * k], pr[2 * k + 1], hi[k], lo[k]);
            pb_hi[x] = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
            pb_lo[x] = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
        // O^T += V^T P^T, V read in two halves of eight column blocks.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 va[2][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int o = vlane + (((8 * h + j) ^ vxor) << 5);
                va[0][j] = lds_read_tr(vs + o);
                va[1][j] = lds_read_tr(vs + o + 512);
            }
            __builtin_amdgcn_sched_barrier(0);  // all sixteen reads in flight
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int db = 8 * h + j;
                const bf16x8 v8 =
                    as_bf16x8(make_uint4(va[0][j].x, va[0][j].y, va[1][j].x, va[1][j].y));
#pragma unroll
                for (int x = 0; x < kVecBlocks; ++x) {
                    acc[x][db] = mfma_16x16x32(v8, pb_hi[x], acc[x][db]);
                    acc[x][db] = mfma_16x16x32(v8, pb_lo[x], acc[x][db]);
                }
            }
        }
    };

    const int nch = fcnt * (kTile / kKeys);
    // The dense sums start at zero: no vector instruction touches the
    // accumulators inside the loop, so they stay in the matrix-core registers.
    auto init = [&]() {
#pragma unroll
        for (int x = 0; x < kVecBlocks; ++x) {
#pragma unroll
            for (int db = 0; db < 16; ++db) acc[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};
            l_part[x] = 0.f;
        }
    };
    // One pass over the full tiles. Without rescaling, a wave that needs it
    // raises the flag of its chunk's parity; every wave reads that flag after
    // the next barrier, before any wave can write it again, so all leave
    // together and the pass reports it.
    auto pass = [&](auto rescale_tag) {
        constexpr bool kRescale = decltype(rescale_tag)::value;
        for (int c0 = 0; c0 < kRing - 1 && c0 < nch; ++c0) issue(c0);
        bool redo = false;
        for (int ch = 0; ch < nch; ++ch) {
            wait_chunk(ch, nch);
            asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
            if (!kRescale && ch > 0 &&
                opaque_u32(__builtin_amdgcn_readfirstlane(redo_flag[(ch - 1) & 1])) != 0u) {
                redo = true;
                break;
            }
            const uint32_t cb = opaque_u32(base + (uint32_t)((ch % kRing) * kBuf));
            if (ch + kRing - 1 < nch) issue(ch + kRing - 1);
            compute(cb, !kRescale && ch == 0, redo_flag + (ch & 1), rescale_tag);
        }
        QSA_WAIT_VM(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
        if (!kRescale && !redo)
            redo = opaque_u32(__builtin_amdgcn_readfirstlane(redo_flag[0] | redo_flag[1])) != 0u;
        return redo;
    };
    init();
    if (pass(std::false_type())) {
        init();
        pass(std::true_type());
    }

    // O = (dense sums + f * hand-over) / (dense sum + f * hand-over sum), with
    // f = 2^(m_hand - m_ref) (0 for an empty hand-over).
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x) {
        const float f = m_hand[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_hand[x] - m_ref[x]);
        float l = l_part[x] + __shfl_xor(l_part[x], 16);
        l += __shfl_xor(l, 32);
        l += l_hand[x] * f;
        const float inv = 1.f / l;
        float *of = p.out_fp32 + vrow[x] * kD + 4 * quad;
        uint16_t *ob = p.out + vrow[x] * kD + 4 * quad;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const float4 h = *reinterpret_cast<const float4 *>(of + 16 * db);
            const float o0 = (acc[x][db][0] + h.x * f) * inv, o1 = (acc[x][db][1] + h.y * f) * inv,
                        o2 = (acc[x][db][2] + h.z * f) * inv, o3 = (acc[x][db][3] + h.w * f) * inv;
            *reinterpret_cast<float4 *>(of + 16 * db) = make_float4(o0, o1, o2, o3);
            *reinterpret_cast<uint2 *>(ob + 16 * db) =
                make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
        if (quad == 0) p.lse[sidx[x]] = (m_ref[x] + log2f(l)) * 0.6931471805599453f;
    }
}

__global__ __launch_bounds__(64 * kDenseWaves) void k_forward_dense(Problem p)
{
    __shared__ __attribute__((aligned(16))) char buf[kRing * kBuf];
    __shared__ uint32_t redo_flag[2];
    if (threadIdx.x < 2) redo_flag[threadIdx.x] = 0;
    __syncthreads();
    forward_dense_item(p, (lds_char *)buf, (lds_flag *)redo_flag);
}

// dQ over full tiles: same tiling and staging as the forward. P = 2^(S c -
// lse log2 e) needs no running maximum; dS = P (dP - delta); dQ^T += K^T dS^T
// with dS as bf16 high + low and K^T through the transposing read of the
// staged K rows. The gathered pass handed over its unscaled FP32 sums.
__device__ __forceinline__ void dq_dense_item(const Problem &p, lds_char *buf)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    DenseTile dt;
    if (!dense_tile(p, dt)) return;
    const int64_t b = dt.b, r = dt.r;
    const int g = dt.g;
    const int fcnt = p.fwd_f_cnt[b * p.nQT + r];
    if (fcnt == 0) return;
    const __attribute__((address_space(4))) int32_t *fidx =
        (const __attribute__((address_space(4))) int32_t *)(p.fwd_f_idx + (b * p.nQT + r) * p.nKT);

    int64_t vrow[kVecBlocks];
    bf16x8 qf[kVecBlocks][8], gf[kVecBlocks][8];
    float lse2[kVecBlocks], dlt[kVecBlocks];
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x) {
        const int v = dt.vb * kGroupVecs + wave * 16 * kVecBlocks + 16 * x + col;
        const int rt = v / kGroup, hd = v - kGroup * rt;
        const int64_t i = r * kTile + rt;
        const int head = g * kGroup + hd;
        vrow[x] = (b * p.Sq + i) * p.Hq + head;
        const int64_t sidx = (b * p.Hq + head) * p.Sq + i;
        lse2[x] = p.lse_in[sidx] * 1.4426950408889634f;
        dlt[x] = p.delta[sidx];
        const uint16_t *qr = p.q + vrow[x] * kD + 8 * quad;
        const uint16_t *gr = p.dout + vrow[x] * kD + 8 * quad;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            qf[x][t] = as_bf16x8(*reinterpret_cast<const uint4 *>(qr + 32 * t));
            gf[x][t] = as_bf16x8(*reinterpret_cast<const uint4 *>(gr + 32 * t));
        }
    }
    QSA_WAIT_VM(0);  // as in the forward: settle before the staging starts
    f32x4 acc[kVecBlocks][16];
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x)
#pragma unroll
        for (int db = 0; db < 16; ++db) acc[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint32_t row_bytes = (uint32_t)(p.Hkv * kD * 2);
    const uint16_t *kbase = p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    const uint16_t *vbase = p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    uint32_t loff[kStage];
#pragma unroll
    for (int y = 0; y < kStage; ++y) {
        const int s = kStage * wave + y;
        loff[y] = (uint32_t)(s + 16 * (lane >> 5)) * row_bytes +
                  ((uint32_t)((lane & 31) ^ swz_mask(s)) << 4);
    }
    const uint32_t base = lds_addr(buf);
    auto issue = [&](int c) {
        const int64_t key0 = (int64_t)fidx[c >> 2] * kTile + (c & 3) * kKeys;
        const i32x4 rk = rsrc_words(kbase + key0 * p.Hkv * kD, kKeys * row_bytes);
        const i32x4 rv = rsrc_words(vbase + key0 * p.Hkv * kD, kKeys * row_bytes);
        const uint32_t dst = base + (uint32_t)((c % kRing) * kBuf);
#pragma unroll
        for (int y = 0; y < kStage; ++y) {
            const uint32_t s = (uint32_t)(kStage * wave + y);
            dma16_asm(rk, dst + s * 1024, loff[y]);
            dma16_asm(rv, dst + kHalf + s * 1024, loff[y]);
        }
    };

    // K and V in the row layout (A operands of S^T = K Q^T and dP^T = V dO^T),
    // K transposed (A operand of dQ^T = K^T dS^T), addressed as in the forward.
    const int kmask = swz_mask(col);
    const int tkey = 4 * quad + (col >> 2);
    const int tm = swz_mask(tkey);
    const int tlane = tkey * 1024 + ((((col >> 1) & 1) ^ (tm & 1)) << 4) + (col & 1) * 8;
    const int txor = tm >> 1;
    const float c = p.scale * 1.4426950408889634f;

    auto compute = [&](uint32_t cb) {
        const lds_char *ks = (const lds_char *)(uintptr_t)cb;
        const lds_char *vs = ks + kHalf;
        f32x4 st[kVecBlocks][2], pt[kVecBlocks][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint4 kr[8], vr[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int o = col * 1024 + 512 * kb + (((4 * t + quad) ^ kmask) << 4);
                kr[t] = lds_read16(ks + o);
                vr[t] = lds_read16(vs + o);
            }
            __builtin_amdgcn_sched_barrier(0);  // all sixteen reads in flight
#pragma unroll
            for (int x = 0; x < kVecBlocks; ++x) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    a = mfma_16x16x32(as_bf16x8(kr[t]), qf[x][t], a);
                    d = mfma_16x16x32(as_bf16x8(vr[t]), gf[x][t], d);
                }
                st[x][kb] = a;
                pt[x][kb] = d;
            }
        }
        bf16x8 ds_hi[kVecBlocks], ds_lo[kVecBlocks];
#pragma unroll
        for (int x = 0; x < kVecBlocks; ++x) {
            float ds[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pr = __builtin_amdgcn_exp2f(st[x][kb][e] * c - lse2[x]);
                    ds[kb * 4 + e] = pr * (pt[x][kb][e] - dlt[x]);
                }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split_bf16x2(ds[2 * k], ds[2 * k + 1], hi[k], lo[k]);
            ds_hi[x] = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
            ds_lo[x] = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 kt[2][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int o = tlane + (((8 * h + j) ^ txor) << 5);
                kt[0][j] = lds_read_tr(ks + o);
                kt[1][j] = lds_read_tr(ks + o + 512);
            }
            __builtin_amdgcn_sched_barrier(0);  // all sixteen reads in flight
            // the high parts of the half's eight column blocks, then the low
            // parts: no product waits on the one just before it
#pragma unroll
            for (int lo = 0; lo < 2; ++lo)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int db = 8 * h + j;
                const bf16x8 ka =
                    as_bf16x8(make_uint4(kt[0][j].x, kt[0][j].y, kt[1][j].x, kt[1][j].y));
#pragma unroll
                for (int x = 0; x < kVecBlocks; ++x)
                    acc[x][db] = mfma_16x16x32(ka, lo ? ds_lo[x] : ds_hi[x], acc[x][db]);
            }
        }
    };

    const int nch = fcnt * (kTile / kKeys);
    for (int c0 = 0; c0 < kRing - 1 && c0 < nch; ++c0) issue(c0);
    for (int ch = 0; ch < nch; ++ch) {
        wait_chunk(ch, nch);
        __builtin_amdgcn_s_barrier();
        const uint32_t cb = opaque_u32(base + (uint32_t)((ch % kRing) * kBuf));
        if (ch + kRing - 1 < nch) issue(ch + kRing - 1);
        compute(cb);
    }
    QSA_WAIT_VM(0);

    // dQ = scale * (dense sums + handed-over sums); lane holds dQ^T[d][vector].
#pragma unroll
    for (int x = 0; x < kVecBlocks; ++x) {
        const float *hp = p.dq_part + vrow[x] * kD + 4 * quad;
        uint16_t *dqp = p.dq + vrow[x] * kD + 4 * quad;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const float4 h = *reinterpret_cast<const float4 *>(hp + 16 * db);
            const float sc = p.scale;
            *reinterpret_cast<uint2 *>(dqp + 16 * db) =
                make_uint2(pack_bf16x2((acc[x][db][0] + h.x) * sc, (acc[x][db][1] + h.y) * sc),
                           pack_bf16x2((acc[x][db][2] + h.z) * sc, (acc[x][db][3] + h.w) * sc));
        }
    }
}

__global__ __launch_bounds__(64 * kDenseWaves) void k_dq_dense(Problem p)
{
    __shared__ __attribute__((aligned(16))) char buf[kRing * kBuf];
    dq_dense_item(p, (lds_char *)buf);
}

// dK and dV over full tiles. One work group per (part of the key tile's list
// of full query tiles, batch, KV head, key tile, half of it): a part is at
// most kDenseSplit query tiles of the list, so the long lists of key tiles at
// the start of causal documents are shared by several work groups instead of
// setting the run time alone (a 32768-token document-causal step went from
// 39 to 25 ms). Each of the four waves owns 16 keys (K and V rows in
// registers, dK and dV accumulators for the whole work group) and the work
// group streams the (row, head) vectors of the key tile's full query tiles in
// chunks of 32: Q, dO, lse and delta of a chunk are staged once, Q and dO in
// the forward's K-staging layout (slot j = vector j of the chunk), through two
// buffers; the kernel is held to 256 registers so that two work groups share
// a CU (15 % faster than one with four buffers). Per chunk a wave computes S = Q K^T and dP = dO V^T
// for its keys (two 16-vector blocks; lane (key col, quad) holds vectors
// 16x + 4 quad + i), P and dS, then dV += P^T dO and dK += dS^T Q with the
// two blocks' vectors as the 32-long contraction, exactly as the gathered
// pass pairs two rows (P and dS as bf16 high + low); the transposed Q and dO
// operands are read like V in the forward. The sums go to the part's partial
// slot, after the gathered pass's slots; the reduce adds them in slot order.
constexpr int kKvStats = 2 * kHalf;          // lse then delta of the chunk's vectors
constexpr int kKvBuf = kKvStats + 2 * 32 * 4;
constexpr int kChunksPerTile = kTileVecs / 32;
constexpr int kKvWaves = 4;                       // waves of a dK/dV work group, 16 keys each
constexpr int kKvStage = 16 / kKvWaves;           // Q (and dO) staging instructions per wave
constexpr int kKvChunkOps = 2 * kKvStage;         // direct-to-LDS loads a wave issues per chunk
constexpr int kKvParts = kTile / (16 * kKvWaves);  // work groups per key tile
static_assert(kKvParts * 16 * kKvWaves == kTile, "waves of 16 keys must tile the key tile");

constexpr int kKvRing = 2;  // dK/dV chunk buffers: one chunk in flight ahead
constexpr int kXcdKeyTiles = 8;  // key tiles of one XCD group (xcd_group_block)

template <int OPS>
__device__ __forceinline__ void wait_chunk_ops(int ch, int nch)
{
    static_assert(kKvRing == 2 || kKvRing == 4, "counted waits for one or three chunks in flight");
    if (kKvRing == 4 && ch + 2 < nch) QSA_WAIT_VM(2 * OPS);
    else if (kKvRing == 4 && ch + 1 < nch) QSA_WAIT_VM(OPS);
    else QSA_WAIT_VM(0);
}

__device__ __forceinline__ void dkdv_dense_item(const Problem &p, lds_char *buf)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;
    // Work group -> (part of the full-tile list, batch and KV head, key tile,
    // half of it); runs of kXcdKeyTiles key tiles go to the XCDs in turn.
    const int64_t per_part = p.B * p.Hkv * p.nKT * kKvParts;
    const int64_t item0 = xcd_group_block(blockIdx.x, kXcdKeyTiles * kKvParts);
    const int64_t part = item0 / per_part;
    if (part >= p.nslot - p.nseg) return;
    const int64_t item = item0 - part * per_part;
    const int64_t per_bg = p.nKT * kKvParts;
    const int64_t bg = item / per_bg;
    const int64_t rem = item - bg * per_bg;
    const int64_t b = bg / p.Hkv;
    const int g = (int)(bg - b * p.Hkv);
    const int64_t t = rem / kKvParts;
    const int64_t key0 = t * kTile + (rem - t * kKvParts) * (16 * kKvWaves) + 16 * wave;
    const int64_t ngroups = p.stride >> 4;
    uint8_t *flag = p.kv_flag + (bg * p.nslot + p.nseg + part) * ngroups + (key0 >> 4);
    // this part's entries of the tile column's list of full query tiles
    const int32_t f_all = p.rev_f_cnt[b * p.nKT + t];
    const int32_t j_lo = (int32_t)part * kDenseSplit;
    const int32_t fcnt = f_all - j_lo < 0 ? 0 : (f_all - j_lo < kDenseSplit ? f_all - j_lo : kDenseSplit);
    if (fcnt == 0) {  // the same for every wave of the group
        if (lane == 0) *flag = 0;
        return;
    }
    const int32_t *flist = p.rev_f_idx + (b * p.nKT + t) * p.nQT + j_lo;
    const __attribute__((address_space(4))) int32_t *ridx =
        (const __attribute__((address_space(4))) int32_t *)flist;

    // K and V of the wave's keys (all exist: full tiles are interior) as the B
    // operands of S and dP: lane (key col, quad) holds columns 32s + 8quad .. +7.
    bf16x8 kf[8], vf[8];
    {
        const int64_t kr = ((b * p.Skv + key0 + col) * p.Hkv + g) * (int64_t)kD + 8 * quad;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            kf[s8] = as_bf16x8(*reinterpret_cast<const uint4 *>(p.k + kr + 32 * s8));
            vf[s8] = as_bf16x8(*reinterpret_cast<const uint4 *>(p.v + kr + 32 * s8));
        }
    }
    QSA_WAIT_VM(0);  // settle before the staging starts
    f32x4 adk[16], adv[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Staging of chunk c: query tile ridx[(c / 48 + rot) mod fcnt], vectors
    // 32 (c % 48) + j.
    // Instruction s puts vectors s (lanes 0..31) and s + 16 (lanes 32..63) at
    // s * 1024, lane l taking chunk (l & 31) ^ swz_mask(s) of its vector; wave
    // w issues s = 4w .. 4w+3 for Q and for dO, wave 0 also lse and delta
    // (lane l < 32: vector l).
    const uint32_t tile_bytes = (uint32_t)((kTile - 1) * p.Hq * kD * 2 + kGroup * kD * 2);
    const uint32_t stat_bytes = (uint32_t)(((kGroup - 1) * p.Sq + kTile) * 4);
    const uint32_t base = lds_addr(buf);
    const uint32_t chunk16 = (uint32_t)(lane & 31) << 4;
    auto vec_off = [&](int v) { return (uint32_t)(((v / kGroup) * p.Hq + v % kGroup) * kD * 2); };
    // The walk over the tile column's full query tiles starts at the first
    // entry whose tile index is a multiple of the list length (else at the
    // first entry). Columns whose lists are the same-length windows shifted
    // by one tile (the recent-window part of causal routes) then visit the
    // same query tile at the same step, so the work groups of neighbouring
    // columns on one XCD stream each tile through its L2 together. The order
    // depends on the list only: results stay reproducible.
    int32_t rot = 0;
    for (int32_t j0 = 0; j0 < fcnt; j0 += 64) {
        const int32_t j = j0 + lane;
        const bool start = j < fcnt && (flist[j] % fcnt) == 0;
        const uint64_t ball = __ballot(start);
        if (ball != 0ull) {
            rot = j0 + (int32_t)__builtin_ctzll(ball);
            break;
        }
    }
    rot = __builtin_amdgcn_readfirstlane(rot);
    auto issue = [&](int c) {
        int32_t tj = c / kChunksPerTile + rot;
        tj = tj >= fcnt ? tj - fcnt : tj;
        const int64_t r = ridx[tj];
        const int cc = c % kChunksPerTile;
        const int64_t tb = ((b * p.Sq + r * kTile) * p.Hq + g * kGroup) * (int64_t)kD;
        const i32x4 rq = rsrc_words(p.q + tb, tile_bytes);
        const i32x4 rg = rsrc_words(p.dout + tb, tile_bytes);
        const uint32_t dst = base + (uint32_t)((c % kKvRing) * kKvBuf);
#pragma unroll
        for (int y = 0; y < kKvStage; ++y) {
            const int s = kKvStage * wave + y;
            const uint32_t o = vec_off(32 * cc + s + 16 * (lane >> 5)) + (chunk16 ^ ((uint32_t)swz_mask(s) << 4));
            dma16_asm(rq, dst + (uint32_t)s * 1024, o);
            dma16_asm(rg, dst + kHalf + (uint32_t)s * 1024, o);
        }
        if (wave == 0) {
            const int64_t sb = (b * p.Hq + g * kGroup) * p.Sq + r * kTile;
            i32x4 rl = rsrc_words(p.lse_in + sb, stat_bytes);
            i32x4 rd = rsrc_words(p.delta + sb, stat_bytes);
            // Keep the descriptors in scalar registers for the loads below.
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                rl[w4] = __builtin_amdgcn_readfirstlane(rl[w4]);
                rd[w4] = __builtin_amdgcn_readfirstlane(rd[w4]);
            }
            const int v = 32 * cc + (lane & 31);
            const uint32_t so = (uint32_t)(((v % kGroup) * p.Sq + v / kGroup) * 4);
            if (lane < 32) {
                dma4_asm(rl, dst + kKvStats, so);
                dma4_asm(rd, dst + kKvStats + 128, so);
            }
        }
    };

    // Reads: Q and dO in the row layout (A operands of S and dP; lane (vector
    // col, quad) takes chunk 4t + quad of slot 16x + col) and transposed (B
    // operands of dK and dV; lane i of group quad names the 8-byte unit of slot
    // 16x + 4 quad + i/4 holding columns 16db + 4(i%4) .. +3).
    const int amask = swz_mask(col);
    const int tvec = 4 * quad + (col >> 2);
    const int tm = swz_mask(tvec);
    const int tlane = tvec * 1024 + ((((col >> 1) & 1) ^ (tm & 1)) << 4) + (col & 1) * 8;
    const int txor = tm >> 1;
    const float c = p.scale * 1.4426950408889634f;

    auto compute = [&](uint32_t cb) {
        const lds_char *qs = (const lds_char *)(uintptr_t)cb;
        const lds_char *gs = qs + kHalf;
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        float pn[2][4], dn[2][4];
        // The two 16-vector blocks side by side: four independent product
        // chains per column step, the step's four reads in flight.
        f32x4 sa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 pd[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
            uint4 qa[2], ga[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int o = col * 1024 + 512 * x + (((4 * t8 + quad) ^ amask) << 4);
                qa[x] = lds_read16(qs + o);
                ga[x] = lds_read16(gs + o);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                sa[x] = mfma_16x16x32(as_bf16x8(qa[x]), kf[t8], sa[x]);
                pd[x] = mfma_16x16x32(as_bf16x8(ga[x]), vf[t8], pd[x]);
            }
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const f32x4 ls = *reinterpret_cast<const lds_f32x4 *>(qs + kKvStats + (16 * x + 4 * quad) * 4);
            const f32x4 dl = *reinterpret_cast<const lds_f32x4 *>(qs + kKvStats + 128 + (16 * x + 4 * quad) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pr = __builtin_amdgcn_exp2f(sa[x][e] * c - ls[e] * 1.4426950408889634f);
                pn[x][e] = pr;
                dn[x][e] = pr * (pd[x][e] - dl[e]);
            }
        }
        uint32_t ph[4], pl[4], dh[4], dlo[4];
        split_bf16x2(pn[0][0], pn[0][1], ph[0], pl[0]);
        split_bf16x2(pn[0][2], pn[0][3], ph[1], pl[1]);
        split_bf16x2(pn[1][0], pn[1][1], ph[2], pl[2]);
        split_bf16x2(pn[1][2], pn[1][3], ph[3], pl[3]);
        split_bf16x2(dn[0][0], dn[0][1], dh[0], dlo[0]);
        split_bf16x2(dn[0][2], dn[0][3], dh[1], dlo[1]);
        split_bf16x2(dn[1][0], dn[1][1], dh[2], dlo[2]);
        split_bf16x2(dn[1][2], dn[1][3], dh[3], dlo[3]);
        const bf16x8 A_p = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
        const bf16x8 A_pl = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
        const bf16x8 A_d = as_bf16x8(make_uint4(dh[0], dh[1], dh[2], dh[3]));
        const bf16x8 A_dl = as_bf16x8(make_uint4(dlo[0], dlo[1], dlo[2], dlo[3]));
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint2 tq[2][4], tg[2][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int o = tlane + (((4 * h + j) ^ txor) << 5);
                tq[0][j] = lds_read_tr(qs + o);
                tq[1][j] = lds_read_tr(qs + o + 512);
                tg[0][j] = lds_read_tr(gs + o);
                tg[1][j] = lds_read_tr(gs + o + 512);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int db = 4 * h + j;
                const bf16x8 Bg = as_bf16x8(make_uint4(tg[0][j].x, tg[0][j].y, tg[1][j].x, tg[1][j].y));
                const bf16x8 Bq = as_bf16x8(make_uint4(tq[0][j].x, tq[0][j].y, tq[1][j].x, tq[1][j].y));
                adv[db] = mfma_16x16x32(A_p, Bg, adv[db]);
                adv[db] = mfma_16x16x32(A_pl, Bg, adv[db]);
                adk[db] = mfma_16x16x32(A_d, Bq, adk[db]);
                adk[db] = mfma_16x16x32(A_dl, Bq, adk[db]);
            }
        }
    };

    const int nch = fcnt * kChunksPerTile;
    for (int c0 = 0; c0 < kKvRing - 1 && c0 < nch; ++c0) issue(c0);
    for (int ch = 0; ch < nch; ++ch) {
        if (wave == 0) wait_chunk_ops<kKvChunkOps + 2>(ch, nch);
        else wait_chunk_ops<kKvChunkOps>(ch, nch);
        __builtin_amdgcn_s_barrier();
        const uint32_t cb = opaque_u32(base + (uint32_t)((ch % kKvRing) * kKvBuf));
        if (ch + kKvRing - 1 < nch) issue(ch + kKvRing - 1);
        compute(cb);
    }
    QSA_WAIT_VM(0);

    // Lane holds dK/dV[key 4*quad+e][d 16*db + col].
    float *psum = p.kv_part + ((bg * p.nslot + p.nseg + part) * p.stride + key0) * (int64_t)(2 * kD);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float *pk = psum + (4 * quad + e) * (int64_t)(2 * kD) + col;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            pk[16 * db] = adk[db][e];
            pk[kD + 16 * db] = adv[db][e];
        }
    }
    if (lane == 0) *flag = 1;
}

__global__ __launch_bounds__(64 * kKvWaves, 2) void k_dkdv_dense(Problem p)
{
    __shared__ __attribute__((aligned(16))) char buf[kKvRing * kKvBuf];
    dkdv_dense_item(p, (lds_char *)buf);
}

}  // namespace

hipError_t launch_dkdv_dense(const Problem &p, hipStream_t s)
{
    const int64_t unit8 = 8 * kXcdKeyTiles * kKvParts;
    const int64_t items = ((p.nslot - p.nseg) * p.B * p.Hkv * p.nKT * kKvParts + unit8 - 1) / unit8 * unit8;
    hipLaunchKernelGGL(k_dkdv_dense, dim3((unsigned)items), dim3(64 * kKvWaves), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_forward_dense(const Problem &p, hipStream_t s)
{
    const int64_t unit8 = 8 * kXcdTiles * kVBlocks;
    const int64_t items = (p.B * p.Hkv * p.nQT * kVBlocks + unit8 - 1) / unit8 * unit8;
    hipLaunchKernelGGL(k_forward_dense, dim3((unsigned)items), dim3(64 * kDenseWaves), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_dq_dense(const Problem &p, hipStream_t s)
{
    const int64_t unit8 = 8 * kXcdTiles * kVBlocks;
    const int64_t items = (p.B * p.Hkv * p.nQT * kVBlocks + unit8 - 1) / unit8 * unit8;
    hipLaunchKernelGGL(k_dq_dense, dim3((unsigned)items), dim3(64 * kDenseWaves), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
