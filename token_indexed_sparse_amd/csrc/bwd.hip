// Backward of route-set grouped-query attention on gfx950.
//
// Definition: cuDNN Frontend "Query Sparse Attention (QSA)" page, section
// "Selection and components", backward equations: P = exp(S - lse) on the
// allowed keys and 0 elsewhere, delta = rowsum(dO * out_fp32), dP = dO V^T,
// dS = P (dP - delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, FP32
// accumulation, bf16 gradients, dK/dV summed over the query heads of a KV head.
//
// Three kernels, no floating-point atomics anywhere:
//  * k_delta: one wave per (row, head) reduces dO . out_fp32.
//  * k_dq: query-major like the forward (one wave per row and KV head walks
//    the row's sorted key list in 32-slot chunks; each chunk's K and V rows
//    are gathered straight into LDS by direct-to-LDS loads, read out, and the
//    next chunk's gathers fly while this chunk is computed). S^T = K Q^T and
//    dP^T = V dO^T take K and V in the row layout; dS^T stays in the
//    accumulator layout and is the B operand of dQ^T = K^T dS^T, whose K^T
//    operand is the transposed read of the same staged K rows.
//  * k_dkdv: key-major. One wave owns 16 consecutive keys of one KV head and
//    keeps their K and V rows in registers and their dK, dV accumulators for
//    the whole run. It walks the reverse tile lists of its 128-key tile column
//    from the last query tile down, reads a 16-bit slice of the bit-packed
//    membership row of every query in those tiles, and collects the rows that
//    select one of its keys into an LDS list (descending). Rows are then
//    processed in that order with two rows' Q, dO, lse and delta loads in
//    flight: S = Q K^T and dP = dO V^T per row (M = heads), then, two rows at
//    a time, dV += P^T dO and dK += dS^T Q with the two rows' heads forming the
//    32-long contraction. Q and dO rows are staged in LDS and read transposed.
//    P and dS enter these products (and dS the dQ product) as bf16 high + low
//    parts, so that sums over thousands of query heads keep FP32-level error.
//    The descending sweep keeps every wave near the same query rows (random
//    selections have one density per query position), and blocks are mapped
//    XCD-aware so neighbouring key groups share an L2.
#include "common.h"

namespace qsa {

namespace {

// ---------------------------------------------------------------- delta
__global__ __launch_bounds__(256) void k_delta(Problem p)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;  // (row, head)
    if (item >= p.B * p.Sq * p.Hq) return;
    const int64_t row = item / p.Hq;
    const int h = (int)(item - row * p.Hq);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int64_t base = item * (int64_t)kD + lane * 4;
    const float4 o = *reinterpret_cast<const float4 *>(p.out_fp32_in + base);
    const uint2 g = *reinterpret_cast<const uint2 *>(p.dout + base);
    float s = o.x * bf16_to_f32((uint16_t)(g.x & 0xffff)) + o.y * bf16_to_f32((uint16_t)(g.x >> 16)) +
              o.z * bf16_to_f32((uint16_t)(g.y & 0xffff)) + o.w * bf16_to_f32((uint16_t)(g.y >> 16));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) p.delta[(b * p.Hq + h) * p.Sq + i] = s;
}

// ---------------------------------------------------------------- dQ
constexpr int kChunk = 32;  // key slots per step

// Body of k_dq; ks and vs are the wave's K and V staging regions (32 rows of
// 512 bytes each, swizzled as described with swz()).
__device__ __forceinline__ void dq_row(const Problem &p, lds_char *ks, lds_char *vs)
{
    const int lane = threadIdx.x;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t item = xcd_logical_block(blockIdx.x, gridDim.x);
    if (item >= p.B * p.Sq * p.Hkv) return;
    const int64_t row = item / p.Hkv;
    const int g = (int)(item - row * p.Hkv);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int head = g * kGroup + col;
    const bool hv = col < kGroup;
    const int n = p.row_cnt[row];
    uint16_t *dqp = p.dq + (row * p.Hq + head) * (int64_t)kD;

    f32x4 acc[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n > 0) {
        const uint32_t row_bytes = (uint32_t)(p.Hkv * kD * 2);
        const uint32_t kv_bytes = (uint32_t)((p.Skv - 1) * p.Hkv * kD * 2 + kD * 2);
        const rsrc_t rk = make_rsrc(p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        const rsrc_t rv = make_rsrc(p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        // Q and dO as B operands: lane (head col, quad) holds columns
        // 32t + 8quad .. +7 for step t.
        bf16x8 qf[8], gf[8];
        float lse2 = 0.f, dlt = 0.f;
        {
            const int64_t rbase = (row * p.Hq + g * kGroup) * (int64_t)kD;
            const rsrc_t rq = make_rsrc(p.q + rbase, (uint32_t)(kGroup * kD * 2));
            const rsrc_t rg = make_rsrc(p.dout + rbase, (uint32_t)(kGroup * kD * 2));
            const uint32_t off = hv ? (uint32_t)(col * kD * 2 + quad * 16) : kOutOfRange;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                qf[t] = as_bf16x8(buf_load16(rq, off + 64 * t));
                gf[t] = as_bf16x8(buf_load16(rg, off + 64 * t));
            }
            if (hv) {
                lse2 = p.lse_in[(b * p.Hq + head) * p.Sq + i] * 1.4426950408889634f;
                dlt = p.delta[(b * p.Hq + head) * p.Sq + i];
            }
            QSA_WAIT_VM(0);  // the counted waits below are then the only ones
        }
        const float c = p.scale * 1.4426950408889634f;
        const rsrc_t rkeys = make_rsrc(p.row_keys + row * p.W, (uint32_t)(p.W * 4));
        auto fetch_key = [&](int ch) -> int {
            const int slot = ch * kChunk + (lane & 31);
            const int kk = (int)__builtin_amdgcn_raw_buffer_load_b32(
                rkeys, slot < n ? (uint32_t)slot * 4 : kOutOfRange, 0, 0);
            return slot < n ? kk : -1;
        };
        auto offsets = [&](int kk, uint32_t (&off)[16]) {
            const uint32_t mine = kk >= 0 ? (uint32_t)kk * row_bytes : kOutOfRange;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const uint32_t e = __builtin_amdgcn_readlane(mine, 2 * s);
                const uint32_t o = __builtin_amdgcn_readlane(mine, 2 * s + 1);
                off[s] = ((lane >> 5) ? o : e) + ((uint32_t)dma_chunk(lane, s) << 4);
            }
        };
        auto gather = [&](rsrc_t r, lds_char *dst, const uint32_t (&off)[16]) {
#pragma unroll
            for (int s = 0; s < 16; ++s) dma16(r, dst + s * 1024, off[s]);
        };
        // Row-layout reads (A operands of S^T = K Q^T and dP^T = V dO^T) and
        // the transposed read of K (A operand of dQ^T = K^T dS^T), as in the
        // forward's K and V reads.
        const int kmask = swz_mask(col);
        const int tkey = 4 * quad + (col >> 2);
        const int tm = swz_mask(tkey);
        const int tbase = tkey * 512 + ((((col >> 1) & 1) ^ (tm & 1)) << 4) + (col & 1) * 8;
        const int txor = tm >> 1;

        const int nchunks = (n + kChunk - 1) / kChunk;
        int knext = fetch_key(1);
        uint32_t off[16];
        offsets(fetch_key(0), off);
        gather(rk, ks, off);
        gather(rv, vs, off);
        for (int ch = 0; ch < nchunks; ++ch) {
            // Read the whole chunk out of LDS, then gather the next one (the
            // compiler orders LDS reads after all earlier direct-to-LDS loads).
            QSA_WAIT_VM(0);
            offsets(knext, off);
            knext = fetch_key(ch + 2);
            uint4 kr[2][8], vr[2][8];
            uint2 kt[2][16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int o = (kb * 16 + col) * 512 + (((4 * t + quad) ^ kmask) << 4);
                    kr[kb][t] = lds_read16(ks + o);
                    vr[kb][t] = lds_read16(vs + o);
                }
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const int o = tbase + ((db ^ txor) << 5);
                kt[0][db] = lds_read_tr(ks + o);
                kt[1][db] = lds_read_tr(ks + o + 16 * 512);
            }
            QSA_WAIT_LDS();
            gather(rk, ks, off);
            gather(rv, vs, off);

            float ds[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    sa = mfma_16x16x32(as_bf16x8(kr[kb][t]), qf[t], sa);
                    pa = mfma_16x16x32(as_bf16x8(vr[kb][t]), gf[t], pa);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool valid = hv && (ch * kChunk + kb * 16 + 4 * quad + e < n);
                    const float pr = valid ? exp2f(sa[e] * c - lse2) : 0.f;
                    // select, never multiply: a padding slot's dP is not used
                    ds[kb * 4 + e] = valid ? pr * (pa[e] - dlt) : 0.f;
                }
            }
            uint32_t dsh[4], dsl[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) split_bf16x2(ds[2 * x], ds[2 * x + 1], dsh[x], dsl[x]);
            const bf16x8 dsv_hi = as_bf16x8(make_uint4(dsh[0], dsh[1], dsh[2], dsh[3]));
            const bf16x8 dsv_lo = as_bf16x8(make_uint4(dsl[0], dsl[1], dsl[2], dsl[3]));
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const bf16x8 ka =
                    as_bf16x8(make_uint4(kt[0][db].x, kt[0][db].y, kt[1][db].x, kt[1][db].y));
                acc[db] = mfma_16x16x32(ka, dsv_hi, acc[db]);
                acc[db] = mfma_16x16x32(ka, dsv_lo, acc[db]);
            }
        }
        QSA_WAIT_VM(0);  // no gather may outlive the wave's LDS
    }
    if (!hv) return;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        const int d = 16 * db + 4 * quad;
        const float s = p.scale;
        *reinterpret_cast<uint2 *>(dqp + d) =
            make_uint2(pack_bf16x2(acc[db][0] * s, acc[db][1] * s),
                       pack_bf16x2(acc[db][2] * s, acc[db][3] * s));
    }
}

__global__ __launch_bounds__(64) void k_dq(Problem p)
{
    __shared__ __attribute__((aligned(16))) char ks[kChunk * 512];
    __shared__ __attribute__((aligned(16))) char vs[kChunk * 512];
    dq_row(p, (lds_char *)ks, (lds_char *)vs);
}

// ---------------------------------------------------------------- dK, dV
constexpr int kKvWaves = 2;
constexpr int kHitCap = 448;    // LDS hit list capacity per wave
constexpr int kHitBatch = 192;  // stop scanning once this many hits are listed
constexpr int kScanWin = 4;     // 64-row windows scanned per step

struct RowOps {
    uint4 q[8], g[8];
    float lse[4], dl[4];
};

__global__ __launch_bounds__(kKvWaves * 64) void k_dkdv(Problem p)
{
    // Per wave: Q and dO of two query rows in the transposed staging layout,
    // and the list of (row, 16-bit mask) hits.
    __shared__ __attribute__((aligned(16))) char st_all[kKvWaves][4 * kTrBlock];
    __shared__ int32_t hit_row[kKvWaves][kHitCap];
    __shared__ uint32_t hit_mask[kKvWaves][kHitCap];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t ngroups = p.stride >> 4;
    // item = (b * Hkv + g) * ngroups + kg. Blocks go to the XCDs round-robin,
    // so the key groups at the start of a causal range, which every later row
    // can select and which carry the most hits, are spread over all XCDs.
    const int64_t item = (int64_t)blockIdx.x * kKvWaves + wave;
    if (item >= p.B * p.Hkv * ngroups) return;
    const int64_t kg = item % ngroups;
    const int64_t bg = item / ngroups;
    const int g = (int)(bg % p.Hkv);
    const int64_t b = bg / p.Hkv;
    const int64_t key0 = kg * 16;
    if (key0 >= p.Skv) return;
    const int64_t t = key0 >> 7;
    char *stq[2] = {st_all[wave], st_all[wave] + kTrBlock};
    char *stg[2] = {st_all[wave] + 2 * kTrBlock, st_all[wave] + 3 * kTrBlock};
    int32_t *hrow = hit_row[wave];
    uint32_t *hmask = hit_mask[wave];

    // Clear the staging area: rows 12..15 (heads past the group) stay zero.
    for (int o = lane * 16; o < 4 * kTrBlock; o += 64 * 16)
        *reinterpret_cast<uint4 *>(st_all[wave] + o) = zero_u4();

    // K and V rows of the 16 keys as B operands of S = Q K^T and dP = dO V^T.
    bf16x8 kf[8], vf[8];
    {
        const uint32_t kv_bytes = (uint32_t)((p.Skv - 1) * p.Hkv * kD * 2 + kD * 2);
        const rsrc_t rk = make_rsrc(p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        const rsrc_t rv = make_rsrc(p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        const int64_t key = key0 + col;
        const uint32_t off =
            key < p.Skv ? (uint32_t)(key * p.Hkv * kD * 2 + quad * 128) : kOutOfRange;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            kf[s] = as_bf16x8(buf_load16(rk, off + 16 * s));
            vf[s] = as_bf16x8(buf_load16(rv, off + 16 * s));
        }
    }
    f32x4 adk[16], adv[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c = p.scale * 1.4426950408889634f;
    const bool hq = quad < 3;      // accumulator rows 4*quad+e are real heads
    const bool hv = col < kGroup;  // lane loads head `col` of a Q/dO row
    const int tr_lane = lane_tr_base(col, quad);

    // Q/dO rows of this batch and group; lse/delta of this batch and group.
    const uint32_t q_bytes = (uint32_t)((p.Sq - 1) * p.Hq * kD * 2 + kGroup * kD * 2);
    const rsrc_t rq = make_rsrc(p.q + (b * p.Sq * p.Hq + g * kGroup) * (int64_t)kD, q_bytes);
    const rsrc_t rg = make_rsrc(p.dout + (b * p.Sq * p.Hq + g * kGroup) * (int64_t)kD, q_bytes);
    const rsrc_t rl = make_rsrc(p.lse_in + (b * p.Hq + g * kGroup) * p.Sq,
                                (uint32_t)(kGroup * p.Sq * 4));
    const rsrc_t rd = make_rsrc(p.delta + (b * p.Hq + g * kGroup) * p.Sq,
                                (uint32_t)(kGroup * p.Sq * 4));
    auto load_row = [&](RowOps &R, int64_t qi) {
        const uint32_t off =
            hv ? (uint32_t)(qi * p.Hq * kD * 2 + col * kD * 2 + quad * 128) : kOutOfRange;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            R.q[s] = buf_load16(rq, off + 16 * s);
            R.g[s] = buf_load16(rg, off + 16 * s);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = hq ? (uint32_t)(((4 * quad + e) * p.Sq + qi) * 4) : kOutOfRange;
            R.lse[e] =
                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, lo, 0, 0));
            R.dl[e] =
                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, lo, 0, 0));
        }
    };

    float pa[4] = {0.f, 0.f, 0.f, 0.f}, da[4] = {0.f, 0.f, 0.f, 0.f};
    int filled = 0;

    // Contract the staged pair into dV and dK. Slot j of lane group quad is
    // head 4*quad + (j & 3) of row (j < 4 ? first : second).
    auto flush = [&](const float *pb, const float *db_) {
        uint32_t ph[4], pl[4], dh[4], dl[4];
        split_bf16x2(pa[0], pa[1], ph[0], pl[0]);
        split_bf16x2(pa[2], pa[3], ph[1], pl[1]);
        split_bf16x2(pb[0], pb[1], ph[2], pl[2]);
        split_bf16x2(pb[2], pb[3], ph[3], pl[3]);
        split_bf16x2(da[0], da[1], dh[0], dl[0]);
        split_bf16x2(da[2], da[3], dh[1], dl[1]);
        split_bf16x2(db_[0], db_[1], dh[2], dl[2]);
        split_bf16x2(db_[2], db_[3], dh[3], dl[3]);
        const bf16x8 A_p = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
        const bf16x8 A_pl = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
        const bf16x8 A_d = as_bf16x8(make_uint4(dh[0], dh[1], dh[2], dh[3]));
        const bf16x8 A_dl = as_bf16x8(make_uint4(dl[0], dl[1], dl[2], dl[3]));
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            uint2 ga[2], gb[2], qa[2], qb[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int o = tr_lane + tile_tr_offset(2 * h + x);
                ga[x] = lds_read_tr(stg[0] + o);
                gb[x] = lds_read_tr(stg[1] + o);
                qa[x] = lds_read_tr(stq[0] + o);
                qb[x] = lds_read_tr(stq[1] + o);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int dbk = 2 * h + x;
                const bf16x8 Bg = as_bf16x8(make_uint4(ga[x].x, ga[x].y, gb[x].x, gb[x].y));
                const bf16x8 Bq = as_bf16x8(make_uint4(qa[x].x, qa[x].y, qb[x].x, qb[x].y));
                adv[dbk] = mfma_16x16x32(A_p, Bg, adv[dbk]);
                adv[dbk] = mfma_16x16x32(A_pl, Bg, adv[dbk]);
                adk[dbk] = mfma_16x16x32(A_d, Bq, adk[dbk]);
                adk[dbk] = mfma_16x16x32(A_dl, Bq, adk[dbk]);
            }
        }
        wave_lds_sync();
    };

    // One query row: S, dP, then P and dS, staged Q/dO, and the pair flush.
    auto process = [&](const RowOps &R, uint32_t mask) {
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            sa = mfma_16x16x32(as_bf16x8(R.q[s]), kf[s], sa);
            pd = mfma_16x16x32(as_bf16x8(R.g[s]), vf[s], pd);
        }
        if (hv) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                tr_store8(stq[filled], col, quad * 64 + 8 * s, R.q[s]);
                tr_store8(stg[filled], col, quad * 64 + 8 * s, R.g[s]);
            }
        }
        // Lane holds S[head 4*quad+e][key col].
        const bool on = hq && ((mask >> col) & 1u);
        float pn[4], dn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float pr = on ? exp2f(sa[e] * c - R.lse[e] * 1.4426950408889634f) : 0.f;
            pn[e] = pr;
            // select, never multiply: an unselected key's dP may be non-finite
            dn[e] = on ? pr * (pd[e] - R.dl[e]) : 0.f;
        }
        if (filled == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pa[e] = pn[e];
                da[e] = dn[e];
            }
            filled = 1;
        } else {
            flush(pn, dn);
            filled = 0;
        }
    };

    // Hits are visited in DESCENDING query order: random selections have the
    // same density for every key group at a given query position, so all waves
    // sweep the query range from the top at about the same rate and the rows
    // they read stay in the caches. Window w (counted from the top) covers
    // rows 64*(w%2) .. of the reverse-list query tiles (full tiles, then
    // partial tiles, both from their last entry down).
    const int64_t bt = b * p.nKT + t;
    const int32_t cnt_p = p.rev_p_cnt[bt], cnt_f = p.rev_f_cnt[bt];
    const int32_t *idx_p = p.rev_p_idx + bt * p.nQT, *idx_f = p.rev_f_idx + bt * p.nQT;
    const int64_t nwin = 2 * ((int64_t)cnt_p + cnt_f);
    const int64_t mstride = p.stride >> 5;
    const uint32_t *mrow = p.mbits + (b * p.Sq) * mstride + (key0 >> 5);
    const int shift = (int)(key0 & 16);
    const uint64_t above = (lane == 63) ? 0ull : (~0ull << (lane + 1));

    int64_t w = 0;
    int32_t ip = cnt_p - 1, jf = cnt_f - 1;  // cursors merging both lists from the top
    int32_t cur_tile = -1;
    RowOps R0, R1, R2;
    while (w < nwin) {
        // Collect hits, kScanWin windows per step, until a batch is listed.
        int nh = 0;
        while (w < nwin && nh < kHitBatch) {
            uint32_t m[kScanWin];
            int64_t rbase[kScanWin];
#pragma unroll
            for (int x = 0; x < kScanWin; ++x) {
                m[x] = 0u;
                rbase[x] = 0;
                if (w + x < nwin) {
                    if (((w + x) & 1) == 0) {
                        // next tile from the top of the merged lists
                        const int32_t vp = ip >= 0 ? idx_p[ip] : -1;
                        const int32_t vf = jf >= 0 ? idx_f[jf] : -1;
                        if (vp > vf) {
                            cur_tile = vp;
                            --ip;
                        } else {
                            cur_tile = vf;
                            --jf;
                        }
                    }
                    rbase[x] = (int64_t)cur_tile * kTile + (((w + x) & 1) ? 0 : 64);
                    const int64_t qi = rbase[x] + lane;
                    if (qi < p.Sq) m[x] = (mrow[qi * mstride] >> shift) & 0xffffu;
                }
            }
#pragma unroll
            for (int x = 0; x < kScanWin; ++x) {
                const uint64_t ball = __ballot(m[x] != 0u);
                if (m[x] != 0u) {
                    const int pos = nh + __popcll(ball & above);
                    hrow[pos] = (int32_t)(rbase[x] + lane);
                    hmask[pos] = m[x];
                }
                nh += __popcll(ball);
            }
            w += kScanWin;
        }
        wave_lds_sync();
        // Process the batch in order, two rows' operands in flight.
        if (nh > 0) load_row(R0, hrow[0]);
        if (nh > 1) load_row(R1, hrow[1]);
        for (int h = 0; h < nh; h += 3) {
            if (h + 2 < nh) load_row(R2, hrow[h + 2]);
            __builtin_amdgcn_sched_barrier(0);
            process(R0, hmask[h]);
            if (h + 1 >= nh) break;
            if (h + 3 < nh) load_row(R0, hrow[h + 3]);
            __builtin_amdgcn_sched_barrier(0);
            process(R1, hmask[h + 1]);
            if (h + 2 >= nh) break;
            if (h + 4 < nh) load_row(R1, hrow[h + 4]);
            __builtin_amdgcn_sched_barrier(0);
            process(R2, hmask[h + 2]);
        }
        wave_lds_sync();
    }
    if (filled) {
        // Second row of the last pair is empty: clear its staged rows.
        const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
        if (hv) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                tr_store8(stq[1], col, quad * 64 + 8 * s, zero_u4());
                tr_store8(stg[1], col, quad * 64 + 8 * s, zero_u4());
            }
        }
        flush(zero4, zero4);
    }

    // Lane holds dK/dV[key 4*quad+e][d 16*db + col].
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        const int64_t key = key0 + 4 * quad + e2;
        if (key >= p.Skv) continue;
        uint16_t *dkp = p.dk + ((b * p.Skv + key) * p.Hkv + g) * (int64_t)kD + col;
        uint16_t *dvp = p.dv + ((b * p.Skv + key) * p.Hkv + g) * (int64_t)kD + col;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            dkp[16 * db] = f32_to_bf16(adk[db][e2] * p.scale);
            dvp[16 * db] = f32_to_bf16(adv[db][e2]);
        }
    }
}

}  // namespace

hipError_t launch_delta(const Problem &p, hipStream_t s)
{
    const int64_t rows_heads = p.B * p.Sq * p.Hq;
    hipLaunchKernelGGL(k_delta, dim3((unsigned)((rows_heads + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_dq(const Problem &p, hipStream_t s)
{
    const int64_t items = p.B * p.Sq * p.Hkv;
    hipLaunchKernelGGL(k_dq, dim3((unsigned)items), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_dkdv(const Problem &p, hipStream_t s)
{
    const int64_t groups = p.B * p.Hkv * (p.stride >> 4);
    hipLaunchKernelGGL(k_dkdv, dim3((unsigned)((groups + kKvWaves - 1) / kKvWaves)),
                       dim3(kKvWaves * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
