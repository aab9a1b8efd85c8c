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
//    the row's sorted key list in 16-slot chunks, two waves per SIMD; each chunk's K and V rows
//    are gathered straight into LDS by direct-to-LDS loads; the V region is
//    refilled with the next chunk's rows once its rows are read, the K region
//    once the transposed K read for dQ is done). S^T = K Q^T and
//    dP^T = V dO^T take K and V in the row layout; dS^T stays in the
//    accumulator layout and is the B operand of dQ^T = K^T dS^T, whose K^T
//    operand is the transposed read of the same staged K rows. The high and
//    low bf16 parts of dS go through one 16x16x32 MFMA whose K = 32 covers
//    the 16 key slots twice, as the forward does with P.
//  * k_dkdv: key-major. One wave owns 16 consecutive keys of one KV head and
//    one segment of query tiles (2 by default, more when the partial sums
//    would not fit the workspace budget). Segments are grouped 8 tiles at a
//    time: k_dkdv_split counts, per group and 16-key group, the rows that
//    select one of the keys, and a group with at most 256 such rows is one
//    work item (its first segment's; the others exit), while a heavier group
//    runs each segment as its own item. Light groups thus keep few partial
//    sums, and the heavy groups of rows near the start of a document (which
//    select every earlier block) no longer leave one wave with a thousand
//    rows. The wave keeps the 16 K and V rows in registers and
//    their dK, dV accumulators for the whole item. It walks the partial
//    entries of the reverse tile list of its 128-key tile column inside the
//    segment from the last query tile down (full tiles are summed by the dense
//    pass), reads a 16-bit slice of the bit-packed membership row of every
//    query in those tiles, and lists the rows that select one of its keys in
//    LDS. Each listed row's Q and dO (12 heads x 512 bytes each), lse and
//    delta are gathered into a 3-slot LDS ring by direct-to-LDS loads (a
//    slot takes the row three ahead once its reads have returned), then read
//    in the row layout (A operands of S = Q K^T and dP = dO V^T, M = heads)
//    and transposed (B operands of dV += P^T dO and dK += dS^T Q, whose
//    32-long contraction takes the row's heads twice: high parts, then low
//    parts). P and dS enter these products (and dS the dQ product) as bf16
//    high + low parts, so that sums over thousands of query heads keep
//    FP32-level error.
//  * k_dkdv_reduce: the FP32 partial sums of the segments and then of the
//    dense full-tile pass's parts are added in that fixed order
//    (deterministic, no atomics) and written as bf16 dK, dV.
//    Splitting the long causal key columns into segments keeps every SIMD
//    busy to the end: the first key groups are selected by almost every later
//    row and would otherwise dominate the run time.
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
constexpr int kChunk = 16;  // key slots per step (one 16-slot MFMA block)

// Body of k_dq; ks and vs are the wave's K and V staging regions (16 rows of
// 512 bytes each, swizzled as described with swz()).
__device__ __forceinline__ void dq_row(const Problem &p, lds_char *ks, lds_char *vs)
{
    const int lane = threadIdx.x;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x;
    if (item >= p.B * p.Sq * p.Hkv) return;
    const int64_t row = item / p.Hkv;
    const int g = (int)(item - row * p.Hkv);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int head = g * kGroup + col;
    const bool hv = col < kGroup;
    // Keys of partial tiles only; when the row's tile row has full tiles the
    // dense pass adds them and writes dQ, and this pass hands over its
    // unscaled FP32 sums instead.
    const int n = p.pcnt[row];
    const bool handoff = p.fwd_f_cnt[b * p.nQT + (i >> 7)] > 0;
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
        const rsrc_t rkeys = make_rsrc(p.pkeys + row * p.W, (uint32_t)(p.W * 4));
        auto fetch_key = [&](int ch) -> int {
            const int slot = ch * kChunk + (lane & 15);
            const int kk = (int)__builtin_amdgcn_raw_buffer_load_b32(
                rkeys, slot < n ? (uint32_t)slot * 4 : kOutOfRange, 0, 0);
            return slot < n ? kk : -1;
        };
        auto offsets = [&](int kk, uint32_t (&off)[8]) {
            const uint32_t mine = kk >= 0 ? (uint32_t)kk * row_bytes : kOutOfRange;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t e = __builtin_amdgcn_readlane(mine, 2 * s);
                const uint32_t o = __builtin_amdgcn_readlane(mine, 2 * s + 1);
                off[s] = ((lane >> 5) ? o : e) + ((uint32_t)dma_chunk(lane, s) << 4);
            }
        };
        auto gather = [&](rsrc_t r, lds_char *dst, const uint32_t (&off)[8]) {
#pragma unroll
            for (int s = 0; s < 8; ++s) dma16(r, dst + s * 1024, off[s]);
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
        // Walk rotation aligned with the rows in flight, as in the forward
        // (its own clock).
        uint32_t *const clk = p.walk ? p.walk + 8 : nullptr;
        int rot = 0;
        if (clk && nchunks > 1) {
            const uint32_t done = __hip_atomic_fetch_add(clk, opaque_u32(0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            rot = (int)__builtin_amdgcn_readfirstlane((done / p.walk_slots) % (uint32_t)nchunks);
        }
        auto phys = [&](int x) {
            return x >= nchunks ? x : (x + rot >= nchunks ? x + rot - nchunks : x + rot);
        };
        int knext = fetch_key(phys(1));
        uint32_t off[8];
        offsets(fetch_key(phys(0)), off);
        gather(rk, ks, off);
        gather(rv, vs, off);
        for (int ch = 0; ch < nchunks; ++ch) {
            // Read the whole chunk out of LDS, then gather the next one (the
            // compiler orders LDS reads after all earlier direct-to-LDS loads).
            QSA_WAIT_VM(0);
            offsets(knext, off);
            knext = fetch_key(phys(ch + 2));
            const int pc = phys(ch);  // the chunk's place in the list
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
            {
                uint4 kr[8], vr[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int o = col * 512 + (((4 * t + quad) ^ kmask) << 4);
                    kr[t] = lds_read16(ks + o);
                    vr[t] = lds_read16(vs + o);
                }
                QSA_WAIT_LDS();  // the V region is free
                gather(rv, vs, off);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    hold_after(kr[t]);
                    hold_after(vr[t]);
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    sa = mfma_16x16x32(as_bf16x8(kr[t]), qf[t], sa);
                    pa = mfma_16x16x32(as_bf16x8(vr[t]), gf[t], pa);
                }
            }
            uint2 kt[16];
            {
                const lds_char *ksr = (const lds_char *)(uintptr_t)opaque_u32(lds_addr(ks));
#pragma unroll
                for (int db = 0; db < 16; ++db) kt[db] = lds_read_tr(ksr + tbase + ((db ^ txor) << 5));
            }
            QSA_WAIT_LDS();  // the K region is free
            gather(rk, ks, off);
            float ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool valid = hv && (pc * kChunk + 4 * quad + e < n);
                const float pr = valid ? exp2f(sa[e] * c - lse2) : 0.f;
                // select, never multiply: a padding slot's dP is not used
                ds[e] = valid ? pr * (pa[e] - dlt) : 0.f;
            }
            // B operand dS^T of a 16x16x32 product whose K = 32 runs over the
            // 16 keys twice: slots 0..3 of lane group quad hold the high bf16
            // parts of keys 4*quad .. +3 (the lane's own accumulator values),
            // slots 4..7 their low parts; the A operand repeats K^T's four
            // keys in both halves.
            uint32_t dsh[2], dsl[2];
            split_bf16x2(ds[0], ds[1], dsh[0], dsl[0]);
            split_bf16x2(ds[2], ds[3], dsh[1], dsl[1]);
            const bf16x8 dsv = __builtin_bit_cast(bf16x8, make_uint4(dsh[0], dsh[1], dsl[0], dsl[1]));
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const uint4 k8 = make_uint4(kt[db].x, kt[db].y, kt[db].x, kt[db].y);
                acc[db] = mfma_16x16x32(as_bf16x8(k8), dsv, acc[db]);
            }
        }
        QSA_WAIT_VM(0);  // no gather may outlive the wave's LDS
        if (clk && lane == 0)
            __hip_atomic_fetch_add(clk, (uint32_t)nchunks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!hv) return;
    if (handoff) {
        float *hp = p.dq_part + (row * p.Hq + head) * (int64_t)kD + 4 * quad;
#pragma unroll
        for (int db = 0; db < 16; ++db)
            *reinterpret_cast<float4 *>(hp + 16 * db) =
                make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
        return;
    }
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
constexpr int kHitCap = 384;  // LDS hit list entries per batch
constexpr int kScanWin = 2;   // 64-row windows scanned per step
// One staged row: Q then dO of the group's 12 heads (512 bytes each), then lse
// and delta of heads 0..15 (16 floats each, zero past head 11).
constexpr int kStatOff = 2 * kGroup * 512;
constexpr int kSlot = kStatOff + 2 * 16 * 4;
constexpr int kRingRows = 3;        // staged rows per wave: two fly while one is computed
constexpr int kRowOps = 2 * 6 + 2;  // direct-to-LDS loads per staged row

// Body of k_dkdv. slots: kRingRows staging slots of kSlot bytes; hrow/hmask:
// the wave's hit list.
__device__ __forceinline__ void dkdv_item(const Problem &p, lds_char *slots, int32_t *hrow,
                                          uint32_t *hmask)
{
    const int lane = threadIdx.x;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t ngroups = p.stride >> 4;
    const int64_t per_seg = p.B * p.Hkv * ngroups;
    // item = seg * per_seg + (b * Hkv + g) * ngroups + kg: all key groups of
    // one query segment run side by side and read the same rows. Segments go
    // in ascending order: under a causal route budget the early segments have
    // the fewest candidate keys, so each of their key groups is hit by the
    // most rows, and their long items start first instead of trailing at the
    // end of the launch.
    const int64_t item = blockIdx.x;
    if (item >= p.nseg * per_seg) return;
    const int64_t seg = item / per_seg;
    const int64_t rem = item - seg * per_seg;
    const int64_t kg = rem % ngroups, bg = rem / ngroups;
    const int g = (int)(bg % p.Hkv);
    const int64_t b = bg / p.Hkv;
    const int64_t key0 = kg * 16;
    uint8_t *flag = p.kv_flag + (bg * p.nslot + seg) * ngroups + kg;
    if (key0 >= p.Skv) {
        if (lane == 0) *flag = 0;
        return;
    }

    // This item's query tiles: the entries of the tile column's reverse list
    // of partial tiles that fall in [t_lo, t_hi) (the full tiles are summed by
    // the dense pass).
    const int64_t t = key0 >> 7;
    const int64_t bt = b * p.nKT + t;
    const int32_t *idx_p = p.rev_p_idx + bt * p.nQT;
    // Entries of an ascending list below lo and below hi, counted by the
    // whole wave at once: one memory latency per 256 entries instead of a
    // chain of dependent loads.
    auto count_below = [&](const int32_t *a, int32_t cnt, int32_t lo, int32_t hi, int32_t &c_lo,
                           int32_t &c_hi) {
        int32_t n_lo = 0, n_hi = 0;
        for (int32_t b0 = 0; b0 < cnt; b0 += 256) {
            int32_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t x = b0 + 64 * u + lane;
                v[u] = x < cnt ? a[x] : INT32_MAX;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                n_lo += __popcll(__ballot(v[u] < lo));
                n_hi += __popcll(__ballot(v[u] < hi));
            }
        }
        c_lo = n_lo;
        c_hi = n_hi;
    };
    const int32_t cnt_p = p.rev_p_cnt[bt];
    const int64_t mstride = p.stride >> 5;
    const uint32_t *mrow = p.mbits + (b * p.Sq) * mstride + (key0 >> 5);
    const int shift = (int)(key0 & 16);
    int32_t t_lo = (int32_t)(seg * p.seg_tiles);
    int32_t t_hi = (int32_t)((seg + 1) * p.seg_tiles);
    if (p.merge > 1) {
        const int64_t s0 = seg - seg % p.merge;
        const bool split = p.kv_split[(bg * ((p.nseg + p.merge - 1) / p.merge) + s0 / p.merge) * ngroups + kg] != 0;
        if (!split) {
            if (seg != s0) {
                if (lane == 0) *flag = 0;
                return;
            }
            t_lo = (int32_t)(s0 * p.seg_tiles);
            t_hi = (int32_t)((s0 + p.merge) * p.seg_tiles);
        }
    }
    int32_t p_lo, p_hi;
    count_below(idx_p, cnt_p, t_lo, t_hi, p_lo, p_hi);
    const int64_t nwin = 2 * (int64_t)(p_hi - p_lo);  // 64-row windows
    if (lane == 0) *flag = nwin > 0 ? 1 : 0;
    if (nwin == 0) return;


    // K and V rows of the 16 keys as B operands of S = Q K^T and dP = dO V^T:
    // lane (key col, quad) holds columns 32t + 8quad .. +7 for step t.
    bf16x8 kf[8], vf[8];
    {
        const uint32_t kv_bytes = (uint32_t)((p.Skv - 1) * p.Hkv * kD * 2 + kD * 2);
        const rsrc_t rk = make_rsrc(p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        const rsrc_t rv = make_rsrc(p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD, kv_bytes);
        const int64_t key = key0 + col;
        const uint32_t off =
            key < p.Skv ? (uint32_t)(key * p.Hkv * kD * 2 + quad * 16) : kOutOfRange;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            kf[s] = as_bf16x8(buf_load16(rk, off + 64 * s));
            vf[s] = as_bf16x8(buf_load16(rv, off + 64 * s));
        }
        // Settle these loads here: the staging below is written in assembly,
        // which the compiler cannot count, and the counted waits in the loop
        // are then the only vector memory waits there.
        QSA_WAIT_VM(0);
    }
    f32x4 adk[16], adv[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c = p.scale * 1.4426950408889634f;
    const bool hq = quad < 3;  // accumulator rows 4*quad+e of S are real heads

    // Rows of Q and dO of this batch and group (12 heads x 512 bytes each,
    // contiguous), lse and delta of this batch and group.
    const uint16_t *qbase = p.q + (b * p.Sq * p.Hq + g * kGroup) * (int64_t)kD;
    const uint16_t *gbase = p.dout + (b * p.Sq * p.Hq + g * kGroup) * (int64_t)kD;
    const float *lbase = p.lse_in + (b * p.Hq + g * kGroup) * p.Sq;
    const float *dbase = p.delta + (b * p.Hq + g * kGroup) * p.Sq;
    // Staging of one row into a slot (direct-to-LDS loads written in
    // assembly): instruction x < 6 stages Q heads 2x and 2x+1, instruction 6+x
    // the same dO heads, in the swizzled layout; then lse and delta, lane h < 16
    // staging head h (heads 12..15 read as zero). The row start goes into the
    // descriptors, so the lanes' offsets never change.
    uint32_t lc[6];
#pragma unroll
    for (int x = 0; x < 6; ++x)
        lc[x] = (uint32_t)(x * 1024 + (lane >> 5) * 512 + (dma_chunk(lane, x) << 4));
    const uint32_t sv = lane < kGroup ? (uint32_t)(lane * p.Sq * 4) : kOutOfRange;
    const uint32_t slots_addr = lds_addr(slots);
    auto stage_row = [&](uint32_t qi, int slot) {
        const int64_t ro = (int64_t)qi * p.Hq * kD;
        const i32x4 rq = rsrc_words(qbase + ro, (uint32_t)(kGroup * kD * 2));
        const i32x4 rg = rsrc_words(gbase + ro, (uint32_t)(kGroup * kD * 2));
        const uint32_t dst = slots_addr + (uint32_t)(slot * kSlot);
#pragma unroll
        for (int x = 0; x < 6; ++x) {
            dma16_asm(rq, dst + x * 1024, lc[x]);
            dma16_asm(rg, dst + kGroup * 512 + x * 1024, lc[x]);
        }
        const uint32_t bytes = (uint32_t)((kGroup * p.Sq - qi) * 4);
        const i32x4 rl = rsrc_words(lbase + qi, bytes);
        const i32x4 rd = rsrc_words(dbase + qi, bytes);
        if (lane < 16) {
            dma4_asm(rl, dst + kStatOff, sv);
            dma4_asm(rd, dst + kStatOff + 64, sv);
        }
    };

    // Row-layout read (A operand of S and dP): lane (head col, quad) takes
    // chunk 4t + quad of its head; the padding heads 12..15 read head 11 (their
    // S rows are never selected).
    const int ahead = col < kGroup ? col : kGroup - 1;
    const int amask = swz_mask(ahead);
    // Transposed read (B operand of dV and dK): lane i of group quad names the
    // 8-byte unit of head 4*quad + i/4 holding columns 16db + 4(i%4) .. +3;
    // group 3 (padding heads 12..15) reads heads 8..11 of the same row, which
    // meet exact zeros of P and dS.
    const int th = (quad < 3 ? 4 * quad : 8) + (col >> 2);
    const int tm = swz_mask(th);
    const int tlane = th * 512 + ((((col >> 1) & 1) ^ (tm & 1)) << 4) + (col & 1) * 8;
    const int txor = tm >> 1;

    // dV += P^T dO and dK += dS^T Q for one row. The 32-long contraction
    // covers the row's 16 head slots twice: k slots 0..3 of lane group quad
    // hold the high bf16 parts of P (or dS) for heads 4*quad .. +3 (the lane's
    // own accumulator values of S), slots 4..7 their low parts, and the B
    // operand repeats the transposed dO (or Q) values of the same four heads.
    auto flush = [&](const float *pn, const float *dn, const uint2 *bq, const uint2 *bg_) {
        uint32_t ph[2], pl[2], dh[2], dl[2];
        split_bf16x2(pn[0], pn[1], ph[0], pl[0]);
        split_bf16x2(pn[2], pn[3], ph[1], pl[1]);
        split_bf16x2(dn[0], dn[1], dh[0], dl[0]);
        split_bf16x2(dn[2], dn[3], dh[1], dl[1]);
        const bf16x8 A_p = as_bf16x8(make_uint4(ph[0], ph[1], pl[0], pl[1]));
        const bf16x8 A_d = as_bf16x8(make_uint4(dh[0], dh[1], dl[0], dl[1]));
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const bf16x8 Bg = as_bf16x8(make_uint4(bg_[db].x, bg_[db].y, bg_[db].x, bg_[db].y));
            const bf16x8 Bq = as_bf16x8(make_uint4(bq[db].x, bq[db].y, bq[db].x, bq[db].y));
            adv[db] = mfma_16x16x32(A_p, Bg, adv[db]);
            adk[db] = mfma_16x16x32(A_d, Bq, adk[db]);
        }
    };

    // Hits are visited in DESCENDING query order (tiles from the top of the
    // reverse list of partial tiles, the upper 64 rows of a tile first): all items of a
    // segment sweep its rows at about the same rate, so the rows they read
    // stay in the caches.
    const uint64_t above = (lane == 63) ? 0ull : (~0ull << (lane + 1));
    // The segment's tiles, read once: lane j holds entry p_lo + j (segments of
    // more than 64 tiles read the list in memory).
    const int32_t nt = p_hi - p_lo;
    const int32_t tl = lane < nt ? idx_p[p_lo + lane] : -1;
    auto seg_tile = [&](int32_t j) {
        return nt <= 64 ? __builtin_amdgcn_readlane(tl, j) : idx_p[p_lo + j];
    };
    int64_t w = 0;
    while (w < nwin) {
        int nh = 0;
        while (w < nwin && nh <= kHitCap - kScanWin * 64) {
            uint32_t m[kScanWin];
            int64_t rbase[kScanWin];
#pragma unroll
            for (int x = 0; x < kScanWin; ++x) {
                m[x] = 0u;
                rbase[x] = 0;
                if (w + x < nwin) {
                    const int32_t tile = seg_tile(nt - 1 - (int32_t)((w + x) >> 1));
                    rbase[x] = (int64_t)tile * kTile + (((w + x) & 1) ? 0 : 64);
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
        if (nh == 0) continue;
        wave_lds_sync();
        // Rows of the batch in order; row h is staged in slot h % 3. A row's
        // slot is refilled with row h+3 as soon as all its reads have returned
        // (before its softmax and products), so up to three rows are in flight
        // while one is computed.
        auto hit_row = [&](int h) { return __builtin_amdgcn_readfirstlane((uint32_t)hrow[h]); };
        for (int r0 = 0; r0 < kRingRows && r0 < nh; ++r0) stage_row(hit_row(r0), r0);
        // Row-layout reads of one slot (A operands of S and dP). The address
        // is made opaque after the wait that precedes the call, so none of
        // the reads is moved above that wait.
        uint4 qa[8], ga[8];
        auto read_rows = [&](int sl_idx) {
            const lds_char *sr =
                (const lds_char *)(uintptr_t)opaque_u32(slots_addr + (uint32_t)(sl_idx * kSlot));
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
                const int o = ahead * 512 + (((4 * t8 + quad) ^ amask) << 4);
                qa[t8] = lds_read16(sr + o);
                ga[t8] = lds_read16(sr + kGroup * 512 + o);
            }
        };
        // Row 0 has landed once at most the rows staged after it are in flight.
        if (nh > 2) QSA_WAIT_VM(2 * kRowOps);
        else if (nh > 1) QSA_WAIT_VM(kRowOps);
        else QSA_WAIT_VM(0);
        read_rows(0);
        int slot = 0;
        for (int h = 0; h < nh; ++h) {
            // Row h has landed (waited for before its row-layout reads, which
            // were issued during the previous row's products).
            const lds_char *sl = (const lds_char *)(uintptr_t)opaque_u32(slots_addr + (uint32_t)(slot * kSlot));
            const uint32_t mcur = hmask[h];
            uint2 tq[16], tg[16];
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const int o = tlane + ((db ^ txor) << 5);
                tq[db] = lds_read_tr(sl + o);
                tg[db] = lds_read_tr(sl + kGroup * 512 + o);
            }
            // lse and delta of heads 4*quad .. 4*quad+3
            typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
            const f32x4 ls_c = *reinterpret_cast<const lds_f32x4 *>(sl + kStatOff + quad * 16);
            const f32x4 dl_c = *reinterpret_cast<const lds_f32x4 *>(sl + kStatOff + 64 + quad * 16);

            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
                sa = mfma_16x16x32(as_bf16x8(qa[t8]), kf[t8], sa);
                pd = mfma_16x16x32(as_bf16x8(ga[t8]), vf[t8], pd);
            }
            // Every read of this slot is issued; once they have returned the
            // slot takes row h+3, whose loads then fly during this row's
            // softmax and products as well.
            if (h + kRingRows < nh) {
                const uint32_t qn = hit_row(h + kRingRows);
                QSA_WAIT_LDS();
                stage_row(qn, slot);
            }
            // Lane holds S[head 4*quad+e][key col].
            const bool on = hq && ((mcur >> col) & 1u);
            float pn[4], dn[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pr =
                    on ? __builtin_amdgcn_exp2f(sa[e] * c - ls_c[e] * 1.4426950408889634f) : 0.f;
                pn[e] = pr;
                // select, never multiply: an unselected key's dP may be non-finite
                dn[e] = on ? pr * (pd[e] - dl_c[e]) : 0.f;
            }
            // The next row's row-layout reads fly during this row's dV/dK
            // products. Rows h+1 .. h+3 are the ones in flight here (staged in
            // order); row h+1 has landed once at most the later rows' loads
            // remain.
            if (h + 1 < nh) {
                if (h + 3 < nh) QSA_WAIT_VM(2 * kRowOps);
                else if (h + 2 < nh) QSA_WAIT_VM(kRowOps);
                else QSA_WAIT_VM(0);
                read_rows(slot == kRingRows - 1 ? 0 : slot + 1);
            }
            flush(pn, dn, tq, tg);
            slot = slot == kRingRows - 1 ? 0 : slot + 1;
        }
        QSA_WAIT_VM(0);
        wave_lds_sync();
    }
    // Lane holds dK/dV[key 4*quad+e][d 16*db + col]; the partial sums of this
    // segment go to its slice of the workspace, dK first, then dV.
    float *part = p.kv_part + ((bg * p.nslot + seg) * p.stride + key0) * (int64_t)(2 * kD);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float *pk = part + (4 * quad + e) * (int64_t)(2 * kD) + col;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            pk[16 * db] = adk[db][e];
            pk[kD + 16 * db] = adv[db][e];
        }
    }
}

// Whether each (batch and KV head, segment group, 16-key group) is split into
// its segments: the rows of the group's partial tiles that select one of the
// 16 keys, counted until the count passes kSplitHits. One wave per entry.
__global__ __launch_bounds__(64) void k_dkdv_split(Problem p)
{
    const int lane = threadIdx.x;
    const int64_t ngroups = p.stride >> 4;
    const int64_t nmg = (p.nseg + p.merge - 1) / p.merge;
    const int64_t item = blockIdx.x;
    if (item >= p.B * p.Hkv * nmg * ngroups) return;
    const int64_t kg = item % ngroups;
    const int64_t mg = (item / ngroups) % nmg;
    const int64_t bg = item / (ngroups * nmg);
    const int64_t b = bg / p.Hkv;
    const int64_t key0 = kg * 16;
    uint8_t *out = p.kv_split + item;
    if (key0 >= p.Skv) {
        if (lane == 0) *out = 0;
        return;
    }
    const int64_t bt = b * p.nKT + (key0 >> 7);
    const int32_t *idx_p = p.rev_p_idx + bt * p.nQT;
    const int32_t cnt = p.rev_p_cnt[bt];
    const int32_t g_lo = (int32_t)(mg * p.merge * p.seg_tiles);
    const int32_t g_hi = (int32_t)((mg + 1) * p.merge * p.seg_tiles);
    int32_t e_lo = 0, e_hi = 0;
    for (int32_t b0 = 0; b0 < cnt; b0 += 64) {
        const int32_t x = b0 + lane;
        const int32_t v = x < cnt ? idx_p[x] : INT32_MAX;
        e_lo += __popcll(__ballot(v < g_lo));
        e_hi += __popcll(__ballot(v < g_hi));
    }
    const int64_t mstride = p.stride >> 5;
    const uint32_t *mrow = p.mbits + (b * p.Sq) * mstride + (key0 >> 5);
    const int shift = (int)(key0 & 16);
    int32_t hits = 0;
    for (int32_t e0 = e_lo; e0 < e_hi && hits <= kSplitHits; e0 += 8) {
        uint32_t m[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int32_t e = e0 + (u >> 1);
            m[u] = 0u;
            if (e < e_hi) {
                const int64_t qi = (int64_t)idx_p[e] * kTile + 64 * (u & 1) + lane;
                if (qi < p.Sq) m[u] = (mrow[qi * mstride] >> shift) & 0xffffu;
            }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) hits += __popcll(__ballot(m[u] != 0u));
    }
    if (lane == 0) *out = hits > kSplitHits ? 1 : 0;
}

__global__ __launch_bounds__(64) void k_dkdv(Problem p)
{
    __shared__ __attribute__((aligned(16))) char slots[kRingRows * kSlot];
    __shared__ int32_t hrow[kHitCap];
    __shared__ uint32_t hmask[kHitCap];
    dkdv_item(p, (lds_char *)slots, hrow, hmask);
}

// dK = scale * sum of the partials, dV = sum, in slot order (the segments,
// then the full tiles); one thread per (batch, KV head, key, 4 columns).
__global__ __launch_bounds__(256) void k_dkdv_reduce(Problem p)
{
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_bg = p.stride * (2 * kD / 4);
    if (x >= p.B * p.Hkv * per_bg) return;
    const int64_t bg = x / per_bg;
    const int64_t r = x - bg * per_bg;
    const int64_t key = r / (2 * kD / 4);
    const int f4 = (int)(r - key * (2 * kD / 4));
    const int64_t b = bg / p.Hkv;
    const int g = (int)(bg - b * p.Hkv);
    if (key >= p.Skv) return;
    const int64_t ngroups = p.stride >> 4;
    const uint8_t *flag = p.kv_flag + bg * p.nslot * ngroups + (key >> 4);
    const float *src = p.kv_part + (bg * p.nslot * p.stride + key) * (int64_t)(2 * kD) + 4 * f4;
    const int64_t slot_floats = p.stride * (int64_t)(2 * kD);
    // A wave covers half of one key, so the flags are the same for all its
    // lanes. Eight slots at a time: their flags, then the loads of the
    // flagged ones (all in flight together), then the sums in slot order.
    constexpr int kU = 8;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t s0 = 0; s0 < p.nslot; s0 += kU) {
        bool on[kU];
        float4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            // every flag load in range (the last slot's flag stands in past the
            // end), so the eight loads fly together
            const int64_t su = s0 + u < p.nslot ? s0 + u : p.nslot - 1;
            on[u] = flag[su * ngroups] != 0 && s0 + u < p.nslot;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = on[u] ? *reinterpret_cast<const float4 *>(src + (s0 + u) * slot_floats)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!on[u]) continue;  // skipped, not added as zero: signed zeros stay
            acc.x += v[u].x;
            acc.y += v[u].y;
            acc.z += v[u].z;
            acc.w += v[u].w;
        }
    }
    const bool is_k = f4 < kD / 4;
    const int d = 4 * (is_k ? f4 : f4 - kD / 4);
    const float s = is_k ? p.scale : 1.f;
    uint16_t *dst = (is_k ? p.dk : p.dv) + ((b * p.Skv + key) * p.Hkv + g) * (int64_t)kD + d;
    *reinterpret_cast<uint2 *>(dst) =
        make_uint2(pack_bf16x2(acc.x * s, acc.y * s), pack_bf16x2(acc.z * s, acc.w * s));
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
    if (p.merge > 1) {
        const int64_t entries = p.B * p.Hkv * ((p.nseg + p.merge - 1) / p.merge) * (p.stride >> 4);
        hipLaunchKernelGGL(k_dkdv_split, dim3((unsigned)entries), dim3(64), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t items = p.nseg * p.B * p.Hkv * (p.stride >> 4);
    hipLaunchKernelGGL(k_dkdv, dim3((unsigned)items), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_dkdv_reduce(const Problem &p, hipStream_t s)
{
    const int64_t threads = p.B * p.Hkv * p.stride * (2 * kD / 4);
    hipLaunchKernelGGL(k_dkdv_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
