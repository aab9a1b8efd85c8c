// Forward of route-set grouped-query attention on gfx950.
//
// Definition: cuDNN Frontend "Query Sparse Attention (QSA)" page, section
// "Selection and components": scaled QK scores over the allowed keys, online
// softmax, PV; FP32 output and natural-log LSE are written, then the output is
// cast to bf16; empty rows give zero output and -inf LSE.
//
// Design (one wave per query row and KV head, one wave per workgroup):
//  * The 12 query heads that share one K/V row are the dense contraction: the
//    wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (M = 16 key slots,
//    N = 12 heads padded to 16, K = 256 in eight steps).
//  * The row's sorted key list is walked in 16-slot chunks. A chunk's K and V
//    rows are gathered straight into LDS with direct-to-LDS buffer loads, two
//    512-byte rows per instruction, so the vector memory path sees whole
//    contiguous rows instead of one row per lane. Slots past the end of the
//    list read as zero without a branch. Once a chunk's K rows have been read
//    out of LDS into registers, the next chunk's K gathers are issued into the
//    same region and fly while the scores and softmax run; the V region is
//    read and refilled the same way just before the PV products (refilling
//    both regions together, after both reads, was 4 % slower).
//    16-slot chunks keep the wave under 256 registers and 16 KB of LDS, so
//    two waves share each SIMD and one's gathers hide behind the other's
//    products (32-slot chunks at one wave per SIMD were 9 % slower).
//  * K is read back in the MFMA operand layout with 16-byte reads, V with the
//    transposing ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T; a
//    per-row swizzle of the 16-byte chunks keeps both reads free of bank
//    conflicts.
//  * The accumulator layout of S^T puts four key slots of one head in a lane,
//    which is the B operand layout of O^T = V^T P^T over 16 key slots, so P
//    never leaves registers. Each lane owns one head: the running maximum and
//    sum are per lane and the rescale of O is a per-lane scalar.
//  * The first chunk fixes each head's reference maximum. P = exp2(s - ref)
//    may then grow up to 2^64, which FP32 and the bf16 split carry exactly as
//    well; a chunk further above the reference raises it and has the row
//    recomputed from its first chunk (the result is the same, only the work
//    repeats). O is therefore never rescaled inside the loop, and its
//    accumulators stay in the matrix-core registers.
//  * P is split into bf16 high and low parts so that the FP32 output keeps
//    about 16 mantissa bits of P; the normaliser is summed from the FP32 P.
//    Both parts go through one v_mfma_f32_16x16x32_bf16 whose K = 32 covers
//    the 16 key slots twice (high parts, then low parts, against the same V
//    values repeated): on gfx950 the 16x16x16 form takes as many cycles as
//    the 16x16x32 one, so two 16x16x16 products would cost twice as much.
//  * Padding slots are zero operands with P = 0 by selection, so no unused
//    K/V value ever enters the arithmetic.
//  * Rows go to blocks in plain order, so the XCDs (which take blocks in
//    turn) run neighbouring rows side by side; with the rotated walks their
//    similar key lists are then read at the same time. Giving each XCD a
//    contiguous range of rows instead was 5 % slower.
#include "common.h"

namespace qsa {

namespace {

constexpr int kChunk = 16;            // key slots per step (one 16-slot MFMA block)
constexpr float kSlack = 64.f;        // log2 of the largest unnormalised P

// Body of k_forward; ks and vs are the wave's K and V staging regions.
__device__ __forceinline__ void forward_row(const Problem &p, lds_char *ks, lds_char *vs)
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
    // dense pass adds them and writes the outputs, and this pass hands over
    // its unnormalised state instead.
    const int n = p.pcnt[row];
    const bool handoff = p.fwd_f_cnt[b * p.nQT + (i >> 7)] > 0;
    const int64_t sidx = (b * p.Hq + head) * p.Sq + i;

    float *of = p.out_fp32 + (row * p.Hq + head) * (int64_t)kD;
    uint16_t *ob = p.out + (row * p.Hq + head) * (int64_t)kD;
    if (n == 0 && handoff) {
        if (hv) {
            for (int db = 0; db < 16; ++db)
                *reinterpret_cast<float4 *>(of + 16 * db + 4 * quad) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (quad == 0) *reinterpret_cast<float2 *>(p.fstate + 2 * sidx) = make_float2(-INFINITY, 0.f);
        }
        return;
    }
    if (n == 0) {
        if (hv) {
            for (int db = 0; db < 16; ++db) {
                const int d = 16 * db + 4 * quad;
                *reinterpret_cast<float4 *>(of + d) = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<uint2 *>(ob + d) = make_uint2(0u, 0u);
            }
            if (quad == 0) p.lse[(b * p.Hq + head) * p.Sq + i] = -INFINITY;
        }
        return;
    }

    // K/V rows of this batch and KV head: row `key` starts at byte key*Hkv*512.
    const uint32_t row_bytes = (uint32_t)(p.Hkv * kD * 2);
    const uint16_t *kbase = p.k + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    const uint16_t *vbase = p.v + (b * p.Skv * p.Hkv + g) * (int64_t)kD;
    const uint32_t kv_bytes = (uint32_t)((p.Skv - 1) * p.Hkv * kD * 2 + kD * 2);
    const rsrc_t rk = make_rsrc(kbase, kv_bytes), rv = make_rsrc(vbase, kv_bytes);

    // Q as the B operand: lane (head col, quad) holds q[head][32t + 8quad ..
    // +7] for step t.
    bf16x8 qf[8];
    {
        const rsrc_t rq = make_rsrc(p.q + (row * p.Hq + g * kGroup) * (int64_t)kD,
                                    (uint32_t)(kGroup * kD * 2));
        const uint32_t off = hv ? (uint32_t)(col * kD * 2 + quad * 16) : kOutOfRange;
#pragma unroll
        for (int t = 0; t < 8; ++t) qf[t] = as_bf16x8(buf_load16(rq, off + 64 * t));
        // Settle these loads here, so that the counted waits in the loop
        // below are the only vector memory waits there.
        QSA_WAIT_VM(0);
    }

    // Gather instruction s (0..7) stages key slot s (lanes 0..31) and slot
    // s + 8 (lanes 32..63), each lane one 16-byte chunk of the row. A lane's 8
    // keys per chunk (slots 8h .. 8h+7 for its half h) are fetched one chunk
    // ahead with two 16-byte loads; slots at or past n read as zero.
    const int half = lane >> 5;
    const rsrc_t rkeys = make_rsrc(p.pkeys + row * p.W, (uint32_t)(p.W * 4));
    auto fetch_keys = [&](int ch, uint4 (&kk)[2]) {
        const int base = ch * kChunk + 8 * half;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            kk[q] = buf_load16(rkeys, base + 4 * q < n ? (uint32_t)(base + 4 * q) * 4 : kOutOfRange);
    };
    // Row slot j sits at rowbase(j) = (j & 7) * 1024 + (j >> 3) * 512 with its
    // chunks swizzled by swz_mask(j); lane l of instruction s holds chunk
    // (l & 31) ^ swz_mask(s + 8h) of slot s + 8h.
    const uint32_t lane16 = (uint32_t)((lane & 31) << 4);
    auto offsets = [&](const uint4 (&kk)[2], int ch, uint32_t (&off)[8]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t k4[4] = {kk[q].x, kk[q].y, kk[q].z, kk[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s2 = 4 * q + e;
                const uint32_t m = (uint32_t)swz_mask(s2 + 8 * half) << 4;
                // key < 2^19 and row_bytes < 2^21: the 24-bit multiply-add is exact
                off[s2] = __umul24(k4[e], row_bytes) + (lane16 ^ m);
            }
        }
        if ((ch + 1) * kChunk > n) {  // the last chunk: slots past n read zeros
            const int rem = n - ch * kChunk - 8 * half;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) off[s2] = s2 < rem ? off[s2] : kOutOfRange;
        }
    };
    auto gather = [&](rsrc_t r, lds_char *dst, const uint32_t (&off)[8]) {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) dma16(r, dst + s2 * 1024, off[s2]);
    };

    const float c = p.scale * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K read: lane (key slot col, quad) takes chunk 4t + quad of slot kb*16 +
    // col. V transposed read: lane i of group quad names the 8-byte unit of
    // slot kb*16 + 4*quad + i/4 holding columns 16db + 4(i%4) .. +3, which is
    // half (i & 1) of chunk 2db + ((i >> 1) & 1); with the swizzle that
    // chunk's slot is 2 (db ^ (m >> 1)) + (((i >> 1) & 1) ^ (m & 1)) for the
    // row's mask m. Slot kb*16 + j lies 512 kb above slot j.
    const int kmask = swz_mask(col);
    const int kbase_lane = (col & 7) * 1024 + (col >> 3) * 512;
    const int vkey = 4 * quad + (col >> 2);
    const int vm = swz_mask(vkey);
    const int vbase_lane = (vkey & 7) * 1024 + (vkey >> 3) * 512 +
                           ((((col >> 1) & 1) ^ (vm & 1)) << 4) + (col & 1) * 8;
    const int vxor = vm >> 1;

    const int nchunks = (n + kChunk - 1) / kChunk;
    // Walk rotation. Rows start whenever a slot frees up, so without it the
    // rows in flight sit at scattered points of their (similar) ascending key
    // lists and share little of the caches. A row starts instead at the chunk
    // that the wave slots have reached on average (the chunks of all finished
    // rows over the resident slots, modulo the row's chunk count) and wraps
    // around, so the rows in flight walk the same part of their lists. Any
    // walk order gives the same result up to FP32 rounding order.
    uint32_t *const clk = p.walk;
    int rot = 0;
    if (clk && nchunks > 1) {
        const uint32_t done = __hip_atomic_fetch_add(clk, opaque_u32(0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rot = (int)__builtin_amdgcn_readfirstlane((done / p.walk_slots) % (uint32_t)nchunks);
    }
    // Chunk x of the walk; positions past the list stay past it.
    auto phys = [&](int x) {
        return x >= nchunks ? x : (x + rot >= nchunks ? x + rot - nchunks : x + rot);
    };
    bool restart = false;
    for (;;) {
        uint4 kn[2];
        uint32_t off[8];
        fetch_keys(phys(0), kn);
        offsets(kn, phys(0), off);
        fetch_keys(phys(1), kn);
        gather(rk, ks, off);
        gather(rv, vs, off);

        for (int ch = 0; ch < nchunks; ++ch) {
            QSA_WAIT_VM(0);
            offsets(kn, phys(ch + 1), off);  // next chunk
            fetch_keys(phys(ch + 2), kn);
            const int pc = phys(ch);  // the chunk's place in the list
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            {
                uint4 kr[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    kr[t] = lds_read16(ks + kbase_lane + (((4 * t + quad) ^ kmask) << 4));
                QSA_WAIT_LDS();  // the K region is free
                gather(rk, ks, off);
#pragma unroll
                for (int t = 0; t < 8; ++t) hold_after(kr[t]);
#pragma unroll
                for (int t = 0; t < 8; ++t) st = mfma_16x16x32(as_bf16x8(kr[t]), qf[t], st);
            }

            // Softmax numerators; lane holds key slots 4*quad + e of head col.
            float t4[4];
            float mx = -INFINITY;
            if ((pc + 1) * kChunk <= n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t4[e] = st[e] * c;
                    mx = fmaxf(mx, t4[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool valid = pc * kChunk + 4 * quad + e < n;
                    t4[e] = valid ? st[e] * c : -INFINITY;
                    mx = fmaxf(mx, t4[e]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (ch == 0) {
                m_run = fmaxf(m_run, mx);
            } else if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
                m_run = fmaxf(m_run, mx);
                restart = true;
                break;
            }
            float pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[e] = __builtin_amdgcn_exp2f(t4[e] - m_run);
                l_part += pr[e];
            }
            // B operand P^T of a 16x16x32 product whose K = 32 runs over the
            // 16 keys twice: slots 0..3 of lane group quad hold the high bf16
            // parts of keys 4*quad .. +3 (the lane's own accumulator values),
            // slots 4..7 their low parts. The A operand repeats V^T's four
            // keys in both halves, so one MFMA adds V^T (P_hi + P_lo)^T.
            uint32_t hi[2], lo[2];
            split_bf16x2(pr[0], pr[1], hi[0], lo[0]);
            split_bf16x2(pr[2], pr[3], hi[1], lo[1]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], lo[0], lo[1]));
            uint2 va[16];
            {
                const lds_char *vsr = (const lds_char *)(uintptr_t)opaque_u32(lds_addr(vs));
#pragma unroll
                for (int db = 0; db < 16; ++db)
                    va[db] = lds_read_tr(vsr + vbase_lane + ((db ^ vxor) << 5));
            }
            QSA_WAIT_LDS();  // the V region is free
            gather(rv, vs, off);
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const uint4 v8 = make_uint4(va[db].x, va[db].y, va[db].x, va[db].y);
                acc[db] = mfma_16x16x32(as_bf16x8(v8), pb, acc[db]);
            }
        }
        QSA_WAIT_VM(0);  // no gather may outlive this pass or the wave's LDS
        if (!restart) break;
        restart = false;
#pragma unroll
        for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        l_part = 0.f;
    }
    if (clk && lane == 0)
        __hip_atomic_fetch_add(clk, (uint32_t)nchunks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    float l = l_part + __shfl_xor(l_part, 16);
    l += __shfl_xor(l, 32);
    if (!hv) return;
    if (handoff) {
#pragma unroll
        for (int db = 0; db < 16; ++db)
            *reinterpret_cast<float4 *>(of + 16 * db + 4 * quad) =
                make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
        if (quad == 0) *reinterpret_cast<float2 *>(p.fstate + 2 * sidx) = make_float2(m_run, l);
        return;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        const int d = 16 * db + 4 * quad;
        const float o0 = acc[db][0] * inv, o1 = acc[db][1] * inv, o2 = acc[db][2] * inv,
                    o3 = acc[db][3] * inv;
        *reinterpret_cast<float4 *>(of + d) = make_float4(o0, o1, o2, o3);
        *reinterpret_cast<uint2 *>(ob + d) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
    if (quad == 0)
        p.lse[(b * p.Hq + head) * p.Sq + i] = (m_run + log2f(l)) * 0.6931471805599453f;
}

__global__ __launch_bounds__(64) void k_forward(Problem p)
{
    __shared__ __attribute__((aligned(16))) char ks[kChunk * 512];
    __shared__ __attribute__((aligned(16))) char vs[kChunk * 512];
    forward_row(p, (lds_char *)ks, (lds_char *)vs);
}

}  // namespace

hipError_t launch_forward(const Problem &p, hipStream_t s)
{
    const int64_t items = p.B * p.Sq * p.Hkv;
    hipLaunchKernelGGL(k_forward, dim3((unsigned)items), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
