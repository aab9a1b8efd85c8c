// Forward of route-set grouped-query attention on gfx950.
//
// Definition: cuDNN Frontend "Query Sparse Attention (QSA)" page, section
// "Selection and components": scaled QK scores over the allowed keys, online
// softmax, PV; FP32 output and natural-log LSE are written, then the output is
// cast to bf16; empty rows give zero output and -inf LSE.
//
// Design (one wave per query row and KV head):
//  * The 12 query heads that share one K/V row are the dense contraction: the
//    wave computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (M = 16 key slots,
//    N = 12 heads padded to 16, K = 256 in eight steps). Each lane feeds the
//    matrix core with 128 contiguous bytes of a gathered key row; the head
//    dimension is visited in an order that makes every lane's slice
//    contiguous (the same order for Q and K, so the dot product is unchanged).
//  * The row's sorted key list is walked in 32-slot chunks. Gathers are
//    branch-free buffer loads (slots past the end read as zero) into two
//    register sets used in turn, so the next chunk's K and V rows are in
//    flight while the current chunk is computed.
//  * The accumulator layout of S^T puts four key slots of one head in a lane,
//    which is exactly the B operand layout of the next product, so P never
//    leaves registers: O^T = V^T P^T (M = 16 head-dim columns, N = heads,
//    K = 32 key slots). V rows are staged in LDS in a layout that
//    ds_read_tr16_b64 reads transposed without bank conflicts.
//  * Each lane owns one head: the running maximum and sum are per lane and the
//    rescale of O is a per-lane scalar.
//  * P is split into bf16 high and low parts (two MFMAs) so that the FP32
//    output keeps about 16 mantissa bits of P; the normaliser is summed from
//    the FP32 P.
//  * Padding slots are zero operands with P = 0 by selection, so no unused
//    K/V value ever enters the arithmetic.
//  * Blocks are mapped XCD-aware: each XCD walks a contiguous range of rows,
//    so the keys that neighbouring rows share stay in that XCD's L2.
#include "common.h"

namespace qsa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kChunk = 32;  // key slots per step (two 16-slot MFMA blocks)

struct Gather {
    uint4 k[2][8];
    uint4 v[2][8];
};

__global__ __launch_bounds__(kFwdWaves * 64) void k_forward(Problem p)
{
    __shared__ __attribute__((aligned(16))) char vs_all[kFwdWaves][2 * kTrBlock];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t nblocks = gridDim.x;
    const int64_t item = xcd_logical_block(blockIdx.x, nblocks) * kFwdWaves + wave;
    if (item >= p.B * p.Sq * p.Hkv) return;
    const int64_t row = item / p.Hkv;
    const int g = (int)(item - row * p.Hkv);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int head = g * kGroup + col;
    const bool hv = col < kGroup;
    const int n = p.row_cnt[row];
    char *vs = vs_all[wave];

    float *of = p.out_fp32 + (row * p.Hq + head) * (int64_t)kD;
    uint16_t *ob = p.out + (row * p.Hq + head) * (int64_t)kD;
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

    // Q as the B operand: lane (head col, quad) holds q[head][quad*64 .. +63].
    bf16x8 qf[8];
    {
        const rsrc_t rq = make_rsrc(p.q + (row * p.Hq + g * kGroup) * (int64_t)kD,
                                    (uint32_t)(kGroup * kD * 2));
        const uint32_t off = hv ? (uint32_t)(col * kD * 2 + quad * 128) : kOutOfRange;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(buf_load16(rq, off + 16 * s));
    }

    // Key indices: branch-free buffer loads; slots at or past n give no key.
    const rsrc_t rkeys = make_rsrc(p.row_keys + row * p.W, (uint32_t)(p.W * 4));
    auto fetch_keys = [&](int c0, int (&kk)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int slot = c0 + kb * 16 + col;
            kk[kb] = (int)__builtin_amdgcn_raw_buffer_load_b32(
                rkeys, slot < n ? (uint32_t)slot * 4 : kOutOfRange, 0, 0);
            kk[kb] = slot < n ? kk[kb] : -1;
        }
    };
    auto offsets = [&](const int (&kk)[2], uint32_t (&off)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            off[kb] = kk[kb] >= 0 ? (uint32_t)kk[kb] * row_bytes + quad * 128 : kOutOfRange;
    };
    auto issue = [&](Gather &G, const uint32_t (&off)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                G.k[kb][s] = buf_load16(rk, off[kb] + 16 * s);
                G.v[kb][s] = buf_load16(rv, off[kb] + 16 * s);
            }
    };

    const float c = p.scale * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tr_lane = lane_tr_base(col, quad);

    auto compute = [&](const Gather &G, int c0) {
        f32x4 st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) a = mfma_16x16x32(as_bf16x8(G.k[kb][s]), qf[s], a);
            st[kb] = a;
        }
        // Stage V rows (slot col of block kb, columns quad*64 + 8s ..) for the
        // transposed read.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 8; ++s) tr_store8(vs + kb * kTrBlock, col, quad * 64 + 8 * s, G.v[kb][s]);
        // Online softmax; lane holds key slots kb*16 + 4*quad + e of head col.
        float t[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool valid = c0 + kb * 16 + 4 * quad + e < n;
                t[kb][e] = valid ? st[kb][e] * c : -INFINITY;
                mx = fmaxf(mx, t[kb][e]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float pr[8];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = exp2f(t[kb][e] - m_new);
                pr[kb * 4 + e] = pv;
                psum += pv;
            }
        l_part = l_part * alpha + psum;
        // B operand P^T: slot j of lane group quad is key 4*quad+j (j<4) or
        // 16+4*quad+j-4 (j>=4): the lane's own accumulator values.
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) split_bf16x2(pr[2 * x], pr[2 * x + 1], hi[x], lo[x]);
        const bf16x8 pb_hi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8 pb_lo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        wave_lds_sync();
        // O^T += V^T P^T; A operand lane (d col, quad) = V[slot(quad, j)][16*db + col].
        // The transposed reads are issued eight tiles at a time ahead of their MFMAs.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint2 a0[8], a1[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                a0[x] = lds_read_tr(vs + tr_lane + tile_tr_offset(8 * h + x));
                a1[x] = lds_read_tr(vs + kTrBlock + tr_lane + tile_tr_offset(8 * h + x));
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int db = 8 * h + x;
                const bf16x8 va = as_bf16x8(make_uint4(a0[x].x, a0[x].y, a1[x].x, a1[x].y));
                f32x4 o = acc[db] * alpha;
                o = mfma_16x16x32(va, pb_hi, o);
                acc[db] = mfma_16x16x32(va, pb_lo, o);
            }
        }
        wave_lds_sync();
    };

    // Pipeline: the gathers of chunk c+1 are issued before chunk c is computed.
    // Key indices are fetched two chunks ahead and always before the gathers
    // of the step, so waiting for them never waits for queued gathers.
    const int nchunks = (n + kChunk - 1) / kChunk;
    Gather G0, G1;
    int kA[2], kB[2];
    uint32_t off[2];
    fetch_keys(0, kA);
    fetch_keys(kChunk, kB);
    offsets(kA, off);
    issue(G0, off);
    auto step = [&](Gather &cur, Gather &nxt, const int (&kn)[2], int (&kfree)[2], int ch) {
        fetch_keys((ch + 2) * kChunk, kfree);
        offsets(kn, off);
        issue(nxt, off);
        __builtin_amdgcn_sched_barrier(0);  // keep the gathers ahead of the compute
        compute(cur, ch * kChunk);
    };
    for (int ch = 0; ch < nchunks; ch += 2) {
        step(G0, G1, kB, kA, ch);
        if (ch + 1 >= nchunks) break;
        step(G1, G0, kA, kB, ch + 1);
    }

    float l = l_part + __shfl_xor(l_part, 16);
    l += __shfl_xor(l, 32);
    if (!hv) return;
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

}  // namespace

hipError_t launch_forward(const Problem &p, hipStream_t s)
{
    const int64_t items = p.B * p.Sq * p.Hkv;
    const int64_t blocks = (items + kFwdWaves - 1) / kFwdWaves;
    hipLaunchKernelGGL(k_forward, dim3((unsigned)blocks), dim3(kFwdWaves * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace qsa
