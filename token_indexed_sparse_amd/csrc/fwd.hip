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
//    matrix core straight from HBM/L2 with 128 contiguous bytes of a gathered
//    key row; the head dimension is visited in an order that makes every lane's
//    slice contiguous (the same order for Q and K, so the dot product is
//    unchanged).
//  * The accumulator layout of S^T puts four key slots of one head in a lane,
//    which is exactly the B operand layout of the next product, so P never
//    leaves registers: O^T = V^T P^T (M = 16 head-dim rows, N = heads, K = 32
//    key slots). V rows are staged in LDS and read transposed.
//  * The row maximum and sum live per lane (each lane owns one head); the
//    rescale of O is a per-lane scalar.
//  * P is split into bf16 high and low parts (two MFMAs) so that the FP32
//    output keeps ~16 mantissa bits of P; the normaliser is summed from the
//    FP32 P.
//  * Gathered slots past the end of the row's key list are zero operands and
//    get P = 0 by selection, so no unused or padding K/V value ever enters the
//    arithmetic.
#include "common.h"

namespace qsa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kChunk = 32;       // key slots per step (two 16-slot MFMA blocks)
constexpr int kLdsStride = 264;  // bf16 elements per staged row (528 bytes)

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kFwdWaves * 64) void k_forward(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint16_t vs_all[kFwdWaves][kChunk * kLdsStride];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x * kFwdWaves + wave;
    if (item >= p.B * p.Sq * p.Hkv) return;
    const int64_t row = item / p.Hkv;
    const int g = (int)(item - row * p.Hkv);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int head = g * kGroup + col;
    const bool hv = col < kGroup;
    const int n = p.row_cnt[row];
    uint16_t *vs = vs_all[wave];

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

    // Q as the B operand: lane (head col, quad) holds q[head][quad*64 .. +63].
    bf16x8 qf[8];
    {
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            p.q + (row * p.Hq + (hv ? head : 0)) * (int64_t)kD + quad * 64);
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(hv ? qp[s] : zero_u4());
    }

    const float c = p.scale * 1.4426950408889634f;  // scores in log2 units
    float m_run = -INFINITY, l_part = 0.f;
    f32x4 acc[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t *keys = p.row_keys + row * p.W;
    const int64_t kv_base = b * p.Skv;
    for (int c0 = 0; c0 < n; c0 += kChunk) {
        // Gather: lane (slot col, quad) loads 128 bytes of K and of V per block.
        f32x4 st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int slot = kb * 16 + col;
            const int key = (c0 + slot < n) ? keys[c0 + slot] : -1;
            const int64_t off =
                key >= 0 ? ((kv_base + key) * p.Hkv + g) * (int64_t)kD + quad * 64 : 0;
            const uint4 *kp = reinterpret_cast<const uint4 *>(p.k + off);
            const uint4 *vp = reinterpret_cast<const uint4 *>(p.v + off);
            uint4 *vd = reinterpret_cast<uint4 *>(vs + slot * kLdsStride + quad * 64);
            bf16x8 kf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                kf[s] = as_bf16x8(key >= 0 ? kp[s] : zero_u4());
                vd[s] = key >= 0 ? vp[s] : zero_u4();
            }
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) a = mfma_16x16x32(kf[s], qf[s], a);
            st[kb] = a;
        }
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
        for (int x = 0; x < 4; ++x) {
            const uint16_t h0 = f32_to_bf16(pr[2 * x]), h1 = f32_to_bf16(pr[2 * x + 1]);
            hi[x] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[x] = pack_bf16x2(pr[2 * x] - bf16_to_f32(h0), pr[2 * x + 1] - bf16_to_f32(h1));
        }
        const bf16x8 pb_hi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8 pb_lo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
        wave_lds_sync();
        // O^T += V^T P^T; A operand lane (d col, quad) = V[slot(quad, j)][16*db + col].
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const uint16_t *vc = vs + 16 * db + col;
            uint32_t a[4];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int s0 = 4 * quad + 2 * x;
                a[x] = (uint32_t)vc[s0 * kLdsStride] | ((uint32_t)vc[(s0 + 1) * kLdsStride] << 16);
                a[x + 2] = (uint32_t)vc[(s0 + 16) * kLdsStride] |
                           ((uint32_t)vc[(s0 + 17) * kLdsStride] << 16);
            }
            const bf16x8 va = as_bf16x8(make_uint4(a[0], a[1], a[2], a[3]));
            f32x4 o = acc[db] * alpha;
            o = mfma_16x16x32(va, pb_hi, o);
            acc[db] = mfma_16x16x32(va, pb_lo, o);
        }
        wave_lds_sync();
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
