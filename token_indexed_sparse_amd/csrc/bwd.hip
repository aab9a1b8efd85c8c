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
//    the row's sorted key list in 32-slot steps). S^T and dP^T come from the
//    gathered K and V rows straight into the matrix core; dS^T stays in the
//    accumulator layout and is the B operand of dQ^T = K^T dS^T, with K staged
//    in LDS and read transposed.
//  * k_dkdv: key-major. One wave owns 16 consecutive keys of one KV head and
//    keeps their K and V rows in registers and their dK, dV accumulators for
//    the whole run. It walks the reverse tile lists of its 128-key tile column
//    (partial tiles, then full tiles) and reads the 16-byte membership slice of
//    every query row in those tiles; rows that select at least one of its keys
//    are processed in ascending order, two at a time: S = Q K^T and dP = dO V^T
//    per row (M = heads), then dV += P^T dO and dK += dS^T Q with the two rows'
//    heads forming the 32-long contraction. Q and dO rows are staged in LDS and
//    read transposed.
#include "common.h"

namespace qsa {

namespace {

constexpr int kLdsStride = 264;  // bf16 elements per staged row (528 bytes)

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
constexpr int kDqWaves = 4;
constexpr int kChunk = 32;

__global__ __launch_bounds__(kDqWaves * 64) void k_dq(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint16_t ks_all[kDqWaves][kChunk * kLdsStride];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x * kDqWaves + wave;
    if (item >= p.B * p.Sq * p.Hkv) return;
    const int64_t row = item / p.Hkv;
    const int g = (int)(item - row * p.Hkv);
    const int64_t b = row / p.Sq, i = row - b * p.Sq;
    const int head = g * kGroup + col;
    const bool hv = col < kGroup;
    const int n = p.row_cnt[row];
    uint16_t *ks = ks_all[wave];
    uint16_t *dqp = p.dq + (row * p.Hq + head) * (int64_t)kD;

    f32x4 acc[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n > 0) {
        bf16x8 qf[8], gf[8];
        const int64_t qoff = (row * p.Hq + (hv ? head : 0)) * (int64_t)kD + quad * 64;
        const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + qoff);
        const uint4 *gp = reinterpret_cast<const uint4 *>(p.dout + qoff);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            qf[s] = as_bf16x8(hv ? qp[s] : zero_u4());
            gf[s] = as_bf16x8(hv ? gp[s] : zero_u4());
        }
        const float lse2 = hv ? p.lse_in[(b * p.Hq + head) * p.Sq + i] * 1.4426950408889634f : 0.f;
        const float dlt = hv ? p.delta[(b * p.Hq + head) * p.Sq + i] : 0.f;
        const float c = p.scale * 1.4426950408889634f;
        const int32_t *keys = p.row_keys + row * p.W;
        const int64_t kv_base = b * p.Skv;

        for (int c0 = 0; c0 < n; c0 += kChunk) {
            float ds[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int slot = kb * 16 + col;
                const int key = (c0 + slot < n) ? keys[c0 + slot] : -1;
                const int64_t off =
                    key >= 0 ? ((kv_base + key) * p.Hkv + g) * (int64_t)kD + quad * 64 : 0;
                const uint4 *kp = reinterpret_cast<const uint4 *>(p.k + off);
                const uint4 *vp = reinterpret_cast<const uint4 *>(p.v + off);
                uint4 *kd = reinterpret_cast<uint4 *>(ks + slot * kLdsStride + quad * 64);
                f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const uint4 kv = key >= 0 ? kp[s] : zero_u4();
                    const uint4 vv = key >= 0 ? vp[s] : zero_u4();
                    kd[s] = kv;
                    sa = mfma_16x16x32(as_bf16x8(kv), qf[s], sa);
                    pa = mfma_16x16x32(as_bf16x8(vv), gf[s], pa);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool valid = hv && (c0 + kb * 16 + 4 * quad + e < n);
                    const float pr = valid ? exp2f(sa[e] * c - lse2) : 0.f;
                    ds[kb * 4 + e] = valid ? pr * (pa[e] - dlt) : 0.f;
                }
            }
            uint32_t dsb[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) dsb[x] = pack_bf16x2(ds[2 * x], ds[2 * x + 1]);
            const bf16x8 dsv = as_bf16x8(make_uint4(dsb[0], dsb[1], dsb[2], dsb[3]));
            wave_lds_sync();
#pragma unroll
            for (int db = 0; db < 16; ++db) {
                const uint16_t *kc = ks + 16 * db + col;
                uint32_t a[4];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int s0 = 4 * quad + 2 * x;
                    a[x] = (uint32_t)kc[s0 * kLdsStride] | ((uint32_t)kc[(s0 + 1) * kLdsStride] << 16);
                    a[x + 2] = (uint32_t)kc[(s0 + 16) * kLdsStride] |
                               ((uint32_t)kc[(s0 + 17) * kLdsStride] << 16);
                }
                acc[db] = mfma_16x16x32(as_bf16x8(make_uint4(a[0], a[1], a[2], a[3])), dsv, acc[db]);
            }
            wave_lds_sync();
        }
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

// ---------------------------------------------------------------- dK, dV
constexpr int kKvWaves = 2;
constexpr int kStage = kGroup * kLdsStride;  // one staged 12-head row block

__global__ __launch_bounds__(kKvWaves * 64) void k_dkdv(Problem p)
{
    // Per wave: Q and dO of two query rows, 12 heads each.
    __shared__ __attribute__((aligned(16))) uint16_t st_all[kKvWaves][4 * kStage];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, quad = lane >> 4;
    const int64_t ngroups = p.stride >> 4;
    const int64_t item = (int64_t)blockIdx.x * kKvWaves + wave;  // ((b * Hkv + g) * ngroups + kg)
    if (item >= p.B * p.Hkv * ngroups) return;
    const int64_t kg = item % ngroups;
    const int64_t bg = item / ngroups;
    const int g = (int)(bg % p.Hkv);
    const int64_t b = bg / p.Hkv;
    const int64_t key0 = kg * 16;
    if (key0 >= p.Skv) return;
    const int64_t t = key0 >> 7;
    uint16_t *stq[2] = {st_all[wave], st_all[wave] + kStage};
    uint16_t *stg[2] = {st_all[wave] + 2 * kStage, st_all[wave] + 3 * kStage};

    // K and V rows of the 16 keys as B operands of S = Q K^T and dP = dO V^T.
    bf16x8 kf[8], vf[8];
    {
        const int64_t key = key0 + col;
        const bool kvalid = key < p.Skv;
        const int64_t off = kvalid ? ((b * p.Skv + key) * p.Hkv + g) * (int64_t)kD + quad * 64 : 0;
        const uint4 *kp = reinterpret_cast<const uint4 *>(p.k + off);
        const uint4 *vp = reinterpret_cast<const uint4 *>(p.v + off);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            kf[s] = as_bf16x8(kvalid ? kp[s] : zero_u4());
            vf[s] = as_bf16x8(kvalid ? vp[s] : zero_u4());
        }
    }
    f32x4 adk[16], adv[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        adk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        adv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c = p.scale * 1.4426950408889634f;
    const bool hq = quad < 3;  // accumulator rows 4*quad+e are real heads
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, da[4] = {0.f, 0.f, 0.f, 0.f};
    int filled = 0;

    // Contract the staged pair into dV and dK. Slot j of lane group quad is
    // head 4*quad + (j & 3) of row (j < 4 ? first : second).
    auto flush = [&](const float *pb, const float *db_) {
        uint32_t ap[4], ad[4];
        ap[0] = pack_bf16x2(pa[0], pa[1]);
        ap[1] = pack_bf16x2(pa[2], pa[3]);
        ap[2] = pack_bf16x2(pb[0], pb[1]);
        ap[3] = pack_bf16x2(pb[2], pb[3]);
        ad[0] = pack_bf16x2(da[0], da[1]);
        ad[1] = pack_bf16x2(da[2], da[3]);
        ad[2] = pack_bf16x2(db_[0], db_[1]);
        ad[3] = pack_bf16x2(db_[2], db_[3]);
        const bf16x8 A_p = as_bf16x8(make_uint4(ap[0], ap[1], ap[2], ap[3]));
        const bf16x8 A_d = as_bf16x8(make_uint4(ad[0], ad[1], ad[2], ad[3]));
        wave_lds_sync();
#pragma unroll
        for (int dbk = 0; dbk < 16; ++dbk) {
            uint32_t bg_[4] = {0u, 0u, 0u, 0u}, bq_[4] = {0u, 0u, 0u, 0u};
            if (hq) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = x >> 1;              // 0: first row, 1: second row
                    const int h0 = 4 * quad + 2 * (x & 1);
                    const uint16_t *gq = stg[r] + h0 * kLdsStride + 16 * dbk + col;
                    const uint16_t *qq = stq[r] + h0 * kLdsStride + 16 * dbk + col;
                    bg_[x] = (uint32_t)gq[0] | ((uint32_t)gq[kLdsStride] << 16);
                    bq_[x] = (uint32_t)qq[0] | ((uint32_t)qq[kLdsStride] << 16);
                }
            }
            adv[dbk] = mfma_16x16x32(A_p, as_bf16x8(make_uint4(bg_[0], bg_[1], bg_[2], bg_[3])),
                                     adv[dbk]);
            adk[dbk] = mfma_16x16x32(A_d, as_bf16x8(make_uint4(bq_[0], bq_[1], bq_[2], bq_[3])),
                                     adk[dbk]);
        }
        wave_lds_sync();
    };

    const int64_t bt = b * p.nKT + t;
    for (int lst = 0; lst < 2; ++lst) {
        const int32_t cnt = lst == 0 ? p.rev_p_cnt[bt] : p.rev_f_cnt[bt];
        const int32_t *idx = (lst == 0 ? p.rev_p_idx : p.rev_f_idx) + bt * p.nQT;
        for (int e = 0; e < cnt; ++e) {
            const int64_t r = idx[e];
            for (int sub = 0; sub < 2; ++sub) {
                const int64_t qi_l = r * 128 + sub * 64 + lane;
                uint32_t m16 = 0;
                if (qi_l < p.Sq) {
                    const uint4 mv = *reinterpret_cast<const uint4 *>(
                        p.memb + (b * p.Sq + qi_l) * p.stride + key0);
                    const uint32_t w[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const uint32_t v = w[x] & 0x01010101u;
                        m16 |= ((v | (v >> 7) | (v >> 14) | (v >> 21)) & 0xfu) << (4 * x);
                    }
                }
                uint64_t ball = __ballot(m16 != 0);
                while (ball) {
                    const int src = __builtin_ctzll(ball);
                    ball &= ball - 1;
                    const int64_t qi = r * 128 + sub * 64 + src;
                    const uint32_t mask = __shfl(m16, src);
                    const int64_t qrow = b * p.Sq + qi;
                    // Q and dO rows of this query as A operands (lane: head col, quad).
                    bf16x8 qf[8], gf[8];
                    const bool hv = col < kGroup;
                    const int64_t qoff =
                        (qrow * p.Hq + g * kGroup + (hv ? col : 0)) * (int64_t)kD + quad * 64;
                    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + qoff);
                    const uint4 *gp = reinterpret_cast<const uint4 *>(p.dout + qoff);
                    uint4 *sq = reinterpret_cast<uint4 *>(stq[filled] + col * kLdsStride + quad * 64);
                    uint4 *sg = reinterpret_cast<uint4 *>(stg[filled] + col * kLdsStride + quad * 64);
                    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const uint4 qv = hv ? qp[s] : zero_u4();
                        const uint4 gv = hv ? gp[s] : zero_u4();
                        if (hv) {
                            sq[s] = qv;
                            sg[s] = gv;
                        }
                        qf[s] = as_bf16x8(qv);
                        gf[s] = as_bf16x8(gv);
                    }
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        sa = mfma_16x16x32(qf[s], kf[s], sa);
                        pd = mfma_16x16x32(gf[s], vf[s], pd);
                    }
                    // Lane holds S[head 4*quad+e][key col].
                    const bool kin = (mask >> col) & 1u;
                    float pn[4], dn[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float pr = 0.f, dl = 0.f;
                        if (hq && kin) {
                            const int64_t hix = (b * p.Hq + g * kGroup + 4 * quad + e2) * p.Sq + qi;
                            pr = exp2f(sa[e2] * c - p.lse_in[hix] * 1.4426950408889634f);
                            dl = p.delta[hix];
                        }
                        pn[e2] = pr;
                        // select, never multiply: an unselected key's dP may be non-finite
                        dn[e2] = (hq && kin) ? pr * (pd[e2] - dl) : 0.f;
                    }
                    if (filled == 0) {
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            pa[e2] = pn[e2];
                            da[e2] = dn[e2];
                        }
                        filled = 1;
                    } else {
                        flush(pn, dn);
                        filled = 0;
                    }
                }
            }
        }
    }
    if (filled) {
        // Second row of the last pair is empty: clear its staged rows.
        const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
        if (col < kGroup) {
            uint4 *sq = reinterpret_cast<uint4 *>(stq[1] + col * kLdsStride + quad * 64);
            uint4 *sg = reinterpret_cast<uint4 *>(stg[1] + col * kLdsStride + quad * 64);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                sq[s] = zero_u4();
                sg[s] = zero_u4();
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
    hipLaunchKernelGGL(k_dq, dim3((unsigned)((items + kDqWaves - 1) / kDqWaves)),
                       dim3(kDqWaves * 64), 0, s, p);
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
