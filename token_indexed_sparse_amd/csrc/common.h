// Internal definitions shared by the gfx950 kernels and the host API of the
// QSA library. Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

constexpr int kD = 256;     // head dimension (QSA page, "Support and execution")
constexpr int kGroup = 12;  // query heads per KV head
constexpr int kTile = 128;  // query and key tile edge of the membership table
constexpr int kMaxSkvLog2 = 19;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Everything the kernels need, with the workspace already carved.
struct Problem {
    int64_t B, Sq, Skv, Hq, Hkv, W;
    int32_t route_is_i64;
    int64_t stride;  // membership row stride = nKT * 128
    int64_t nQT, nKT;
    float scale;
    // inputs
    const void *routes;
    const uint16_t *q, *k, *v, *dout;
    const float *out_fp32_in, *lse_in;
    // preprocessing results (workspace or caller buffers)
    uint8_t *memb, *has_routes;
    int32_t *row_keys, *row_cnt;
    int32_t *tile_cnt, *kinds;
    int32_t *fwd_p_cnt, *fwd_p_idx, *fwd_f_cnt, *fwd_f_idx;
    int32_t *rev_p_cnt, *rev_p_idx, *rev_f_cnt, *rev_f_idx;
    // forward outputs
    uint16_t *out;
    float *out_fp32, *lse;
    // backward
    float *delta;
    uint16_t *dq, *dk, *dv;
};

hipError_t launch_preprocess(const Problem &p, hipStream_t s);
hipError_t launch_forward(const Problem &p, hipStream_t s);
hipError_t launch_delta(const Problem &p, hipStream_t s);
hipError_t launch_dq(const Problem &p, hipStream_t s);
hipError_t launch_dkdv(const Problem &p, hipStream_t s);

#if defined(__HIPCC__)
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }
#endif

}  // namespace qsa
