// Gather-rate probe for the benchmark (declared in qsa_bench.h): measures how
// fast direct-to-LDS buffer loads bring rows named by an index list into LDS,
// the access the gathered kernels make (K/V rows of 512 bytes in the forward
// and dQ, Q/dO rows of 12 x 512 bytes in dK/dV). The rows are staged and never
// read, so the rate is that of the staging alone.
#include "../../include/qsa_bench.h"
#include "common.h"

namespace qsa {
namespace {

// Launch shapes of the probe (waves per work group, LDS bytes per wave); the
// caller times several and takes the best as the staging ceiling.
struct ProbeShape {
    int waves, wave_lds;
};
constexpr ProbeShape kShapes[] = {{4, 32768}, {8, 16384}, {8, 20480}, {4, 16384}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

template <int OPS, int WAVES, int WAVE_LDS>
__device__ void gather_rows(const char *src, uint32_t src_bytes, const int32_t *rows_in, int64_t n,
                            int row_bytes, lds_char *slots)
{
    constexpr int RING = WAVE_LDS / (OPS * 1024) < 32 ? WAVE_LDS / (OPS * 1024) : 32;
    static_assert(RING >= 2, "a ring of at least two item slots");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Row numbers are read as constant data (scalar loads, counted apart from
    // the vector memory loads), so reading them never waits for the staging.
    const __attribute__((address_space(4))) int32_t *rows =
        (const __attribute__((address_space(4))) int32_t *)rows_in;
    const rsrc_t r = make_rsrc(src, src_bytes);
    lds_char *mine = slots + wave * WAVE_LDS;
    const int64_t items = OPS == 1 ? n / 2 : n;
    // Each wave takes a contiguous run of items, four at a time (one scalar
    // load of four or eight row numbers per round).
    const int64_t waves = (int64_t)gridDim.x * WAVES;
    const int64_t per = (items / waves) & ~(int64_t)3;
    const int64_t first = ((int64_t)blockIdx.x * WAVES + wave) * per;
    int64_t issued = 0;
    // The next round's row numbers are loaded while this round's loads issue.
    constexpr int NR = OPS == 1 ? 8 : 4;
    uint32_t rr[NR], nx[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) rr[u] = per > 0 ? (uint32_t)rows[(OPS == 1 ? 2 : 1) * first + u] : 0u;
    for (int64_t i = first; i < first + per; i += 4) {
        const bool more = i + 4 < first + per;
#pragma unroll
        for (int u = 0; u < NR; ++u)
            nx[u] = more ? (uint32_t)rows[(OPS == 1 ? 2 : 1) * (i + 4) + u] : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t base;
            if (OPS == 1)
                base = ((lane >> 5) ? rr[2 * u + 1] : rr[2 * u]) * (uint32_t)row_bytes +
                       (uint32_t)(lane & 31) * 16u;
            else
                base = rr[u] * (uint32_t)row_bytes + (uint32_t)lane * 16u;
            if (issued >= RING - 1) QSA_WAIT_VM((RING - 2) * OPS);
            lds_char *dst = mine + (issued % RING) * (OPS * 1024);
#pragma unroll
            for (int x = 0; x < OPS; ++x) dma16(r, dst + x * 1024, base + x * 1024u);
            ++issued;
        }
#pragma unroll
        for (int u = 0; u < NR; ++u) rr[u] = nx[u];
    }
    QSA_WAIT_VM(0);
}

template <int SHAPE>
__global__ __launch_bounds__(64 * kShapes[SHAPE].waves) void k_gather_probe(
    const char *src, uint32_t src_bytes, const int32_t *rows, int64_t n, int row_bytes)
{
    constexpr int W = kShapes[SHAPE].waves, L = kShapes[SHAPE].wave_lds;
    __shared__ __attribute__((aligned(16))) char slots[W * L];
    lds_char *s = (lds_char *)slots;
    if (row_bytes == 512) gather_rows<1, W, L>(src, src_bytes, rows, n, row_bytes, s);
    else gather_rows<6, W, L>(src, src_bytes, rows, n, row_bytes, s);
}

template <int SHAPE>
hipError_t launch_probe(const char *src, uint32_t src_bytes, const int32_t *rows, int64_t n,
                        int row_bytes, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL(k_gather_probe<SHAPE>, dim3((unsigned)blocks),
                       dim3(64 * kShapes[SHAPE].waves), 0, s, src, src_bytes, rows, n, row_bytes);
    return hipGetLastError();
}

}  // namespace
}  // namespace qsa

extern "C" qsa_status qsa_bench_gather(const void *src, size_t src_bytes, const int32_t *rows,
                                       int64_t n_rows, int32_t row_bytes, int32_t blocks,
                                       int32_t shape, void *stream)
{
    if (!src || !rows) return QSA_ERR_NULL;
    if ((row_bytes != 512 && row_bytes != 6144) || n_rows < 2 || blocks < 1 || shape < 0 ||
        shape >= qsa::kNumShapes || src_bytes >= ((size_t)1 << 31))
        return QSA_ERR_SHAPE;
    const char *sp = static_cast<const char *>(src);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t sb = (uint32_t)src_bytes;
    hipError_t e;
    switch (shape) {
    case 0: e = qsa::launch_probe<0>(sp, sb, rows, n_rows, row_bytes, blocks, s); break;
    case 1: e = qsa::launch_probe<1>(sp, sb, rows, n_rows, row_bytes, blocks, s); break;
    case 2: e = qsa::launch_probe<2>(sp, sb, rows, n_rows, row_bytes, blocks, s); break;
    default: e = qsa::launch_probe<3>(sp, sb, rows, n_rows, row_bytes, blocks, s); break;
    }
    return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH;
}
