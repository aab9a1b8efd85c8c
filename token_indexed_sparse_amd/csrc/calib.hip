// Gather-rate probe for the benchmark (declared in qsa_bench.h): measures how
// fast direct-to-LDS buffer loads bring rows named by an index list into LDS,
// the access the gathered kernels make (K/V rows of 512 bytes in the forward
// and dQ, Q/dO rows of 12 x 512 bytes in dK/dV). The rows are staged and never
// read, so the rate is that of the staging alone.
#include "../../include/qsa_bench.h"
#include "common.h"

namespace qsa {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeWaveLds = 32768;  // LDS bytes per wave: a ring of item slots

// An item is 1024 bytes per load instruction: with 512-byte rows, two rows
// per instruction (lanes 0..31 the first, 32..63 the second, as the gathered
// forward stages two key rows); with 6144-byte rows, one row in six
// instructions of 1024 contiguous bytes. Every wave takes an equal contiguous
// run of items (a multiple of four; the remainder is not staged); a slot is
// reused once its loads have landed (counted waits with up to RING - 1 items
// in flight: 31 KB per wave with 512-byte rows, 24 KB with 6144-byte rows).
template <int OPS>
__device__ void gather_rows(const char *src, uint32_t src_bytes, const int32_t *rows_in, int64_t n,
                            int row_bytes, lds_char *slots)
{
    constexpr int RING = kProbeWaveLds / (OPS * 1024) < 32 ? kProbeWaveLds / (OPS * 1024) : 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Row numbers are read as constant data (scalar loads, counted apart from
    // the vector memory loads), so reading them never waits for the staging.
    const __attribute__((address_space(4))) int32_t *rows =
        (const __attribute__((address_space(4))) int32_t *)rows_in;
    const rsrc_t r = make_rsrc(src, src_bytes);
    lds_char *mine = slots + wave * kProbeWaveLds;
    const int64_t items = OPS == 1 ? n / 2 : n;
    // Each wave takes a contiguous run of items, four at a time (one scalar
    // load of four or eight row numbers per round).
    const int64_t waves = (int64_t)gridDim.x * kProbeWaves;
    const int64_t per = (items / waves) & ~(int64_t)3;
    const int64_t first = ((int64_t)blockIdx.x * kProbeWaves + wave) * per;
    int64_t issued = 0;
    for (int64_t i = first; i < first + per; i += 4) {
        uint32_t rr[8];
#pragma unroll
        for (int u = 0; u < (OPS == 1 ? 8 : 4); ++u) rr[u] = (uint32_t)rows[(OPS == 1 ? 2 : 1) * i + u];
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
    }
    QSA_WAIT_VM(0);
}

__global__ __launch_bounds__(64 * kProbeWaves) void k_gather_probe(const char *src,
                                                                   uint32_t src_bytes,
                                                                   const int32_t *rows, int64_t n,
                                                                   int row_bytes)
{
    __shared__ __attribute__((aligned(16))) char slots[kProbeWaves * kProbeWaveLds];
    lds_char *s = (lds_char *)slots;
    if (row_bytes == 512) gather_rows<1>(src, src_bytes, rows, n, row_bytes, s);
    else gather_rows<6>(src, src_bytes, rows, n, row_bytes, s);
}

}  // namespace
}  // namespace qsa

extern "C" qsa_status qsa_bench_gather(const void *src, size_t src_bytes, const int32_t *rows,
                                       int64_t n_rows, int32_t row_bytes, int32_t blocks,
                                       void *stream)
{
    if (!src || !rows) return QSA_ERR_NULL;
    if ((row_bytes != 512 && row_bytes != 6144) || n_rows < 2 || blocks < 1 ||
        src_bytes >= ((size_t)1 << 31))
        return QSA_ERR_SHAPE;
    hipLaunchKernelGGL(qsa::k_gather_probe, dim3((unsigned)blocks), dim3(64 * qsa::kProbeWaves), 0,
                       static_cast<hipStream_t>(stream), static_cast<const char *>(src),
                       (uint32_t)src_bytes, rows, n_rows, (int)row_bytes);
    return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH;
}
