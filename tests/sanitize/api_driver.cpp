// Host-only sanitizer driver for the C ABI (built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side, linked with launcher stubs).
// It calls every entry point with invalid arguments, with extreme but valid
// dimensions (workspace arithmetic near the stated limits), and with valid
// arguments on a machine without a GPU, and checks the returned statuses.
// Fake device addresses are never dereferenced: every call here returns
// before any launch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qsa.h"
#include "qsa_bench.h"

static int g_fail = 0;

#define EXPECT(expr, want)                                                               \
    do {                                                                                 \
        const int got_ = (int)(expr);                                                    \
        if (got_ != (int)(want)) {                                                       \
            std::fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, \
                         got_, (int)(want));                                             \
            g_fail = 1;                                                                  \
        }                                                                                \
    } while (0)

static qsa_dims dims(int64_t B, int64_t Sq, int64_t Skv, int64_t Hkv, int64_t W)
{
    qsa_dims d;
    std::memset(&d, 0, sizeof(d));
    d.B = B;
    d.Sq = Sq;
    d.Skv = Skv;
    d.Hq = 12 * Hkv;
    d.Hkv = Hkv;
    d.D = 256;
    d.W = W;
    return d;
}

int main()
{
    void *a = reinterpret_cast<void *>(uintptr_t(4096));
    float *af = static_cast<float *>(a);
    void *odd = reinterpret_cast<void *>(uintptr_t(4098));

    // workspace sizes: valid dims up to the stated limits, and invalid ones
    const qsa_dims sizes[] = {
        dims(1, 1, 1, 1, 1),
        dims(1, 256, 256, 1, 36),
        dims(1, 32768, 32768, 1, 2052),
        dims(1, 1 << 20, 1 << 19, 1, 1),
        dims(64, 1 << 18, 1 << 12, 2, 1 << 20),
        dims(1, 1 << 24, 4096, 1, 4),
        dims(4, 4096, 4096, 2, 260),
    };
    for (const qsa_dims &d : sizes) {
        const size_t f = qsa_forward_workspace_bytes(&d), b = qsa_backward_workspace_bytes(&d);
        const size_t p = qsa_plan_bytes(&d);
        if (f != 0) {
            EXPECT(b > 0 && p > 0, 1);
            EXPECT(p + qsa_backward_planned_workspace_bytes(&d) == b, 1);
            EXPECT(qsa_preprocess_workspace_bytes(&d) > 0, 1);
        }
    }
    qsa_dims big = dims(1, int64_t(1) << 40, int64_t(1) << 40, 1, int64_t(1) << 40);
    EXPECT(qsa_forward_workspace_bytes(&big), 0);
    big = dims(INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX / 16, INT64_MAX);
    EXPECT(qsa_backward_workspace_bytes(&big), 0);
    big = dims(-1, 5, 5, 1, 5);
    EXPECT(qsa_plan_bytes(&big), 0);
    EXPECT(qsa_forward_workspace_bytes(nullptr), 0);

    // forward / backward / preprocess validation
    qsa_dims d = dims(1, 256, 256, 1, 36);
    const size_t wf = qsa_forward_workspace_bytes(&d), wb = qsa_backward_workspace_bytes(&d);
    EXPECT(qsa_forward(nullptr, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_NULL);
    EXPECT(qsa_forward(&d, a, a, a, nullptr, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_NULL);
    EXPECT(qsa_forward(&d, a, a, a, a, NAN, a, af, af, a, wf, nullptr), QSA_ERR_SCALE);
    EXPECT(qsa_forward(&d, a, a, a, a, INFINITY, a, af, af, a, wf, nullptr), QSA_ERR_SCALE);
    EXPECT(qsa_forward(&d, odd, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_ALIGN);
    EXPECT(qsa_forward(&d, a, a, a, odd, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_ALIGN);
    EXPECT(qsa_forward(&d, a, a, a, a, 0.0625f, a, af, af, a, wf - 1, nullptr), QSA_ERR_WORKSPACE);
    EXPECT(qsa_forward(&d, a, a, a, a, 0.0625f, a, af, af, nullptr, wf, nullptr),
           QSA_ERR_WORKSPACE);
    EXPECT(qsa_forward(&d, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_DEVICE);
    EXPECT(qsa_backward(&d, a, a, a, a, af, af, a, 0.0625f, a, a, a, a, wb, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_backward(&d, a, a, a, a, af, af, a, -1.f, a, a, a, a, wb, nullptr), QSA_ERR_SCALE);
    EXPECT(qsa_backward(&d, a, a, a, a, af, af, a, 0.0625f, a, a, nullptr, a, wb, nullptr),
           QSA_ERR_NULL);
    qsa_dims bad = d;
    bad.D = 128;
    EXPECT(qsa_forward(&bad, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_HEADDIM);
    bad = d;
    bad.Hq = 13;
    EXPECT(qsa_backward(&bad, a, a, a, a, af, af, a, 0.0625f, a, a, a, a, wb, nullptr),
           QSA_ERR_HEADS);
    bad = d;
    bad.flags = 8;
    EXPECT(qsa_forward(&bad, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_ROUTE_DTYPE);
    bad = d;
    bad.Skv = (int64_t(1) << 19) + 1;
    EXPECT(qsa_forward(&bad, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr), QSA_ERR_SHAPE);
    int32_t *ai = static_cast<int32_t *>(a);
    uint8_t *a8 = static_cast<uint8_t *>(a);
    const size_t wp = qsa_preprocess_workspace_bytes(&d);
    EXPECT(qsa_preprocess(&d, a, a8, a8, ai, ai, ai, ai, ai, ai, ai, ai, ai, nullptr, nullptr, a,
                          wp, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_preprocess(&d, a, nullptr, a8, ai, ai, ai, ai, ai, ai, ai, ai, ai, nullptr,
                          nullptr, a, wp, nullptr),
           QSA_ERR_NULL);
    EXPECT(qsa_forward_noalloc(&d, a, a, a, a, 0.0625f, a, af, af, nullptr), QSA_ERR_DEVICE);
    qsa_dims huge = dims(1, 32768, 32768, 1, 2052);
    EXPECT(qsa_forward_noalloc(&huge, a, a, a, a, 0.0625f, a, af, af, nullptr), QSA_ERR_SCRATCH);

    // timed variants: too few events
    void *ev[2] = {a, a};
    EXPECT(qsa_forward_timed(&d, a, a, a, a, 0.0625f, a, af, af, a, wf, nullptr, ev, 2),
           QSA_ERR_NULL);

    // plans
    qsa_plan plan;
    std::memset(&plan, 0x5a, sizeof(plan));
    const size_t pb = qsa_plan_bytes(&d);
    EXPECT(qsa_plan_build(&d, a, a, pb, nullptr, nullptr), QSA_ERR_NULL);
    EXPECT(qsa_plan_build(&d, a, a, pb - 1, &plan, nullptr), QSA_ERR_WORKSPACE);
    EXPECT(plan.tag, 0u);
    EXPECT(qsa_plan_build(&d, a, a, pb, &plan, nullptr), QSA_ERR_DEVICE);
    EXPECT(plan.tag, 0u);
    const size_t fp = qsa_forward_planned_workspace_bytes(&d);
    const size_t bp = qsa_backward_planned_workspace_bytes(&d);
    EXPECT(qsa_forward_planned(&plan, a, a, a, 0.0625f, a, af, af, a, fp, nullptr), QSA_ERR_PLAN);
    EXPECT(qsa_forward_planned(nullptr, a, a, a, 0.0625f, a, af, af, a, fp, nullptr),
           QSA_ERR_NULL);
    plan.dims = d;
    plan.mem = a;
    plan.bytes = pb;
    plan.device = 0;
    plan.tag = QSA_PLAN_TAG;
    EXPECT(qsa_forward_planned(&plan, a, a, a, 0.0625f, a, af, af, a, fp, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_backward_planned(&plan, a, a, a, a, af, af, 0.0625f, a, a, a, a, bp, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_backward_planned(&plan, a, a, a, a, af, af, 0.0625f, a, a, a, a, bp - 1, nullptr),
           QSA_ERR_WORKSPACE);
    uint32_t *au = static_cast<uint32_t *>(a);
    EXPECT(qsa_plan_tables(&plan, au, ai, ai, ai, ai, ai, ai, ai, ai, ai, ai, ai, nullptr),
           QSA_ERR_DEVICE);
    plan.bytes = pb - 1;
    EXPECT(qsa_forward_planned(&plan, a, a, a, 0.0625f, a, af, af, a, fp, nullptr), QSA_ERR_PLAN);
    plan.bytes = pb;
    plan.dims.W = int64_t(1) << 40;
    EXPECT(qsa_forward_planned(&plan, a, a, a, 0.0625f, a, af, af, a, fp, nullptr), QSA_ERR_SHAPE);

    // block-bitmap entries
    qsa_block_dims bd;
    std::memset(&bd, 0, sizeof(bd));
    bd.T = 300;
    bd.NB = 80;
    bd.Hq = 12;
    bd.Hkv = 1;
    bd.D = 256;
    bd.block_size = 4;
    const size_t bf = qsa_block_forward_workspace_bytes(&bd);
    const size_t bb = qsa_block_backward_workspace_bytes(&bd);
    EXPECT(bf > 0 && bb > bf, 1);
    EXPECT(qsa_block_forward(&bd, a, a, a, a8, ai, ai, ai, ai, ai, ai, 0.0625f, a, af, af, a, bf,
                             nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_block_backward(&bd, a, a, a, a, af, af, a8, ai, ai, ai, ai, ai, ai, 0.0625f, a, a,
                              a, a, bb, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_block_forward(&bd, a, a, a, a8, ai, nullptr, ai, ai, ai, ai, 0.0625f, a, af, af, a,
                             bf, nullptr),
           QSA_ERR_NULL);
    EXPECT(qsa_block_plan_build(&bd, a8, ai, ai, ai, ai, ai, ai, a, bf, &plan, nullptr),
           QSA_ERR_DEVICE);
    qsa_block_dims bbad = bd;
    bbad.block_size = 8;
    EXPECT(qsa_block_plan_bytes(&bbad), 0);
    bbad = bd;
    bbad.NB = INT64_MAX;
    EXPECT(qsa_block_forward_workspace_bytes(&bbad), 0);
    bbad = bd;
    bbad.T = INT64_MAX;
    EXPECT(qsa_block_backward_workspace_bytes(&bbad), 0);
    bbad.T = int64_t(1) << 18;  // one batch row of Q stays below 2^31 bytes
    bbad.NB = int64_t(1) << 16;
    EXPECT(qsa_block_plan_bytes(&bbad) > 0, 1);
    bbad.T = int64_t(1) << 19;  // 2^19 * 12 heads * 512 bytes: beyond 32-bit offsets
    EXPECT(qsa_block_plan_bytes(&bbad), 0);

    // status strings, in and out of range
    // block selector
    qsa_select_dims sd;
    std::memset(&sd, 0, sizeof(sd));
    sd.B = 2;
    sd.Sq = 300;
    sd.NB = 80;
    sd.H = 64;
    sd.D = 128;
    sd.top_k = 16;
    const size_t sw = qsa_select_workspace_bytes(&sd);
    EXPECT(sw == size_t(2) * 300 * 80 * 4, 1);
    EXPECT(qsa_select(&sd, a, a, nullptr, nullptr, 0.5f, ai, ai, nullptr, a, sw, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_select(&sd, a, a, ai, ai, 0.5f, nullptr, nullptr, af, nullptr, 0, nullptr),
           QSA_ERR_DEVICE);
    EXPECT(qsa_select(&sd, a, a, nullptr, nullptr, 0.5f, ai, ai, nullptr, a, sw - 1, nullptr),
           QSA_ERR_WORKSPACE);
    EXPECT(qsa_select(&sd, a, a, nullptr, nullptr, NAN, ai, ai, nullptr, a, sw, nullptr),
           QSA_ERR_SCALE);
    EXPECT(qsa_select(&sd, a, a, nullptr, nullptr, 0.5f, nullptr, nullptr, nullptr, a, sw, nullptr),
           QSA_ERR_NULL);
    EXPECT(qsa_select(nullptr, a, a, nullptr, nullptr, 0.5f, ai, ai, nullptr, a, sw, nullptr),
           QSA_ERR_NULL);
    // extreme but valid: B * Sq just below 2^31, the largest NB; the workspace
    // size is then 2^31 * 32768 * 4 bytes, no overflow
    sd.B = 1;
    sd.Sq = INT32_MAX;
    sd.NB = 32768;
    sd.top_k = 4096;
    EXPECT(qsa_select_workspace_bytes(&sd) == size_t(INT32_MAX) * 32768 * 4, 1);
    sd.q_offset = 1;  // q_offset + Sq beyond 2^31 - 1
    EXPECT(qsa_select_workspace_bytes(&sd), 0);
    sd.q_offset = 0;
    sd.Sq = INT64_MAX;
    EXPECT(qsa_select_workspace_bytes(&sd), 0);
    EXPECT(qsa_select(&sd, a, a, nullptr, nullptr, 0.5f, ai, ai, nullptr, a, sw, nullptr),
           QSA_ERR_SHAPE);

    for (int s = -3; s < 20; ++s) EXPECT(qsa_status_string(static_cast<qsa_status>(s)) != nullptr, 1);
    EXPECT(qsa_version() >> 16, 1);

    if (g_fail) return 1;
    std::printf("api driver ok\n");
    return 0;
}
