// Host side of the QSA C ABI: validation before any launch, workspace sizing
// and carving, and the launch sequence of each call. See include/qsa.h for the
// contract of every entry point.
#include "../../include/qsa_bench.h"

#include <cmath>
#include <cstring>
#include <mutex>

#include "common.h"

namespace {

using namespace qsa;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Query tiles per dK/dV segment: short segments keep the rows that the
// concurrent work items stage close together (more L2 hits), at the cost of
// more partial sums, which are bounded by kPartialBudget.
int64_t seg_tiles_for(const qsa_dims *d)
{
    const int64_t nQT = (d->Sq + kTile - 1) / kTile;
    const int64_t stride = (d->Skv + kTile - 1) / kTile * kTile;
    int64_t seg = kSegTilesMin;
    for (;;) {
        const int64_t nseg = (nQT + seg - 1) / seg;
        const int64_t bytes = d->B * d->Hkv * (nseg + 1) * stride * 2 * kD * 4;
        if (bytes <= kPartialBudget || seg >= nQT) return seg;
        seg *= 2;
    }
}

qsa_status check_dims(const qsa_dims *d)
{
    if (!d) return QSA_ERR_NULL;
    if ((d->route_is_i64 != 0 && d->route_is_i64 != 1) || (d->flags & ~QSA_FLAG_DETERMINISTIC) != 0)
        return QSA_ERR_ROUTE_DTYPE;
    if (d->B < 1 || d->Sq < 1 || d->Skv < 1 || d->W < 1) return QSA_ERR_SHAPE;
    if (d->D != kD) return QSA_ERR_HEADDIM;
    if (d->Hkv < 1 || d->Hkv > 4096 || d->Hq != (int64_t)kGroup * d->Hkv) return QSA_ERR_HEADS;
    if (d->Skv > (int64_t(1) << kMaxSkvLog2) || d->W > (int64_t(1) << 20)) return QSA_ERR_SHAPE;
    // Grid limits: every launch stays below 2^32 work-items.
    if (d->B > (int64_t(1) << 24) || d->Sq > (int64_t(1) << 24)) return QSA_ERR_SHAPE;
    if (d->B * d->Sq > (int64_t(1) << 24) || d->B * d->Sq * d->Hq > (int64_t(1) << 26))
        return QSA_ERR_SHAPE;
    const int64_t stride = (d->Skv + kTile - 1) / kTile * kTile;
    if (d->B * d->Hkv * stride > (int64_t(1) << 30)) return QSA_ERR_SHAPE;
    // dK/dV work items: one per query segment and 16-key group.
    const int64_t seg = seg_tiles_for(d);
    const int64_t nseg = ((d->Sq + kTile - 1) / kTile + seg - 1) / seg;
    if (nseg * d->B * d->Hkv * (stride / 16) >= (int64_t(1) << 31)) return QSA_ERR_SHAPE;
    // Gathers use 32-bit buffer offsets within one batch row of K/V or Q/dO.
    if (d->Skv * d->Hkv * kD * 2 >= (int64_t(1) << 31)) return QSA_ERR_SHAPE;
    if (d->Sq * d->Hq * kD * 2 >= (int64_t(1) << 31)) return QSA_ERR_SHAPE;
    if (d->W * 4 >= (int64_t(1) << 31)) return QSA_ERR_SHAPE;
    return QSA_OK;
}

struct Layout {
    size_t memb, has, mbits, row_keys, row_cnt, pkeys, pcnt, tile_cnt, kinds, fpc, fpi, ffc, ffi,
        rpc, rpi, rfc, rfi, fstate, delta, kv_part, kv_flag, walk, total;
};

// which: 0 forward, 1 backward, 2 preprocess (only tile counts and, if the
// caller does not want them, the row key lists).
Layout layout(const qsa_dims *d, int which)
{
    const int64_t nQT = (d->Sq + kTile - 1) / kTile, nKT = (d->Skv + kTile - 1) / kTile;
    const int64_t stride = nKT * kTile;
    const int64_t rows = d->B * d->Sq;
    Layout L;
    std::memset(&L, 0, sizeof(L));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    const size_t none = (size_t)-1;
    // The byte membership table and has_routes are outputs of qsa_preprocess
    // only (caller buffers): no forward or backward kernel reads them, so those
    // calls do not materialise them.
    L.memb = none;
    L.has = none;
    L.mbits = which == 1 ? take((size_t)(rows * (stride / 32)) * 4) : none;
    L.row_keys = take((size_t)(rows * d->W) * 4);
    L.row_cnt = take((size_t)rows * 4);
    L.pkeys = which == 2 ? none : take((size_t)(rows * d->W) * 4);
    L.pcnt = which == 2 ? none : take((size_t)rows * 4);
    L.tile_cnt = take((size_t)(d->B * nQT * nKT) * 4);
    if (which == 2) {
        L.kinds = L.fpc = L.fpi = L.ffc = L.ffi = L.rpc = L.rpi = L.rfc = L.rfi = none;
    } else {
        L.kinds = take((size_t)(d->B * nQT * nKT) * 4);
        L.fpc = take((size_t)(d->B * nQT) * 4);
        L.fpi = take((size_t)(d->B * nQT * nKT) * 4);
        L.ffc = take((size_t)(d->B * nQT) * 4);
        L.ffi = take((size_t)(d->B * nQT * nKT) * 4);
        L.rpc = take((size_t)(d->B * nKT) * 4);
        L.rpi = take((size_t)(d->B * nKT * nQT) * 4);
        L.rfc = take((size_t)(d->B * nKT) * 4);
        L.rfi = take((size_t)(d->B * nKT * nQT) * 4);
    }
    L.fstate = which == 0 ? take((size_t)(d->B * d->Hq * d->Sq) * 8) : none;
    L.delta = which == 1 ? take((size_t)(d->B * d->Hq * d->Sq) * 4) : none;
    const int64_t seg = seg_tiles_for(d);
    const int64_t nseg = (nQT + seg - 1) / seg;
    // The dK/dV partial sums and the dQ hand-over are never live together
    // (dQ finishes before dK/dV starts), so they share one region.
    const size_t kv_bytes = (size_t)(d->B * d->Hkv * (nseg + 1) * stride) * 2 * kD * 4;
    const size_t dq_bytes = (size_t)(rows * d->Hq) * kD * 4;
    L.kv_part = which == 1 ? take(kv_bytes > dq_bytes ? kv_bytes : dq_bytes) : none;
    L.kv_flag = which == 1 ? take((size_t)(d->B * d->Hkv * (nseg + 1) * (stride / 16))) : none;
    L.walk = which == 2 ? none : take(16 * 4);
    L.total = off;
    return L;
}

// Properties of each device the library has run on, read once per device
// (std::call_once, so concurrent first calls on one device do not race) and
// never changed afterwards.
constexpr int kMaxDevices = 64;
struct DeviceInfo {
    bool ok = false;
    size_t max_lds = 0;
    uint32_t cus = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

const DeviceInfo *device_info(int &dev)
{
    dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        DeviceInfo &info = g_dev[dev];
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        info.max_lds = prop.sharedMemPerBlock;
        info.cus = (uint32_t)prop.multiProcessorCount;
        info.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && info.cus > 0;
    });
    return &g_dev[dev];
}

qsa_status check_device(const qsa_dims *d)
{
    int dev = 0;
    const DeviceInfo *info = device_info(dev);
    if (!info || !info->ok) return QSA_ERR_DEVICE;
    const int64_t stride = (d->Skv + kTile - 1) / kTile * kTile;
    const size_t lds = (size_t)(stride / 32) * 4 + 257 * 4;
    if (lds > info->max_lds) return QSA_ERR_SHAPE;
    return QSA_OK;
}

// Resident waves of the gathered forward and dQ passes: two per SIMD, four
// SIMDs per CU (their register use keeps two waves per SIMD). Called after
// check_device has succeeded on the current device.
uint32_t walk_slots()
{
    int dev = 0;
    const DeviceInfo *info = device_info(dev);
    return info && info->ok ? info->cus * 8u : 1u;
}

void fill_common(Problem &p, const qsa_dims *d, const void *routes, float scale)
{
    std::memset(&p, 0, sizeof(p));
    p.B = d->B;
    p.Sq = d->Sq;
    p.Skv = d->Skv;
    p.Hq = d->Hq;
    p.Hkv = d->Hkv;
    p.W = d->W;
    p.route_is_i64 = d->route_is_i64;
    p.flags = d->flags;
    p.nQT = (d->Sq + kTile - 1) / kTile;
    p.nKT = (d->Skv + kTile - 1) / kTile;
    p.stride = p.nKT * kTile;
    p.seg_tiles = seg_tiles_for(d);
    p.nseg = (p.nQT + p.seg_tiles - 1) / p.seg_tiles;
    p.nslot = p.nseg + 1;
    p.scale = scale;
    p.routes = routes;
}

void carve(Problem &p, const Layout &L, void *ws)
{
    char *w = static_cast<char *>(ws);
    const size_t none = (size_t)-1;
    if (L.memb != none) p.memb = reinterpret_cast<uint8_t *>(w + L.memb);
    if (L.has != none) p.has_routes = reinterpret_cast<uint8_t *>(w + L.has);
    if (L.mbits != none) p.mbits = reinterpret_cast<uint32_t *>(w + L.mbits);
    p.row_keys = reinterpret_cast<int32_t *>(w + L.row_keys);
    p.row_cnt = reinterpret_cast<int32_t *>(w + L.row_cnt);
    if (L.pkeys != none) {
        p.pkeys = reinterpret_cast<int32_t *>(w + L.pkeys);
        p.pcnt = reinterpret_cast<int32_t *>(w + L.pcnt);
    }
    p.tile_cnt = reinterpret_cast<int32_t *>(w + L.tile_cnt);
    if (L.kinds != none) {
        p.kinds = reinterpret_cast<int32_t *>(w + L.kinds);
        p.fwd_p_cnt = reinterpret_cast<int32_t *>(w + L.fpc);
        p.fwd_p_idx = reinterpret_cast<int32_t *>(w + L.fpi);
        p.fwd_f_cnt = reinterpret_cast<int32_t *>(w + L.ffc);
        p.fwd_f_idx = reinterpret_cast<int32_t *>(w + L.ffi);
        p.rev_p_cnt = reinterpret_cast<int32_t *>(w + L.rpc);
        p.rev_p_idx = reinterpret_cast<int32_t *>(w + L.rpi);
        p.rev_f_cnt = reinterpret_cast<int32_t *>(w + L.rfc);
        p.rev_f_idx = reinterpret_cast<int32_t *>(w + L.rfi);
    }
    if (L.fstate != none) p.fstate = reinterpret_cast<float *>(w + L.fstate);
    if (L.delta != none) p.delta = reinterpret_cast<float *>(w + L.delta);
    if (L.kv_part != none) {
        p.kv_part = reinterpret_cast<float *>(w + L.kv_part);
        p.dq_part = p.kv_part;
    }
    if (L.kv_flag != none) p.kv_flag = reinterpret_cast<uint8_t *>(w + L.kv_flag);
    // Deterministic calls walk every key list from its start (no walk
    // clocks), and so do calls with fewer than eight rows per wave slot: their
    // rows run in a few nearly simultaneous rounds, already in step, and the
    // clock of finished chunks lags the rows in flight (measured: the 8192-
    // and 4096-row workloads were 50 % slower in those passes with rotation).
    const uint32_t slots = walk_slots();
    if (L.walk != none && !(p.flags & QSA_FLAG_DETERMINISTIC) &&
        p.B * p.Sq * p.Hkv >= (int64_t)kWalkRounds * slots) {
        p.walk = reinterpret_cast<uint32_t *>(w + L.walk);
        p.walk_slots = slots;
    }
}

qsa_status check_scale(float scale)
{
    return (std::isfinite(scale) && scale > 0.f) ? QSA_OK : QSA_ERR_SCALE;
}

size_t route_align(const qsa_dims *d) { return d->route_is_i64 ? 8 : 4; }

hipError_t mark(void *const *events, int at, hipStream_t s)
{
    if (!events) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[at]), s);
}

}  // namespace

extern "C" {

size_t qsa_forward_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, 0).total : 0;
}

size_t qsa_backward_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, 1).total : 0;
}

size_t qsa_preprocess_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, 2).total : 0;
}

qsa_status qsa_forward_timed(const qsa_dims *dims, const void *q, const void *k, const void *v,
                             const void *routes, float scale, void *out, float *out_fp32,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream,
                             void *const *events, int32_t n_events)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!q || !k || !v || !routes || !out || !out_fp32 || !lse) return QSA_ERR_NULL;
    if ((st = check_scale(scale)) != QSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(out_fp32, 16) || !aligned(lse, 4) || !aligned(routes, route_align(dims)))
        return QSA_ERR_ALIGN;
    const Layout L = layout(dims, 0);
    if (!workspace || workspace_bytes < L.total) return QSA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QSA_ERR_ALIGN;
    if ((st = check_device(dims)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, routes, scale);
    carve(p, L, workspace);
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.out = static_cast<uint16_t *>(out);
    p.out_fp32 = out_fp32;
    p.lse = lse;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (events && n_events < QSA_FORWARD_STAGES + 1) return QSA_ERR_NULL;
    if (mark(events, 0, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 1, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_forward(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 2, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_forward_dense(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 3, s) != hipSuccess) return QSA_ERR_DEVICE;
    return QSA_OK;
}

qsa_status qsa_forward(const qsa_dims *dims, const void *q, const void *k, const void *v,
                       const void *routes, float scale, void *out, float *out_fp32, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    return qsa_forward_timed(dims, q, k, v, routes, scale, out, out_fp32, lse, workspace,
                             workspace_bytes, stream, nullptr, 0);
}

qsa_status qsa_backward_timed(const qsa_dims *dims, const void *grad_out, const void *q,
                              const void *k, const void *v, const float *out_fp32,
                              const float *lse, const void *routes, float scale, void *dq,
                              void *dk, void *dv, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *events, int32_t n_events)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!grad_out || !q || !k || !v || !out_fp32 || !lse || !routes || !dq || !dk || !dv)
        return QSA_ERR_NULL;
    if ((st = check_scale(scale)) != QSA_OK) return st;
    if (!aligned(grad_out, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(out_fp32, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(routes, route_align(dims)))
        return QSA_ERR_ALIGN;
    const Layout L = layout(dims, 1);
    if (!workspace || workspace_bytes < L.total) return QSA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QSA_ERR_ALIGN;
    if ((st = check_device(dims)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, routes, scale);
    carve(p, L, workspace);
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.dout = static_cast<const uint16_t *>(grad_out);
    p.out_fp32_in = out_fp32;
    p.lse_in = lse;
    p.dq = static_cast<uint16_t *>(dq);
    p.dk = static_cast<uint16_t *>(dk);
    p.dv = static_cast<uint16_t *>(dv);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (events && n_events < QSA_BACKWARD_STAGES + 1) return QSA_ERR_NULL;
    if (mark(events, 0, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 1, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_delta(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 2, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_dq(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 3, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_dq_dense(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 4, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_dkdv(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 5, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_dkdv_dense(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 6, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_dkdv_reduce(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 7, s) != hipSuccess) return QSA_ERR_DEVICE;
    return QSA_OK;
}

qsa_status qsa_backward(const qsa_dims *dims, const void *grad_out, const void *q, const void *k,
                        const void *v, const float *out_fp32, const float *lse,
                        const void *routes, float scale, void *dq, void *dk, void *dv,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return qsa_backward_timed(dims, grad_out, q, k, v, out_fp32, lse, routes, scale, dq, dk, dv,
                              workspace, workspace_bytes, stream, nullptr, 0);
}

qsa_status qsa_preprocess(const qsa_dims *dims, const void *routes, uint8_t *memb,
                          uint8_t *has_routes, int32_t *kinds, int32_t *fwd_p_cnt,
                          int32_t *fwd_p_idx, int32_t *fwd_f_cnt, int32_t *fwd_f_idx,
                          int32_t *rev_p_cnt, int32_t *rev_p_idx, int32_t *rev_f_cnt,
                          int32_t *rev_f_idx, int32_t *row_keys, int32_t *row_cnt,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!routes || !memb || !has_routes || !kinds || !fwd_p_cnt || !fwd_p_idx || !fwd_f_cnt ||
        !fwd_f_idx || !rev_p_cnt || !rev_p_idx || !rev_f_cnt || !rev_f_idx)
        return QSA_ERR_NULL;
    if (!aligned(memb, 16) || !aligned(kinds, 4) || !aligned(fwd_p_cnt, 4) ||
        !aligned(fwd_p_idx, 4) || !aligned(fwd_f_cnt, 4) || !aligned(fwd_f_idx, 4) ||
        !aligned(rev_p_cnt, 4) || !aligned(rev_p_idx, 4) || !aligned(rev_f_cnt, 4) ||
        !aligned(rev_f_idx, 4) || (row_keys && !aligned(row_keys, 4)) ||
        (row_cnt && !aligned(row_cnt, 4)) || !aligned(routes, route_align(dims)))
        return QSA_ERR_ALIGN;
    const Layout L = layout(dims, 2);
    if (!workspace || workspace_bytes < L.total) return QSA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QSA_ERR_ALIGN;
    if ((st = check_device(dims)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, routes, 1.f);
    carve(p, L, workspace);
    p.memb = memb;
    p.has_routes = has_routes;
    p.kinds = kinds;
    p.fwd_p_cnt = fwd_p_cnt;
    p.fwd_p_idx = fwd_p_idx;
    p.fwd_f_cnt = fwd_f_cnt;
    p.fwd_f_idx = fwd_f_idx;
    p.rev_p_cnt = rev_p_cnt;
    p.rev_p_idx = rev_p_idx;
    p.rev_f_cnt = rev_f_cnt;
    p.rev_f_idx = rev_f_idx;
    if (row_keys) p.row_keys = row_keys;
    if (row_cnt) p.row_cnt = row_cnt;
    if (launch_preprocess(p, static_cast<hipStream_t>(stream)) != hipSuccess)
        return QSA_ERR_LAUNCH;
    return QSA_OK;
}

const char *qsa_status_string(qsa_status status)
{
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "a required pointer is NULL";
    case QSA_ERR_SHAPE: return "a dimension is < 1 or beyond the supported limits";
    case QSA_ERR_HEADS: return "Hkv must be >= 1 and Hq must equal 12 * Hkv";
    case QSA_ERR_HEADDIM: return "head dimension must be 256";
    case QSA_ERR_SCALE: return "scale must be finite and > 0";
    case QSA_ERR_ALIGN: return "a pointer is not aligned (16 bytes for tensors, 4/8 for lse and routes)";
    case QSA_ERR_ROUTE_DTYPE: return "routes must be int32 or int64 (route_is_i64 0 or 1), and flags only QSA_FLAG_* bits";
    case QSA_ERR_WORKSPACE: return "workspace is NULL or smaller than the size query returned";
    case QSA_ERR_DEVICE: return "no gfx950 device is current, or the HIP runtime failed";
    case QSA_ERR_LAUNCH: return "a kernel launch failed";
    case QSA_ERR_SCRATCH:
        return "the call needs more workspace than the fixed device scratch of "
               "qsa_forward_noalloc holds (QSA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

int32_t qsa_version(void) { return (1 << 16) | 0; }

}  // extern "C"
