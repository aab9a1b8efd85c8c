// Host side of the QSA C ABI: validation before any launch, workspace sizing
// and carving, and the launch sequence of each call. See include/qsa.h for the
// contract of every entry point.
#include "../../include/qsa_bench.h"

#include <cmath>
#include <climits>
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
        const int64_t bytes = d->B * d->Hkv * (nseg + dense_parts(nQT)) * stride * 2 * kD * 4;
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
        rpc, rpi, rfc, rfi, fstate, delta, kv_part, dq_part, kv_flag, kv_split, walk, total;
};

// Parts of a workspace. The route plan: key lists and tile counts (core),
// the membership bits that dK/dV reads (bits), the partial-tile key lists
// (pkeys) and the tile kinds and tile lists (lists). The per-call scratch:
// the forward's hand-over state (fwd), the backward's delta, partial sums and
// flags (bwd), and the walk clocks of the gathered passes (walk).
enum Part : unsigned {
    kKeys = 1u,
    kBits = 2u,
    kPkeys = 4u,
    kLists = 8u,
    kFwd = 16u,
    kBwd = 32u,
    kWalk = 64u,
    kTiles = 128u,
    kCore = kKeys | kTiles,
    // Plans and backward calls keep the membership bits, from which the
    // partial-tile lists are built directly (no full key lists); the plain
    // forward keeps the full key lists instead, which are the smaller of the
    // two when Skv is large against W.
    kPlanParts = kTiles | kBits | kPkeys | kLists,
    kForwardParts = kCore | kPkeys | kLists | kFwd | kWalk,
    kBackwardParts = kTiles | kBits | kPkeys | kLists | kBwd | kWalk,
};

Layout layout(const qsa_dims *d, unsigned parts)
{
    const int64_t nQT = (d->Sq + kTile - 1) / kTile, nKT = (d->Skv + kTile - 1) / kTile;
    const int64_t stride = nKT * kTile;
    const int64_t rows = d->B * d->Sq;
    const size_t none = (size_t)-1;
    Layout L;
    std::memset(&L, 0xff, sizeof(L));
    size_t off = 0;
    auto take = [&](bool want, size_t bytes) {
        if (!want) return none;
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    // The byte membership table and has_routes are outputs of qsa_preprocess
    // only (caller buffers): no forward or backward kernel reads them, so those
    // calls do not materialise them.
    L.mbits = take(parts & kBits, (size_t)(rows * (stride / 32)) * 4);
    L.row_keys = take(parts & kKeys, (size_t)(rows * d->W) * 4);
    L.row_cnt = take(parts & kKeys, (size_t)rows * 4);
    L.pkeys = take(parts & kPkeys, (size_t)(rows * d->W) * 4);
    L.pcnt = take(parts & kPkeys, (size_t)rows * 4);
    L.tile_cnt = take(parts & kTiles, (size_t)(d->B * nQT * nKT) * 4);
    const bool lists = parts & kLists;
    L.kinds = take(lists, (size_t)(d->B * nQT * nKT) * 4);
    L.fpc = take(lists, (size_t)(d->B * nQT) * 4);
    L.fpi = take(lists, (size_t)(d->B * nQT * nKT) * 4);
    L.ffc = take(lists, (size_t)(d->B * nQT) * 4);
    L.ffi = take(lists, (size_t)(d->B * nQT * nKT) * 4);
    L.rpc = take(lists, (size_t)(d->B * nKT) * 4);
    L.rpi = take(lists, (size_t)(d->B * nKT * nQT) * 4);
    L.rfc = take(lists, (size_t)(d->B * nKT) * 4);
    L.rfi = take(lists, (size_t)(d->B * nKT * nQT) * 4);
    L.fstate = take(parts & kFwd, (size_t)(d->B * d->Hq * d->Sq) * 8);
    L.delta = take(parts & kBwd, (size_t)(d->B * d->Hq * d->Sq) * 4);
    const int64_t seg = seg_tiles_for(d);
    const int64_t nseg = (nQT + seg - 1) / seg;
    // The dK/dV partial sums and the dQ hand-over each have a region: the
    // backward runs its dQ passes beside the dK/dV passes.
    const int64_t nslot = nseg + dense_parts(nQT);
    const size_t kv_bytes = (size_t)(d->B * d->Hkv * nslot * stride) * 2 * kD * 4;
    const size_t dq_bytes = (size_t)(rows * d->Hq) * kD * 4;
    L.kv_part = take(parts & kBwd, kv_bytes);
    L.dq_part = take(parts & kBwd, dq_bytes);
    L.kv_flag = take(parts & kBwd, (size_t)(d->B * d->Hkv * nslot * (stride / 16)));
    const int64_t merge = seg < kMergeTiles ? kMergeTiles / seg : 1;
    L.kv_split = take(parts & kBwd, (size_t)(d->B * d->Hkv * ((nseg + merge - 1) / merge) * (stride / 16)));
    L.walk = take(parts & kWalk, 16 * 4);
    L.memb = L.has = none;
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

// A second stream per device for the backward's dQ passes, which run beside
// its dK/dV passes: the two share only read-only inputs, delta and the plan.
// Created on first use with the default priority and kept until the process
// ends; the mutex makes each call's fork and join one unit, so calls from
// several host threads cannot pair their events with another call's.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool ok = false;
    std::mutex m;
};
SideStream g_side[kMaxDevices];
std::once_flag g_side_once[kMaxDevices];

SideStream *side_stream()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_side_once[dev], [dev]() {
        SideStream &x = g_side[dev];
        x.ok = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess &&
               hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) == hipSuccess &&
               hipEventCreateWithFlags(&x.join, hipEventDisableTiming) == hipSuccess;
    });
    return g_side[dev].ok ? &g_side[dev] : nullptr;
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
    p.nslot = p.nseg + dense_parts(p.nQT);
    p.merge = p.seg_tiles < kMergeTiles ? kMergeTiles / p.seg_tiles : 1;
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
    if (L.row_keys != none) {
        p.row_keys = reinterpret_cast<int32_t *>(w + L.row_keys);
        p.row_cnt = reinterpret_cast<int32_t *>(w + L.row_cnt);
    }
    if (L.tile_cnt != none) p.tile_cnt = reinterpret_cast<int32_t *>(w + L.tile_cnt);
    if (L.pkeys != none) {
        p.pkeys = reinterpret_cast<int32_t *>(w + L.pkeys);
        p.pcnt = reinterpret_cast<int32_t *>(w + L.pcnt);
    }
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
    if (L.kv_part != none) p.kv_part = reinterpret_cast<float *>(w + L.kv_part);
    if (L.dq_part != none) p.dq_part = reinterpret_cast<float *>(w + L.dq_part);
    if (L.kv_flag != none) p.kv_flag = reinterpret_cast<uint8_t *>(w + L.kv_flag);
    if (L.kv_split != none) p.kv_split = reinterpret_cast<uint8_t *>(w + L.kv_split);
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

qsa_status check_forward_args(const void *q, const void *k, const void *v, float scale,
                              const void *out, const float *out_fp32, const float *lse)
{
    if (!q || !k || !v || !out || !out_fp32 || !lse) return QSA_ERR_NULL;
    const qsa_status st = check_scale(scale);
    if (st != QSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(out_fp32, 16) || !aligned(lse, 4))
        return QSA_ERR_ALIGN;
    return QSA_OK;
}

qsa_status check_backward_args(const void *grad_out, const void *q, const void *k, const void *v,
                               const float *out_fp32, const float *lse, float scale,
                               const void *dq, const void *dk, const void *dv)
{
    if (!grad_out || !q || !k || !v || !out_fp32 || !lse || !dq || !dk || !dv)
        return QSA_ERR_NULL;
    const qsa_status st = check_scale(scale);
    if (st != QSA_OK) return st;
    if (!aligned(grad_out, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(out_fp32, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16))
        return QSA_ERR_ALIGN;
    return QSA_OK;
}

// A workspace of `need` bytes: present (when needed), large enough, aligned.
qsa_status check_workspace(const void *ws, size_t bytes, size_t need)
{
    if (need > 0 && (!ws || bytes < need)) return QSA_ERR_WORKSPACE;
    if (ws && !aligned(ws, 16)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

// A plan that qsa_plan_build filled in and that still describes valid dims
// and a large enough buffer (the caller may have edited the struct).
qsa_status check_plan(const qsa_plan *plan)
{
    if (!plan) return QSA_ERR_NULL;
    if (plan->tag != QSA_PLAN_TAG) return QSA_ERR_PLAN;
    const qsa_status st = check_dims(&plan->dims);
    if (st != QSA_OK) return st;
    if (!plan->mem || plan->bytes < layout(&plan->dims, kPlanParts).total) return QSA_ERR_PLAN;
    if (!aligned(plan->mem, 16)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

// The current device is the one the plan was built on.
qsa_status check_plan_device(const qsa_plan *plan)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;
    return dev == plan->device ? QSA_OK : QSA_ERR_PLAN;
}

// The route-set dims of a block-bitmap call: one batch of T packed tokens as
// queries and keys, and a per-row key capacity that no selection can exceed
// (a block holds at most four keys of a row's range, so at most 4 NB keys,
// and there are T keys in all).
qsa_status block_dims(const qsa_block_dims *bd, qsa_dims *d)
{
    if (!bd) return QSA_ERR_NULL;
    if (bd->block_size != 4 || bd->T < 1 || bd->NB < 1 || bd->NB > INT32_MAX)
        return QSA_ERR_SHAPE;
    d->B = 1;
    d->Sq = d->Skv = bd->T;
    d->Hq = bd->Hq;
    d->Hkv = bd->Hkv;
    d->D = bd->D;
    d->W = bd->T < 4 * bd->NB ? bd->T : 4 * bd->NB;
    d->route_is_i64 = 0;
    d->flags = bd->flags;
    return check_dims(d);
}

qsa_status check_block_meta(const uint8_t *sel, const int32_t *lo, const int32_t *hi,
                            const int32_t *blk_base, const int32_t *tok_base,
                            const int32_t *block_first, const int32_t *block_last)
{
    if (!sel || !lo || !hi || !blk_base || !tok_base || !block_first || !block_last)
        return QSA_ERR_NULL;
    if (!aligned(lo, 4) || !aligned(hi, 4) || !aligned(blk_base, 4) || !aligned(tok_base, 4) ||
        !aligned(block_first, 4) || !aligned(block_last, 4))
        return QSA_ERR_ALIGN;
    return QSA_OK;
}

// Build a plan from a block selection into plan_mem (validated by the caller).
qsa_status build_block_plan(const qsa_dims *d, int64_t NB, const uint8_t *sel, const int32_t *lo,
                            const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                            void *plan_mem, size_t plan_bytes, qsa_plan *plan, hipStream_t s)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;
    Problem p;
    fill_common(p, d, nullptr, 1.f);
    p.sel = sel;
    p.sel_lo = lo;
    p.sel_hi = hi;
    p.sel_blk_base = blk_base;
    p.sel_tok_base = tok_base;
    p.NB = NB;
    carve(p, layout(d, kPlanParts), plan_mem);
    if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    plan->dims = *d;
    plan->mem = plan_mem;
    plan->bytes = plan_bytes;
    plan->device = dev;
    plan->tag = QSA_PLAN_TAG;
    return QSA_OK;
}

// The route-set dims of a document-causal call: a row holds at most the keys
// up to its global position, so min(Skv, q_global_start + Sq) per row.
qsa_status doc_dims(const qsa_doc_dims *dd, qsa_dims *d)
{
    if (!dd) return QSA_ERR_NULL;
    if (dd->reserved != 0) return QSA_ERR_ROUTE_DTYPE;
    if (dd->q_global_start < 0 || dd->Sq < 1 || dd->Skv < 1 ||
        dd->q_global_start > (int64_t(1) << 40))
        return QSA_ERR_SHAPE;
    d->B = dd->B;
    d->Sq = dd->Sq;
    d->Skv = dd->Skv;
    d->Hq = dd->Hq;
    d->Hkv = dd->Hkv;
    d->D = dd->D;
    const int64_t reach = dd->q_global_start + dd->Sq;
    d->W = dd->Skv < reach ? dd->Skv : reach;
    d->route_is_i64 = 0;
    d->flags = dd->flags;
    return check_dims(d);
}

qsa_status check_doc_ids(const int32_t *q_doc, const int32_t *kv_doc)
{
    if (!q_doc || !kv_doc) return QSA_ERR_NULL;
    if (!aligned(q_doc, 4) || !aligned(kv_doc, 4)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

// Build a plan from document ids into plan_mem (validated by the caller).
qsa_status build_doc_plan(const qsa_dims *d, const int32_t *q_doc, const int32_t *kv_doc,
                          int64_t q_global_start, void *plan_mem, size_t plan_bytes,
                          qsa_plan *plan, hipStream_t s)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;
    Problem p;
    fill_common(p, d, nullptr, 1.f);
    p.q_doc = q_doc;
    p.kv_doc = kv_doc;
    p.q_global_start = q_global_start;
    carve(p, layout(d, kPlanParts), plan_mem);
    if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    plan->dims = *d;
    plan->mem = plan_mem;
    plan->bytes = plan_bytes;
    plan->device = dev;
    plan->tag = QSA_PLAN_TAG;
    return QSA_OK;
}

// Forward launches after validation. With `prep` the route preprocessing
// runs first into the workspace; otherwise a plan supplies its results and
// only the walk clocks are reset.
qsa_status run_forward(Problem &p, const void *q, const void *k, const void *v, void *out,
                       float *out_fp32, float *lse, hipStream_t s, void *const *events, bool prep)
{
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.out = static_cast<uint16_t *>(out);
    p.out_fp32 = out_fp32;
    p.lse = lse;
    if (mark(events, 0, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (prep) {
        if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    } else if (launch_walk_reset(p, s) != hipSuccess) {
        return QSA_ERR_LAUNCH;
    }
    if (mark(events, 1, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_forward(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 2, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_forward_dense(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 3, s) != hipSuccess) return QSA_ERR_DEVICE;
    return QSA_OK;
}

// Backward launches after validation; `prep` as for run_forward.
qsa_status run_backward(Problem &p, const void *grad_out, const void *q, const void *k,
                        const void *v, const float *out_fp32, const float *lse, void *dq, void *dk,
                        void *dv, hipStream_t s, void *const *events, bool prep)
{
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.dout = static_cast<const uint16_t *>(grad_out);
    p.out_fp32_in = out_fp32;
    p.lse_in = lse;
    p.dq = static_cast<uint16_t *>(dq);
    p.dk = static_cast<uint16_t *>(dk);
    p.dv = static_cast<uint16_t *>(dv);
    if (mark(events, 0, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (prep) {
        if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    } else if (launch_walk_reset(p, s) != hipSuccess) {
        return QSA_ERR_LAUNCH;
    }
    if (mark(events, 1, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (launch_delta(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    // Without stage events the dQ passes run on the side stream, forked after
    // delta and joined before the reduce, beside the dK/dV passes. The dense
    // dK/dV pass goes first, so that each stream's gathered pass meets the
    // other's dense (matrix-core-bound) pass: the gathered dQ beside the dense
    // dK/dV, then the dense dQ beside the gathered dK/dV (measured 0.35 ms
    // faster per 32k step than the gathered dK/dV first). With stage events
    // the passes run one after the other, so that each has its own time.
    SideStream *x = events ? nullptr : side_stream();
    if (x) {
        std::lock_guard<std::mutex> lock(x->m);
        if (hipEventRecord(x->fork, s) != hipSuccess ||
            hipStreamWaitEvent(x->s, x->fork, 0) != hipSuccess)
            return QSA_ERR_DEVICE;
        if (launch_dkdv_dense(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (launch_dq(p, x->s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (launch_dq_dense(p, x->s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (hipEventRecord(x->join, x->s) != hipSuccess) return QSA_ERR_DEVICE;
        if (launch_dkdv(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
        if (hipStreamWaitEvent(s, x->join, 0) != hipSuccess) return QSA_ERR_DEVICE;
        if (launch_dkdv_reduce(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
        return QSA_OK;
    }
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

// ---- block selector ----

qsa_status check_select_dims(const qsa_select_dims *d)
{
    if (!d) return QSA_ERR_NULL;
    if (d->flags != 0) return QSA_ERR_ROUTE_DTYPE;
    if (d->D != kSelD) return QSA_ERR_HEADDIM;
    if (d->B < 1 || d->Sq < 1 || d->NB < 1 || d->NB > 32768 || d->H < 1 || d->H > 64 ||
        d->top_k < 1 || d->top_k > 4096 || d->q_offset < 0)
        return QSA_ERR_SHAPE;
    if (d->B > INT32_MAX / d->Sq || d->q_offset + d->Sq > (int64_t)INT32_MAX) return QSA_ERR_SHAPE;
    return QSA_OK;
}

size_t select_scores_bytes(const qsa_select_dims *d)
{
    return (size_t)d->B * (size_t)d->Sq * (size_t)d->NB * sizeof(float);
}

}  // namespace

extern "C" {

size_t qsa_forward_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kForwardParts).total : 0;
}

size_t qsa_backward_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kBackwardParts).total : 0;
}

size_t qsa_preprocess_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kCore).total : 0;
}

qsa_status qsa_forward_timed(const qsa_dims *dims, const void *q, const void *k, const void *v,
                             const void *routes, float scale, void *out, float *out_fp32,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream,
                             void *const *events, int32_t n_events)
{
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!routes) return QSA_ERR_NULL;
    if ((st = check_forward_args(q, k, v, scale, out, out_fp32, lse)) != QSA_OK) return st;
    if (!aligned(routes, route_align(dims))) return QSA_ERR_ALIGN;
    const Layout L = layout(dims, kForwardParts);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != QSA_OK) return st;
    if (events && n_events < QSA_FORWARD_STAGES + 1) return QSA_ERR_NULL;
    if ((st = check_device(dims)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, routes, scale);
    carve(p, L, workspace);
    return run_forward(p, q, k, v, out, out_fp32, lse, static_cast<hipStream_t>(stream), events,
                       true);
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
    if (!routes) return QSA_ERR_NULL;
    if ((st = check_backward_args(grad_out, q, k, v, out_fp32, lse, scale, dq, dk, dv)) != QSA_OK)
        return st;
    if (!aligned(routes, route_align(dims))) return QSA_ERR_ALIGN;
    const Layout L = layout(dims, kBackwardParts);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != QSA_OK) return st;
    if (events && n_events < QSA_BACKWARD_STAGES + 1) return QSA_ERR_NULL;
    if ((st = check_device(dims)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, routes, scale);
    carve(p, L, workspace);
    return run_backward(p, grad_out, q, k, v, out_fp32, lse, dq, dk, dv,
                        static_cast<hipStream_t>(stream), events, true);
}

qsa_status qsa_backward(const qsa_dims *dims, const void *grad_out, const void *q, const void *k,
                        const void *v, const float *out_fp32, const float *lse,
                        const void *routes, float scale, void *dq, void *dk, void *dv,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return qsa_backward_timed(dims, grad_out, q, k, v, out_fp32, lse, routes, scale, dq, dk, dv,
                              workspace, workspace_bytes, stream, nullptr, 0);
}

size_t qsa_plan_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kPlanParts).total : 0;
}

size_t qsa_forward_planned_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kFwd | kWalk).total : 0;
}

size_t qsa_backward_planned_workspace_bytes(const qsa_dims *dims)
{
    return check_dims(dims) == QSA_OK ? layout(dims, kBwd | kWalk).total : 0;
}

qsa_status qsa_plan_build(const qsa_dims *dims, const void *routes, void *plan_mem,
                          size_t plan_bytes, qsa_plan *plan, void *stream)
{
    if (!plan) return QSA_ERR_NULL;
    std::memset(plan, 0, sizeof(*plan));
    qsa_status st = check_dims(dims);
    if (st != QSA_OK) return st;
    if (!routes) return QSA_ERR_NULL;
    if (!aligned(routes, route_align(dims))) return QSA_ERR_ALIGN;
    const Layout L = layout(dims, kPlanParts);
    if ((st = check_workspace(plan_mem, plan_bytes, L.total)) != QSA_OK) return st;
    if ((st = check_device(dims)) != QSA_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;

    Problem p;
    fill_common(p, dims, routes, 1.f);
    carve(p, L, plan_mem);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_preprocess(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_partial_keys(p, s) != hipSuccess) return QSA_ERR_LAUNCH;
    plan->dims = *dims;
    plan->mem = plan_mem;
    plan->bytes = plan_bytes;
    plan->device = dev;
    plan->tag = QSA_PLAN_TAG;
    return QSA_OK;
}

qsa_status qsa_forward_planned_timed(const qsa_plan *plan, const void *q, const void *k,
                                     const void *v, float scale, void *out, float *out_fp32,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream, void *const *events, int32_t n_events)
{
    qsa_status st = check_plan(plan);
    if (st != QSA_OK) return st;
    const qsa_dims *dims = &plan->dims;
    if ((st = check_forward_args(q, k, v, scale, out, out_fp32, lse)) != QSA_OK) return st;
    const Layout L = layout(dims, kFwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != QSA_OK) return st;
    if (events && n_events < QSA_FORWARD_STAGES + 1) return QSA_ERR_NULL;
    if ((st = check_device(dims)) != QSA_OK) return st;
    if ((st = check_plan_device(plan)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, nullptr, scale);
    carve(p, layout(dims, kPlanParts), plan->mem);
    carve(p, L, workspace);
    return run_forward(p, q, k, v, out, out_fp32, lse, static_cast<hipStream_t>(stream), events,
                       false);
}

qsa_status qsa_forward_planned(const qsa_plan *plan, const void *q, const void *k, const void *v,
                               float scale, void *out, float *out_fp32, float *lse,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    return qsa_forward_planned_timed(plan, q, k, v, scale, out, out_fp32, lse, workspace,
                                     workspace_bytes, stream, nullptr, 0);
}

qsa_status qsa_backward_planned_timed(const qsa_plan *plan, const void *grad_out, const void *q,
                                      const void *k, const void *v, const float *out_fp32,
                                      const float *lse, float scale, void *dq, void *dk,
                                      void *dv, void *workspace, size_t workspace_bytes,
                                      void *stream, void *const *events, int32_t n_events)
{
    qsa_status st = check_plan(plan);
    if (st != QSA_OK) return st;
    const qsa_dims *dims = &plan->dims;
    if ((st = check_backward_args(grad_out, q, k, v, out_fp32, lse, scale, dq, dk, dv)) != QSA_OK)
        return st;
    const Layout L = layout(dims, kBwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != QSA_OK) return st;
    if (events && n_events < QSA_BACKWARD_STAGES + 1) return QSA_ERR_NULL;
    if ((st = check_device(dims)) != QSA_OK) return st;
    if ((st = check_plan_device(plan)) != QSA_OK) return st;

    Problem p;
    fill_common(p, dims, nullptr, scale);
    carve(p, layout(dims, kPlanParts), plan->mem);
    carve(p, L, workspace);
    return run_backward(p, grad_out, q, k, v, out_fp32, lse, dq, dk, dv,
                        static_cast<hipStream_t>(stream), events, false);
}

qsa_status qsa_backward_planned(const qsa_plan *plan, const void *grad_out, const void *q,
                                const void *k, const void *v, const float *out_fp32,
                                const float *lse, float scale, void *dq, void *dk, void *dv,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    return qsa_backward_planned_timed(plan, grad_out, q, k, v, out_fp32, lse, scale, dq, dk, dv,
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
    const Layout L = layout(dims, kCore);
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

qsa_status qsa_plan_tables(const qsa_plan *plan, uint32_t *mbits, int32_t *kinds,
                           int32_t *fwd_p_cnt, int32_t *fwd_p_idx, int32_t *fwd_f_cnt,
                           int32_t *fwd_f_idx, int32_t *rev_p_cnt, int32_t *rev_p_idx,
                           int32_t *rev_f_cnt, int32_t *rev_f_idx, int32_t *row_keys,
                           int32_t *row_cnt, void *stream)
{
    qsa_status st = check_plan(plan);
    if (st != QSA_OK) return st;
    if (!mbits || !kinds || !fwd_p_cnt || !fwd_p_idx || !fwd_f_cnt || !fwd_f_idx || !rev_p_cnt ||
        !rev_p_idx || !rev_f_cnt || !rev_f_idx || !row_keys || !row_cnt)
        return QSA_ERR_NULL;
    for (const void *x : {(const void *)mbits, (const void *)kinds, (const void *)fwd_p_cnt,
                          (const void *)fwd_p_idx, (const void *)fwd_f_cnt,
                          (const void *)fwd_f_idx, (const void *)rev_p_cnt,
                          (const void *)rev_p_idx, (const void *)rev_f_cnt,
                          (const void *)rev_f_idx, (const void *)row_keys, (const void *)row_cnt})
        if (!aligned(x, 4)) return QSA_ERR_ALIGN;
    if ((st = check_device(&plan->dims)) != QSA_OK) return st;
    if ((st = check_plan_device(plan)) != QSA_OK) return st;
    const qsa_dims *d = &plan->dims;
    const Layout L = layout(d, kPlanParts);
    const int64_t nQT = (d->Sq + kTile - 1) / kTile, nKT = (d->Skv + kTile - 1) / kTile;
    const int64_t rows = d->B * d->Sq;
    const char *m = static_cast<const char *>(plan->mem);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    struct Copy {
        void *dst;
        size_t at, bytes;
    } copies[] = {
        {mbits, L.mbits, (size_t)(rows * (nKT * kTile / 32)) * 4},
        {kinds, L.kinds, (size_t)(d->B * nQT * nKT) * 4},
        {fwd_p_cnt, L.fpc, (size_t)(d->B * nQT) * 4},
        {fwd_p_idx, L.fpi, (size_t)(d->B * nQT * nKT) * 4},
        {fwd_f_cnt, L.ffc, (size_t)(d->B * nQT) * 4},
        {fwd_f_idx, L.ffi, (size_t)(d->B * nQT * nKT) * 4},
        {rev_p_cnt, L.rpc, (size_t)(d->B * nKT) * 4},
        {rev_p_idx, L.rpi, (size_t)(d->B * nKT * nQT) * 4},
        {rev_f_cnt, L.rfc, (size_t)(d->B * nKT) * 4},
        {rev_f_idx, L.rfi, (size_t)(d->B * nKT * nQT) * 4},
    };
    for (const Copy &c : copies)
        if (hipMemcpyAsync(c.dst, m + c.at, c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return QSA_ERR_DEVICE;
    // The plan holds no full key lists: they are built from its membership bits.
    Problem p;
    fill_common(p, d, nullptr, 1.f);
    carve(p, L, plan->mem);
    if (launch_row_keys(p, row_keys, row_cnt, s) != hipSuccess) return QSA_ERR_LAUNCH;
    return QSA_OK;
}

size_t qsa_block_plan_bytes(const qsa_block_dims *dims)
{
    qsa_dims d;
    return block_dims(dims, &d) == QSA_OK ? layout(&d, kPlanParts).total : 0;
}

size_t qsa_block_forward_workspace_bytes(const qsa_block_dims *dims)
{
    qsa_dims d;
    if (block_dims(dims, &d) != QSA_OK) return 0;
    return layout(&d, kPlanParts).total + layout(&d, kFwd | kWalk).total;
}

size_t qsa_block_backward_workspace_bytes(const qsa_block_dims *dims)
{
    qsa_dims d;
    if (block_dims(dims, &d) != QSA_OK) return 0;
    return layout(&d, kPlanParts).total + layout(&d, kBwd | kWalk).total;
}

qsa_status qsa_block_plan_build(const qsa_block_dims *dims, const uint8_t *sel_blocks,
                                const int32_t *lo, const int32_t *hi, const int32_t *blk_base,
                                const int32_t *tok_base, const int32_t *block_first,
                                const int32_t *block_last, void *plan_mem, size_t plan_bytes,
                                qsa_plan *plan, void *stream)
{
    if (!plan) return QSA_ERR_NULL;
    std::memset(plan, 0, sizeof(*plan));
    qsa_dims d;
    qsa_status st = block_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last)) !=
        QSA_OK)
        return st;
    if ((st = check_workspace(plan_mem, plan_bytes, layout(&d, kPlanParts).total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    return build_block_plan(&d, dims->NB, sel_blocks, lo, hi, blk_base, tok_base, plan_mem,
                            plan_bytes, plan, static_cast<hipStream_t>(stream));
}

qsa_status qsa_block_forward(const qsa_block_dims *dims, const void *q, const void *k,
                             const void *v, const uint8_t *sel_blocks, const int32_t *lo,
                             const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                             const int32_t *block_first, const int32_t *block_last, float scale,
                             void *out, float *out_fp32, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    qsa_dims d;
    qsa_status st = block_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last)) !=
        QSA_OK)
        return st;
    if ((st = check_forward_args(q, k, v, scale, out, out_fp32, lse)) != QSA_OK) return st;
    const size_t plan_bytes = layout(&d, kPlanParts).total;
    const Layout L = layout(&d, kFwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, plan_bytes + L.total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    qsa_plan plan;
    std::memset(&plan, 0, sizeof(plan));
    if ((st = build_block_plan(&d, dims->NB, sel_blocks, lo, hi, blk_base, tok_base, workspace,
                               plan_bytes, &plan, s)) != QSA_OK)
        return st;
    Problem p;
    fill_common(p, &d, nullptr, scale);
    carve(p, layout(&d, kPlanParts), workspace);
    carve(p, L, static_cast<char *>(workspace) + plan_bytes);
    return run_forward(p, q, k, v, out, out_fp32, lse, s, nullptr, false);
}

qsa_status qsa_block_backward(const qsa_block_dims *dims, const void *grad_out, const void *q,
                              const void *k, const void *v, const float *out_fp32,
                              const float *lse, const uint8_t *sel_blocks, const int32_t *lo,
                              const int32_t *hi, const int32_t *blk_base, const int32_t *tok_base,
                              const int32_t *block_first, const int32_t *block_last, float scale,
                              void *dq, void *dk, void *dv, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    qsa_dims d;
    qsa_status st = block_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last)) !=
        QSA_OK)
        return st;
    if ((st = check_backward_args(grad_out, q, k, v, out_fp32, lse, scale, dq, dk, dv)) != QSA_OK)
        return st;
    const size_t plan_bytes = layout(&d, kPlanParts).total;
    const Layout L = layout(&d, kBwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, plan_bytes + L.total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    qsa_plan plan;
    std::memset(&plan, 0, sizeof(plan));
    if ((st = build_block_plan(&d, dims->NB, sel_blocks, lo, hi, blk_base, tok_base, workspace,
                               plan_bytes, &plan, s)) != QSA_OK)
        return st;
    Problem p;
    fill_common(p, &d, nullptr, scale);
    carve(p, layout(&d, kPlanParts), workspace);
    carve(p, L, static_cast<char *>(workspace) + plan_bytes);
    return run_backward(p, grad_out, q, k, v, out_fp32, lse, dq, dk, dv, s, nullptr, false);
}

size_t qsa_doc_plan_bytes(const qsa_doc_dims *dims)
{
    qsa_dims d;
    return doc_dims(dims, &d) == QSA_OK ? layout(&d, kPlanParts).total : 0;
}

size_t qsa_doc_forward_workspace_bytes(const qsa_doc_dims *dims)
{
    qsa_dims d;
    if (doc_dims(dims, &d) != QSA_OK) return 0;
    return layout(&d, kPlanParts).total + layout(&d, kFwd | kWalk).total;
}

size_t qsa_doc_backward_workspace_bytes(const qsa_doc_dims *dims)
{
    qsa_dims d;
    if (doc_dims(dims, &d) != QSA_OK) return 0;
    return layout(&d, kPlanParts).total + layout(&d, kBwd | kWalk).total;
}

qsa_status qsa_doc_plan_build(const qsa_doc_dims *dims, const int32_t *q_doc_ids,
                              const int32_t *kv_doc_ids, void *plan_mem, size_t plan_bytes,
                              qsa_plan *plan, void *stream)
{
    if (!plan) return QSA_ERR_NULL;
    std::memset(plan, 0, sizeof(*plan));
    qsa_dims d;
    qsa_status st = doc_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_doc_ids(q_doc_ids, kv_doc_ids)) != QSA_OK) return st;
    if ((st = check_workspace(plan_mem, plan_bytes, layout(&d, kPlanParts).total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    return build_doc_plan(&d, q_doc_ids, kv_doc_ids, dims->q_global_start, plan_mem, plan_bytes,
                          plan, static_cast<hipStream_t>(stream));
}

qsa_status qsa_doc_forward(const qsa_doc_dims *dims, const void *q, const void *k, const void *v,
                           const int32_t *q_doc_ids, const int32_t *kv_doc_ids, float scale,
                           void *out, float *out_fp32, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    qsa_dims d;
    qsa_status st = doc_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_doc_ids(q_doc_ids, kv_doc_ids)) != QSA_OK) return st;
    if ((st = check_forward_args(q, k, v, scale, out, out_fp32, lse)) != QSA_OK) return st;
    const size_t plan_bytes = layout(&d, kPlanParts).total;
    const Layout L = layout(&d, kFwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, plan_bytes + L.total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    qsa_plan plan;
    std::memset(&plan, 0, sizeof(plan));
    if ((st = build_doc_plan(&d, q_doc_ids, kv_doc_ids, dims->q_global_start, workspace,
                             plan_bytes, &plan, s)) != QSA_OK)
        return st;
    Problem p;
    fill_common(p, &d, nullptr, scale);
    carve(p, layout(&d, kPlanParts), workspace);
    carve(p, L, static_cast<char *>(workspace) + plan_bytes);
    return run_forward(p, q, k, v, out, out_fp32, lse, s, nullptr, false);
}

qsa_status qsa_doc_backward(const qsa_doc_dims *dims, const void *grad_out, const void *q,
                            const void *k, const void *v, const float *out_fp32,
                            const float *lse, const int32_t *q_doc_ids,
                            const int32_t *kv_doc_ids, float scale, void *dq, void *dk, void *dv,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    qsa_dims d;
    qsa_status st = doc_dims(dims, &d);
    if (st != QSA_OK) return st;
    if ((st = check_doc_ids(q_doc_ids, kv_doc_ids)) != QSA_OK) return st;
    if ((st = check_backward_args(grad_out, q, k, v, out_fp32, lse, scale, dq, dk, dv)) != QSA_OK)
        return st;
    const size_t plan_bytes = layout(&d, kPlanParts).total;
    const Layout L = layout(&d, kBwd | kWalk);
    if ((st = check_workspace(workspace, workspace_bytes, plan_bytes + L.total)) != QSA_OK)
        return st;
    if ((st = check_device(&d)) != QSA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    qsa_plan plan;
    std::memset(&plan, 0, sizeof(plan));
    if ((st = build_doc_plan(&d, q_doc_ids, kv_doc_ids, dims->q_global_start, workspace,
                             plan_bytes, &plan, s)) != QSA_OK)
        return st;
    Problem p;
    fill_common(p, &d, nullptr, scale);
    carve(p, layout(&d, kPlanParts), workspace);
    carve(p, L, static_cast<char *>(workspace) + plan_bytes);
    return run_backward(p, grad_out, q, k, v, out_fp32, lse, dq, dk, dv, s, nullptr, false);
}

size_t qsa_select_workspace_bytes(const qsa_select_dims *dims)
{
    return check_select_dims(dims) == QSA_OK ? select_scores_bytes(dims) : 0;
}

qsa_status qsa_select_timed(const qsa_select_dims *dims, const void *q_idx, const void *kbar,
                            const int32_t *doc_start, const int32_t *blk_base, float scale,
                            int32_t *blocks, int32_t *routes, float *scores, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events,
                            int32_t n_events)
{
    qsa_status st = check_select_dims(dims);
    if (st != QSA_OK) return st;
    if (!q_idx || !kbar || (!blocks && !routes && !scores)) return QSA_ERR_NULL;
    if ((st = check_scale(scale)) != QSA_OK) return st;
    if (!aligned(q_idx, 16) || !aligned(kbar, 16) || !aligned(doc_start, 4) ||
        !aligned(blk_base, 4) || !aligned(blocks, 4) || !aligned(routes, 16) || !aligned(scores, 4))
        return QSA_ERR_ALIGN;
    if (!scores && (st = check_workspace(workspace, workspace_bytes, select_scores_bytes(dims))) !=
                       QSA_OK)
        return st;
    if (events && n_events < QSA_SELECT_STAGES + 1) return QSA_ERR_NULL;
    int dev = 0;
    const DeviceInfo *info = device_info(dev);
    if (!info || !info->ok) return QSA_ERR_DEVICE;

    SelectProblem a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const uint16_t *>(q_idx);
    a.kbar = static_cast<const uint16_t *>(kbar);
    a.doc_start = doc_start;
    a.blk_base = blk_base;
    a.scores = scores ? scores : static_cast<float *>(workspace);
    a.blocks = blocks;
    a.routes = routes;
    a.B = dims->B;
    a.Sq = dims->Sq;
    a.NB = dims->NB;
    a.q_offset = dims->q_offset;
    a.H = dims->H;
    a.top_k = dims->top_k;
    a.scale = scale;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (mark(events, 0, s) != hipSuccess) return QSA_ERR_DEVICE;
    if (scores && launch_select_fill(a, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (launch_select_scores(a, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 1, s) != hipSuccess) return QSA_ERR_DEVICE;
    if ((blocks || routes) && launch_select_topk(a, s) != hipSuccess) return QSA_ERR_LAUNCH;
    if (mark(events, 2, s) != hipSuccess) return QSA_ERR_DEVICE;
    return QSA_OK;
}

qsa_status qsa_select(const qsa_select_dims *dims, const void *q_idx, const void *kbar,
                      const int32_t *doc_start, const int32_t *blk_base, float scale,
                      int32_t *blocks, int32_t *routes, float *scores, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    return qsa_select_timed(dims, q_idx, kbar, doc_start, blk_base, scale, blocks, routes, scores,
                            workspace, workspace_bytes, stream, nullptr, 0);
}

const char *qsa_status_string(qsa_status status)
{
    // A C caller may pass any int: read the bits as an integer, since a C++
    // enum object holding a value outside its enumerators' range is undefined.
    int32_t code;
    static_assert(sizeof(code) == sizeof(status), "qsa_status is 32 bits");
    std::memcpy(&code, &status, sizeof(code));
    switch (code) {
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
    case QSA_ERR_PLAN:
        return "the plan was not built by qsa_plan_build, no longer matches its buffer, or was "
               "built on another device";
    }
    return "unknown status";
}

int32_t qsa_version(void) { return (1 << 16) | 2; }

}  // extern "C"
