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
// dK/dV work segments: kSegTilesMin query tiles, doubled while the FP32
// partial sums of all segments would exceed kPartialBudget bytes. Segments
// are grouped kMergeTiles tiles at a time: one work item takes a whole group
// unless its rows hit the item's 16 keys more than kSplitHits times, and then
// each segment of the group is an item of its own.
constexpr int kSegTilesMin = 2;
constexpr int kMergeTiles = 8;
constexpr int kSplitHits = 256;
constexpr int64_t kPartialBudget = int64_t(4) << 30;
// The dense dK/dV pass takes a key tile's full query tiles kDenseSplit at a
// time, each run into a partial-sum slot of its own after the segments'.
constexpr int kDenseSplit = 48;
__host__ __device__ constexpr int64_t dense_parts(int64_t nQT)
{
    return (nQT + kDenseSplit - 1) / kDenseSplit;
}
constexpr int kMaxSkvLog2 = 19;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Everything the kernels need, with the workspace already carved.
struct Problem {
    int64_t B, Sq, Skv, Hq, Hkv, W;
    int32_t route_is_i64;
    int32_t flags;  // QSA_FLAG_* bits of the call
    int64_t stride;  // membership row stride = nKT * 128
    int64_t nQT, nKT;
    float scale;
    // inputs: route rows, or (routes == nullptr, sel set) a block-selection bitmap
    // sel [Sq, NB] with per-query lo, hi, blk_base, tok_base over packed
    // tokens (B == 1, Sq == Skv)
    const void *routes;
    const uint8_t *sel;
    const int32_t *sel_lo, *sel_hi, *sel_blk_base, *sel_tok_base;
    int64_t NB;
    // or (routes == sel == nullptr) document-causal selection: query i of batch
    // row b at global position q_global_start + i sees key j of its document
    // (q_doc [B, Sq], kv_doc [B, Skv], 0 = padding) with j <= that position
    const int32_t *q_doc, *kv_doc;
    int64_t q_global_start;
    const uint16_t *q, *k, *v, *dout;
    const float *out_fp32_in, *lse_in;
    // preprocessing results (workspace or caller buffers)
    uint8_t *memb, *has_routes;
    uint32_t *mbits;  // bit-packed membership [B*Sq, stride/32] (backward only)
    int32_t *row_keys, *row_cnt;
    // Row key lists without the keys of full tiles (those take the dense
    // path): same layout as row_keys, only the first pcnt[row] entries valid.
    int32_t *pkeys, *pcnt;
    int32_t *tile_cnt, *kinds;
    int32_t *fwd_p_cnt, *fwd_p_idx, *fwd_f_cnt, *fwd_f_idx;
    int32_t *rev_p_cnt, *rev_p_idx, *rev_f_cnt, *rev_f_idx;
    // forward outputs
    uint16_t *out;
    float *out_fp32, *lse;
    // Hand-off from the gathered to the dense forward for rows whose tile row
    // has full tiles: out_fp32 holds the unnormalised output and fstate the
    // (reference maximum in log2 units, sum) pair, [B, Hq, Sq] x 2.
    float *fstate;
    // backward
    float *delta;
    uint16_t *dq, *dk, *dv;
    // dK/dV partial sums: [B*Hkv][nslot][stride][dK 256 | dV 256] FP32, one
    // slot per query segment of the gathered pass, then one per part of the
    // full tiles (dense_parts),
    // and per (B*Hkv, slot, 16-key group) whether a partial was written
    float *kv_part;
    uint8_t *kv_flag;
    // per (B*Hkv, segment group, 16-key group): whether the group's segments
    // are separate work items (see kMergeTiles)
    uint8_t *kv_split;
    int64_t nseg;
    int64_t nslot;      // nseg + dense_parts(nQT) partial-sum slots per (batch, KV head)
    int64_t seg_tiles;  // query tiles per segment
    int64_t merge;      // segments per group (kMergeTiles / seg_tiles, at least 1)
    // Hand-off from the gathered to the dense dQ: unscaled FP32 sums
    // [B, Sq, Hq, 256] of the rows whose tile row has full tiles.
    float *dq_part;
    // Walk clocks of the gathered forward (word 0) and dQ (word 8) passes,
    // zeroed by the preprocessing: the key chunks of the rows finished so far.
    // Null when the call asks for deterministic results.
    uint32_t *walk;
    // Resident waves of those passes (CUs x 4 SIMDs x 2 waves): the walk
    // clock divided by this is how many chunks a wave slot has walked so far.
    uint32_t walk_slots;
};

// Rows per wave slot from which the gathered passes rotate their key walks.
constexpr int kWalkRounds = 8;

hipError_t launch_preprocess(const Problem &p, hipStream_t s);
hipError_t launch_walk_reset(const Problem &p, hipStream_t s);
hipError_t launch_partial_keys(const Problem &p, hipStream_t s);
// The full per-row key lists from the bit-packed membership, into keys [B*Sq, W]
// and cnt [B*Sq].
hipError_t launch_row_keys(const Problem &p, int32_t *keys, int32_t *cnt, hipStream_t s);
hipError_t launch_forward(const Problem &p, hipStream_t s);
hipError_t launch_forward_dense(const Problem &p, hipStream_t s);
hipError_t launch_dq_dense(const Problem &p, hipStream_t s);
hipError_t launch_dkdv_dense(const Problem &p, hipStream_t s);
hipError_t launch_delta(const Problem &p, hipStream_t s);
hipError_t launch_dq(const Problem &p, hipStream_t s);
hipError_t launch_dkdv(const Problem &p, hipStream_t s);
hipError_t launch_dkdv_reduce(const Problem &p, hipStream_t s);

// Block selector: indexer queries q [B, Sq, H, kSelD] and compressed keys
// kbar [B, NB, kSelD] (bf16), optional per-query document start and kbar row
// base [B, Sq]; scores [B, Sq, NB] FP32 by kbar row; outputs block numbers
// [B, Sq, top_k] and route rows [B, Sq, 4 top_k + 4] (either may be null).
constexpr int kSelD = 128;
struct SelectProblem {
    const uint16_t *q, *kbar;
    const int32_t *doc_start, *blk_base;
    float *scores;
    int32_t *blocks, *routes;
    int64_t B, Sq, NB, q_offset;
    int32_t H, top_k;
    float scale;
};

hipError_t launch_select_fill(const SelectProblem &a, hipStream_t s);
hipError_t launch_select_scores(const SelectProblem &a, hipStream_t s);
hipError_t launch_select_topk(const SelectProblem &a, hipStream_t s);

#if defined(__HIPCC__)
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two FP32 values to packed bf16 in one instruction (gfx950's packed convert):
// round to nearest even, NaN stays NaN. `lo` lands in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.0f); }

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): a bf16 MFMA fed with
// both parts keeps about 16 mantissa bits of an FP32 operand.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// ---- buffer loads: out-of-range offsets read as zero, without a branch ----
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // >= every num_records used here

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                            0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---- LDS staging for operands that must be read transposed ----
// A staged block holds 16 rows x 256 bf16 columns. Element (row, d) lives at
// byte (d/4 >> 4) * kTrRegion + ((d/4) & 15) * 128 + row * 8 + (d % 4) * 2:
// four consecutive columns of one row are one 8-byte unit, and the 16 rows of
// a 4-column group are 128 contiguous bytes. One ds_read_tr16_b64 per 16
// columns x 4 rows then reads 512 contiguous bytes, and a lane's 16-byte
// chunk of a row is written with two 8-byte stores whose four column regions
// are 2176 bytes apart (a 128-byte bank shift between neighbouring regions).
constexpr int kTrRegion = 2176;
constexpr int kTrBlock = 4 * kTrRegion;  // 8704 bytes per 16-row block

__device__ __forceinline__ int tr_offset(int row, int d4)
{
    return (d4 >> 4) * kTrRegion + (d4 & 15) * 128 + row * 8;
}

// Store 8 consecutive columns d0 .. d0+7 (d0 % 8 == 0) of `row`.
__device__ __forceinline__ void tr_store8(char *blk, int row, int d0, uint4 v)
{
    *reinterpret_cast<uint2 *>(blk + tr_offset(row, d0 >> 2)) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2 *>(blk + tr_offset(row, (d0 >> 2) + 1)) = make_uint2(v.z, v.w);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposed read. Within each 16-lane group, lane i names the 8-byte unit
// R_i; lane j receives R_{j/4 + 4v}[j % 4] for v = 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const char *p)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                         (lds_bf16x4 *)(const_cast<char *>(p))));
}

// For the A/B operand of a 16x16x32 MFMA over the 16 x 256 staged block: lane
// (col = l % 16, quad = l / 16) gets rows 4*quad .. 4*quad+3 of column
// 16*db + col. lane_tr_base() is the lane's part of the address.
__device__ __forceinline__ int lane_tr_base(int col, int quad)
{
    return tr_offset(4 * quad + (col >> 2), col & 3);
}
__device__ __forceinline__ int tile_tr_offset(int db)
{
    return tr_offset(0, 4 * db);
}

// ---- gathered rows staged in LDS by direct-to-LDS buffer loads ----
// One dma16() moves 64 lanes x 16 bytes; lane l's bytes land at lds + 16 l.
// A gather instruction therefore covers two 512-byte rows: every group of
// consecutive lanes reads consecutive memory, which the vector memory path
// serves far faster than a lane-per-row pattern.
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ void dma16(rsrc_t r, lds_char *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}

// The same with an immediate byte offset IMM added to every lane's memory
// offset. The instruction adds its immediate to the LDS address too, so the
// LDS base passed down is lds - IMM: the 64 x 16 bytes still land at lds.
template <int IMM>
__device__ __forceinline__ void dma16_imm(rsrc_t r, lds_char *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds - IMM, 16, off, 0, IMM, 0);
}

// Column-sliced staging of 32 gathered rows of 512 bytes (16 KB): gather
// instruction s (0..15) loads the 32-byte column slice s of every row, lane l
// taking row (l & 31) ^ (8 (l >> 5)) and half l >> 5 of the slice. Each lane
// therefore serves one row for all 16 instructions and addresses them with
// one register plus an immediate. Byte (row r, 16-byte chunk c) sits at
// (c >> 1) * 1024 + (c & 1) * 512 + (r ^ 8 (c & 1)) * 16: 16 lanes reading
// one chunk of 16 consecutive rows, and 32 lanes reading 8-byte units of 8
// consecutive rows in both halves of a slice, touch distinct banks.
__device__ __forceinline__ int colslice_row(int lane) { return (lane & 31) ^ ((lane >> 5) << 3); }
__device__ __forceinline__ int colslice(int row, int chunk)
{
    return (chunk >> 1) * 1024 + (chunk & 1) * 512 + ((row ^ ((chunk & 1) << 3)) << 4);
}

// Row j of a staged region occupies bytes [512 j, 512 j + 512); its 16-byte
// chunk c (elements 8c .. 8c+7) sits at slot c ^ swz_mask(j), with the mask
// 2 (j mod 8): 8 consecutive rows put one chunk in 8 distinct 32-byte bank
// groups, for the 16-byte row reads and for the transposed read of 32-byte
// column pairs alike. Measured on gfx950 with the operand read patterns of
// these kernels, this runs the 16-byte reads at the rate of a contiguous read
// (about 500 B/ns per CU); a mask that also flips the low chunk bit for rows
// 8..15 halves it.
__device__ __forceinline__ int swz_mask(int row)
{
    return (row & 7) << 1;
}
__device__ __forceinline__ int swz(int row, int chunk)
{
    return row * 512 + ((chunk ^ swz_mask(row)) << 4);
}

// Lane l of gather instruction s stages row 2s + (l >> 5) at LDS slot l & 31;
// the chunk it fetches so that the region holds the swizzled layout.
__device__ __forceinline__ int dma_chunk(int lane, int s)
{
    return (lane & 31) ^ swz_mask(2 * s + (lane >> 5));
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ uint4 lds_read16(const lds_char *p)
{
    return __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4 *>(p));
}

__device__ __forceinline__ uint2 lds_read_tr(const lds_char *p)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                         (lds_bf16x4 *)(const_cast<lds_char *>(p))));
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr(const lds_char *p)
{
    return (uint32_t)(uintptr_t)p;
}

// LDS reads written in inline assembly. The compiler makes every LDS read it
// emits wait for all direct-to-LDS loads the wave has in flight, which would
// cap the gather pipeline at one chunk; these blocks are invisible to that
// rule, and the counted waits at the call sites order them after the loads
// they depend on. Each block ends with its own lgkmcnt(0), so all outputs are
// written when it ends, and the outputs are early-clobber, so no read can
// land in a register that a later read of the block still uses as address.
// OFF is an immediate byte offset added to every address.
template <int OFF>
__device__ __forceinline__ void lds_read16_x8(u32x4 (&d)[8], const uint32_t (&a)[8])
{
    asm volatile(
        "ds_read_b128 %0, %8 offset:%c16\n"
        "ds_read_b128 %1, %9 offset:%c16\n"
        "ds_read_b128 %2, %10 offset:%c16\n"
        "ds_read_b128 %3, %11 offset:%c16\n"
        "ds_read_b128 %4, %12 offset:%c16\n"
        "ds_read_b128 %5, %13 offset:%c16\n"
        "ds_read_b128 %6, %14 offset:%c16\n"
        "ds_read_b128 %7, %15 offset:%c16\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]),
          "=&v"(d[6]), "=&v"(d[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "n"(OFF)
        : "memory");
}

template <int OFF>
__device__ __forceinline__ void lds_read_tr_x8(u32x2 (&d)[8], const uint32_t (&a)[8])
{
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%c16\n"
        "ds_read_b64_tr_b16 %1, %9 offset:%c16\n"
        "ds_read_b64_tr_b16 %2, %10 offset:%c16\n"
        "ds_read_b64_tr_b16 %3, %11 offset:%c16\n"
        "ds_read_b64_tr_b16 %4, %12 offset:%c16\n"
        "ds_read_b64_tr_b16 %5, %13 offset:%c16\n"
        "ds_read_b64_tr_b16 %6, %14 offset:%c16\n"
        "ds_read_b64_tr_b16 %7, %15 offset:%c16\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]),
          "=&v"(d[6]), "=&v"(d[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "n"(OFF)
        : "memory");
}

// Explicit waits for direct-to-LDS loads, which produce no register the
// compiler could track. The s_waitcnt immediate of this architecture holds
// vmcnt in bits 3..0 and 15..14, expcnt in 6..4 and lgkmcnt in 11..8; a
// field at its maximum does not wait. QSA_WAIT_VM(n): at most n vector memory
// operations stay in flight. QSA_WAIT_LDS(): every LDS operation has finished.
#define QSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
#define QSA_WAIT_LDS() __builtin_amdgcn_s_waitcnt(0xC07F)

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8). Map them so that every XCD works on one contiguous range of logical
// blocks: neighbouring rows or key groups then share that XCD's L2.
// Direct-to-LDS loads written in assembly. The compiler tracks its own
// direct-to-LDS loads, and when it reuses one of their address registers
// while the load is in flight it waits for every load of the wave, which
// drains a staging pipeline. These blocks carry their own M0 set-up (the
// kernels that use them keep nothing else in M0, so the clobber loses
// nothing); their callers order the LDS reads after them with counted waits
// and a work-group barrier. Descriptor words: 48-bit base, stride 0,
// num_records, raw 32-bit data format.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// 64 lanes x 16 bytes: lane l's bytes land at LDS address lds + 16 l.
__device__ __forceinline__ void dma16_asm(i32x4 r, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// 4 bytes per active lane: lane l's word lands at LDS address lds + 4 l.
__device__ __forceinline__ void dma4_asm(i32x4 r, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n s_nop 0\n buffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// An address that the compiler cannot know before this point: LDS reads made
// through it stay after the barrier that precedes it.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x)
{
    asm volatile("" : "+s"(x) : : "memory");
    return x;
}

// The compiler takes x as rewritten here, so arithmetic that reads it stays
// after this point and after the volatile asm before it (a wait, the issue of
// direct-to-LDS loads) instead of being interleaved with the reads that
// produced it.
__device__ __forceinline__ void hold_after(uint4 &x)
{
    u32x4 v = __builtin_bit_cast(u32x4, x);
    asm volatile("" : "+v"(v));
    x = __builtin_bit_cast(uint4, v);
}

// The same dispatch, for work whose cost varies along the logical range (the
// full tiles of causal documents grow towards each document's end): groups of
// `unit` consecutive logical blocks stay on one XCD (they share their operands
// in its L2) and consecutive groups go to consecutive XCDs, so every XCD takes
// its share of the heavy and the light parts. The grid must be a multiple of
// 8 * unit blocks; the logical blocks past the work are to be skipped.
__device__ __forceinline__ int64_t xcd_group_block(int64_t b, int64_t unit)
{
    const int64_t x = b & 7, y = b >> 3;
    return ((y / unit) * 8 + x) * unit + (y % unit);
}

__device__ __forceinline__ int64_t xcd_logical_block(int64_t b, int64_t n)
{
    const int64_t x = b & 7, y = b >> 3;
    const int64_t per = n >> 3, rem = n & 7;
    return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + y;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
#endif

}  // namespace qsa
