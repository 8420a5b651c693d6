// rmsn_api.cpp -- host side of the RMSNorm C ABI: argument checks, the
// launch-configuration ladder, occupancy-sized grids and kernel launches.
//
// Every check runs before the first HIP call, so invalid arguments are
// reported without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <unordered_map>

#include "../../include/rmsnorm.h"
#include "rmsn_tables.h"

#ifndef RMSN_BUILD_INFO
#define RMSN_BUILD_INFO "unknown build"
#endif

namespace {

using rmsn::KernelEntry;

constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxVecLanes = 1024;

// bytes per activation element (x, y, dy, dx, res, h, dh); weights are fp32
// for RMSN_F32 and the *_WF32 formats, 16-bit otherwise
int elem_size(int dtype) { return dtype == RMSN_F32 ? 4 : 2; }
bool valid_dtype(int dtype) { return dtype >= RMSN_F32 && dtype <= RMSN_F16_WF32; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// bytes per weight element
int w_size(int dtype) { return (dtype == RMSN_BF16 || dtype == RMSN_F16) ? 2 : 4; }

// Common alignment in bytes (a power of two, capped at 16) of the activation
// pointers and of the weight pointer.
struct Align {
    int act;
    int w;
};

int low_align(uintptr_t bits) {
    int a = 1;
    while (a < 16 && (bits & uintptr_t(a)) == 0) a <<= 1;
    return a;
}

Align align_of(std::initializer_list<const void *> acts, const void *w) {
    uintptr_t bits = 0;
    for (const void *p : acts) bits |= reinterpret_cast<uintptr_t>(p);
    return {low_align(bits), low_align(reinterpret_cast<uintptr_t>(w))};
}

bool all16(const Align &a) { return a.act >= 16 && a.w >= 16; }

// Every element access is naturally aligned (required of every pointer).
bool natural(const Align &a, int dtype) { return a.act >= elem_size(dtype) && a.w >= w_size(dtype); }

// Elements per access of the element kernels: the largest power of two G with
// at most 16 bytes per access of activations and weights, N % G == 0 (no row
// ends inside a group) and every pointer aligned to its G-element access.
int elem_group(int64_t N, int dtype, const Align &a) {
    const int s = elem_size(dtype), sw = w_size(dtype), big = s > sw ? s : sw;
    int g = 1;
    while (2 * g * big <= 16 && N % (2 * g) == 0 && a.act % (2 * g * s) == 0 && a.w % (2 * g * sw) == 0) g *= 2;
    return g;
}

bool elem_group_ok(int64_t N, int dtype, const Align &a, int64_t g) {
    const int s = elem_size(dtype), sw = w_size(dtype), big = s > sw ? s : sw;
    return (g == 1 || g == 2 || g == 4 || g == 8) && g * big <= 16 && N % g == 0 && a.act % (g * s) == 0 &&
           a.w % (g * sw) == 0;
}

int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

int check_shape(int64_t M, int64_t N, int dtype) {
    if (!valid_dtype(dtype)) return RMSN_EDTYPE;
    if (M < 0 || N < 1 || N > kMaxN) return RMSN_EINVAL;
    if (M > INT64_MAX / N / 4) return RMSN_EINVAL;  // element and byte counts fit in int64
    return RMSN_OK;
}

// The row-width ladder: which kernel shape serves a row of N elements, and
// how many workgroups run it. Measured on MI355X over the synthetic workloads
// (widths 128 to 32768, bf16 and fp32), the rules below were the fastest or
// within noise of it.
//   Forward: lanes per row chosen so each lane holds at most 4 16-byte
//     vectors (rows of at most 32 vectors: one lane per vector, several rows
//     per wavefront, e.g. QK-norm's 128 bf16 = 16 lanes, 4 rows per wave);
//     one row block per workgroup (grid = row blocks), so the hardware
//     dispatcher balances the tail; mid-size inputs of the plain call take a
//     prefetching grid of three per compute unit instead (see ladder_grid;
//     one 1024-lane workgroup per CU where each would walk exactly two
//     blocks, see fwd_mid_wide), as do 64-lane rows of one or two vectors a
//     little beyond that range on 512-lane workgroups (fwd_rows64_512); rows
//     narrower than a wavefront from 9 to 24 blocks per CU take four per CU,
//     rows of exactly 64 vectors further out 16 rows per 1024-lane
//     workgroup, and 16-bit rows of 8192 columns over 32768 rows or more one
//     row per 1024-lane workgroup, two rows walked per workgroup (see
//     fwd_row_walk).
//   Backward: one vector per lane up to 1024 lanes per row (more lanes, fewer
//     registers, more rows in flight); workgroups of 1024 lanes for rows of
//     64 to 256 lanes (4 to 16 rows per pass), of the row itself otherwise
//     (256 lanes at least); a persistent grid of about two workgroups per
//     compute unit (three for rows of under a wavefront), fewer when the fp32
//     dW partial rows (written and read once) would exceed 1/6 of the
//     algorithmic bytes, never fewer than one per compute unit. The next row
//     block is prefetched below 1024 lanes per row; at 1024 lanes (one or
//     two vectors per lane) only when each workgroup walks at most 16 rows:
//     over longer walks the second buffer costs more occupancy than it
//     hides. Rows of 512 or 1024 well-filled lanes instead prefetch two
//     blocks with one workgroup per compute unit (see deep_prefetch). Some
//     16-bit rows of 257 to 1023 vectors run on whole wavefronts rather than
//     the next power of two (see rowwg_lanes). Measured over 39 shapes (M 1024..1M, N 128..32768) against the
//     earlier rules (workgroup = row, 5% partial cap, no prefetch at 1024
//     lanes): 5% faster by geometric mean, up to 21% at mid-size M, within
//     1% at 16384 x 4096. Rows of more than 1024 vectors: 16-bit
//     activations take the wide-row kernel (dW sums in LDS, 2 to 4 vectors
//     per lane, prefetching when the weights are 16-bit too: 5-16% faster
//     than keeping the sums in registers at 16384 to 32768 columns); fp32
//     rows keep the register kernel up to 4 vectors per lane (as fast) and
//     take the wide kernel from 5 to 8 (the register kernel spills there). One
//     wide workgroup per compute unit (its LDS allows no more at 4 vectors).
//   Rows the vector kernels cannot take because N*elem is not a multiple of
//     16 bytes or a pointer is not 16-byte aligned go to the element kernels
//     from 257 to 16384 columns (see ladder_shape).
//   Wider rows: the plain forward holds up to 16 vectors per lane on 1024
//     lanes (16384 vectors: 131072 16-bit or 65536 fp32 columns; the fused
//     residual forward up to 8); wider forward rows take the two-pass kernel
//     (the row read twice, the second time from cache), of any width. The
//     backward splits rows of more than
//     1024 * 4 16-bit or 1024 * 8 fp32 vectors over K = 2..16 workgroups of
//     1024 lanes (the split-row kernel: each member's dW sums for its slice
//     in LDS, the row sum exchanged through the workspace). 16-bit rows:
//     K is the fewest whose slices hold 2 vectors per lane, two members per
//     CU, while that is at most 16; wider rows, and fp32 rows, take the
//     fewest of one per CU (up to 4 or 8 vectors per lane). No prefetch: at
//     two per CU it spills, and at one per CU it measured 2% slower (bf16
//     4096 x 65536). Measured (graph-timed, rotating inputs) two per CU
//     against one: bf16 4096 x 65536 311.8 -> 293.9 us, 2048 x 131072 340.8
//     -> 317.8, 1024 x 262144 373.5 -> 378.4 (the one loss), bf16 with fp32
//     weights 8192 x 49152 646.7 -> 492.8; fp32 rows lose at two per CU (3
//     vectors per lane: 4096 x 65536 581.3 -> 641.7 us, 4096 x 36864 308.8
//     -> 330.0). At 32768 16-bit columns the wide kernel stays (148.3 us
//     against 155.4 split over two). Anything wider goes to the scalar
//     kernel.
constexpr int kWidePath = 2;  // rmsnorm_config::vector_path of the wide-row backward kernels
constexpr int kSplitPath = 4;  // rmsnorm_config::vector_path of the split-row backward kernels
constexpr int kFwdXWideVecs = 16;  // vectors per lane of the widest plain forward rows
constexpr int kLoopPath = 5;  // rmsnorm_config::vector_path of the forward's two-pass kernels
// vectors per lane the two-pass kernels with copy_mode 1 hold in LDS (128 KiB)
constexpr int kLoopLdsVecs = 8;
// The two-pass kernel's shape the ladder picks, by format, residual add and
// v = vectors per lane of the row: the chunk, the vectors kept in registers
// between the passes (the most each format keeps without spilling at one
// workgroup per CU) and whether the next kLoopLdsVecs are held in LDS.
// Holding pays where much of the row would be read again; a remainder of up
// to about 4-6 vectors per lane is cheaper to read again from the cache.
// Graph-timed, rotating inputs, us (every shape's outputs bit-identical):
//   16-bit:   v = 20: (4, 16) 225.6, (4, 12) + LDS 232.0; v = 22: 267.0 and
//             257.3; v = 24 (bf16 2048 x 196608): 288.1 and 272.2; v = 32
//             (1024 x 262144): (4, 16) 225.0, (2, 16) + LDS 193.6, (4, 12) +
//             LDS 218.0; 4096 x 262144: 901.4 and 794.1.
//   fp32:     v = 18: (2, 14) 228.0, + LDS 239.8; v = 20: 252.2 and 257.6;
//             v = 24: 313.8 and 297.4; v = 32: 424.6 and 396.3.
//   16-bit with fp32 weights: v = 18: (2, 14) 235.8, (2, 10) + LDS 244.7;
//             v = 20: 246.8 and 245.7; v = 32: 229.9 and 221.5.
//   residual, 16-bit: v <= 12 keeps the whole row at (4, 12); v = 16 (2, 16)
//             407.6 (whole row); v = 20: 503.6 against (4, 12) + LDS 473.0;
//             v = 28: 777.4 and 675.5; v = 32: 462.8 and 430.4.
//   residual, fp32: v = 18: (2, 12) 459.7, + LDS 484.9; v = 20: 503.4 and
//             515.7; v = 32: 502.9 and 461.5.
//   residual, fp32 weights: (4, 8) + LDS 381.2 against 420.4 without (v =
//             16), 587.8 against 637.4 (v = 24), ties at v = 12 and 32.
// Against the earlier choice of chunks of 4 with nothing kept, at two
// workgroups per CU: bf16 1024 x 262144 242.2 us, 4096 x 262144 952.2, 2048 x
// 196608 352.3; fp32 2048 x 131072 501.1; residual bf16 1024 x 262144 524.3.
void loop_choice(int dtype, int res, int64_t nvec, int *ch, int *kv, int *lds) {
    const bool w32 = dtype == RMSN_BF16_WF32 || dtype == RMSN_F16_WF32;
    const int64_t v = (nvec + kMaxVecLanes - 1) / kMaxVecLanes;
    auto pick = [&](int c, int k, int l) {
        *ch = c;
        *kv = k;
        *lds = l;
    };
    if (!res) {
        if (w32)
            v <= 20 ? pick(2, 14, 0) : pick(2, 10, 1);
        else if (dtype == RMSN_F32)
            v <= 20 ? pick(2, 14, 0) : pick(2, 14, 1);
        else
            v <= 20 ? pick(4, 16, 0) : v <= 28 ? pick(4, 12, 1) : pick(2, 16, 1);
    } else if (w32) {
        pick(4, 8, 1);
    } else if (dtype == RMSN_F32) {
        v <= 20 ? pick(2, 12, 0) : pick(2, 12, 1);
    } else {
        v <= 12 ? pick(4, 12, 0) : v <= 16 ? pick(2, 16, 0) : pick(4, 12, 1);
    }
}

constexpr int kCopyLds = 1;   // rmsnorm_config::copy_mode of the LDS-staged kernels (backward rings, two-pass forward)
constexpr int kMaxLdsStages = 8;
constexpr int kLdsStages = 2;  // LDS stages the ladder picks
constexpr int kElemPath = 3;  // rmsnorm_config::vector_path of the element kernels
constexpr int64_t kElemFwdMaxBytes = 32;  // forward element rows: bytes of row per lane (elem_lanes)
constexpr int64_t kElemBwdMaxElems = 12, kElemBwdMaxBytes = 40;  // backward: elements and bytes per lane
constexpr int kFwdMaxVecs = 4;
constexpr int64_t kFwdExactVecs = 5;  // forward rows that split exactly into this many vectors per lane take it
// forward row blocks per CU (inclusive range) taking a prefetching grid of kFwdMidPerCU workgroups per CU
constexpr int64_t kFwdMidLo = 4, kFwdMidHi = 8, kFwdMidPerCU = 3;
constexpr int64_t kFwdWidePerCU = 2;     // resident forward workgroups per CU with fp32 weights
constexpr int64_t kFwdWideMinLanes = 128;  // ... for rows of at least this many lanes
// plain forward rows of 1024 16-bit vectors over at least kFwdLongRows rows
// walk kFwdLongWalk rows per 1024-lane workgroup (fwd_row_walk)
constexpr int64_t kFwdLongRows = 32768, kFwdLongWalk = 2;
// plain forward rows of exactly 64 vectors beyond this many 256-lane row blocks
// per CU run 16 rows per 1024-lane workgroup
constexpr int64_t kFwdRows64MinBlocks = 16;
// plain forward 64-lane rows of one (two) vectors up to this many 256-lane row
// blocks per CU, beyond the mid-size range, run 512-lane workgroups (fwd_rows64_512)
constexpr int64_t kFwd512MaxBlocks1 = 20, kFwd512MaxBlocks2 = 16;
// plain forward rows narrower than a wavefront, beyond the mid-size range up to this
// many row blocks per CU: a prefetching grid of kFwdNarrowPerCU per CU
constexpr int64_t kFwdNarrowMaxBlocks = 24, kFwdNarrowPerCU = 4;
constexpr int kBwdGroupLanes = 1024;  // backward workgroup for rows of 64 to 256 lanes
constexpr int64_t kPartialShare = 6;  // partial-row traffic at most 1/kPartialShare of the bytes
constexpr int64_t kShortWalk = 16;    // rows per workgroup up to which 1024-lane rows prefetch
constexpr int64_t kBwdSingleElems = 16384, kBwdSinglePasses = 4;  // backward inputs one workgroup walks
constexpr int64_t kStreamMinBytes = int64_t(4) << 20;  // forward inputs from this size stream (one XCD's L2)
constexpr int kBwdMaxVecs = 4;
constexpr int64_t kRowWGMinVecs = 256;  // backward rows wider than this may run on whole wavefronts (rowwg_lanes)
constexpr int64_t kMaxGrid = int64_t(1) << 20;

void set_vector_shape(int64_t lpr, int64_t vpt, int wg, int pf, rmsnorm_config *c) {
    c->vector_path = 1;
    c->lanes_per_row = (int32_t)lpr;
    c->vecs_per_lane = (int32_t)vpt;
    c->wg_threads = wg > 0 ? wg : rmsn::wg_for_lpr((int)lpr);
    c->rows_per_wg = c->wg_threads / c->lanes_per_row;
    c->prefetch = pf;
}

// Element kernels: one row per workgroup of `lanes` lanes, g elements per
// access, k = ceil(N / (g * lanes)) accesses per lane. A one-row register
// prefetch measured no faster (bf16 and fp32, 1500 to 15000 columns, one
// element per access) and, in the backward, costs the second workgroup per CU
// from 5 elements per lane, so there is none.
void set_elem_shape(int64_t N, int g, int lanes, rmsnorm_config *c) {
    c->vector_path = kElemPath;
    c->lanes_per_row = lanes;
    c->vecs_per_lane = (int32_t)((N + int64_t(g) * lanes - 1) / (int64_t(g) * lanes));
    c->elems_per_access = g;
    c->wg_threads = lanes;
    c->rows_per_wg = 1;
    c->prefetch = 0;
}

bool elem_lanes_ok(int64_t lanes) {
    return lanes >= rmsn::kElemMinLanes && lanes <= rmsn::kElemMaxLanes && (lanes & (lanes - 1)) == 0;
}

// Lanes of an element row: the fewest (a power of two from 64) that keep each
// lane's share of the row within a budget, so that short rows do not leave
// most of a 1024-lane workgroup idle and a compute unit holds more rows. The
// forward budget is 32 bytes of row per lane; the backward's, which also holds
// dy and the dW sums, 12 elements and 40 bytes. Measured at 16384 rows against
// every lane count, graph-timed: the forward rule picked the fastest at every
// row (bf16 300 columns 29.4 -> 7.9 us with 64 lanes, 1500 43.5 -> 21.2 with
// 128, 2050 45.9 -> 26.9 with 256, 4100 58.4 -> 52.5 with 512); the backward
// rule the fastest or within 1-3% everywhere but bf16 1500 (128 lanes 40.0
// us, 256 lanes 37.5): 300 38.2 -> 16.7 us, 700 45.0 -> 22.1, 4100 82.4 ->
// 77.6, fp32 4098 158.4 -> 155.1.
int elem_lanes(int64_t N, int g, int dtype, int is_bwd) {
    const int64_t es = elem_size(dtype);
    const int64_t max_elems = is_bwd ? kElemBwdMaxElems : rmsn::kElemMaxK;
    const int64_t max_bytes = is_bwd ? kElemBwdMaxBytes : kElemFwdMaxBytes;
    for (int64_t lanes = rmsn::kElemMinLanes; lanes < rmsn::kElemMaxLanes; lanes *= 2) {
        const int64_t per_lane = (N + g * lanes - 1) / (g * lanes) * g;
        if (per_lane <= max_elems && per_lane * es <= max_bytes) return (int)lanes;
    }
    return rmsn::kElemMaxLanes;
}

bool elem_ok(int64_t N) { return N <= int64_t(rmsn::kElemMaxLanes) * rmsn::kElemMaxK; }

void set_scalar_shape(rmsnorm_config *c) {
    c->vector_path = 0;
    c->lanes_per_row = rmsn::kScalarWG;
    c->vecs_per_lane = 0;
    c->wg_threads = rmsn::kScalarWG;
    c->rows_per_wg = 1;
    c->prefetch = 0;
}

bool vector_ok(int64_t N, int dtype, const Align &a) { return all16(a) && (N * elem_size(dtype)) % 16 == 0; }

// A backward row on whole wavefronts whose count is not a power of two runs
// on the kernels whose row is the whole workgroup (its size set at launch).
bool row_is_wg(const rmsnorm_config &c) {
    const int64_t l = c.lanes_per_row;
    return c.vector_path == 1 && c.vecs_per_lane == 1 && l > 64 && l <= kMaxVecLanes && l % 64 == 0 &&
           (l & (l - 1)) != 0 && c.wg_threads == l;
}

// Largest vectors per lane of the wide-row backward kernels: their dW sums
// (vectors x 1024 lanes x elements per vector, fp32) fill at most 128 KiB.
int64_t wide_max_vecs(int dtype) { return dtype == RMSN_F32 ? 8 : 4; }

// Lanes of a backward row on whole wavefronts (not a power of two), or 0
// where the power-of-two row is kept. Measured on MI355X (bf16, M 4096 to
// 65536, graph-timed, inputs not cache-resident) against the power-of-two
// rows at their best prefetch depth and grid:
//   320-384 lanes (2560-3072 columns): depth 2, two per CU, 4-12% faster;
//   448 lanes: the 512-lane row is as fast or faster (kept);
//   576-640 lanes: depth 2, one per CU, 7-8% faster when each workgroup walks
//     at most kShortWalk rows; over longer walks the 1024-lane row without
//     prefetch is within 2% either way (kept);
//   704-768 lanes (6144 columns): depth 2, one per CU, 2-8% faster;
//   832-960 lanes: the 1024-lane row is 1-4% faster (kept).
// fp32 activations or weights measured as ties and keep the power-of-two row.
int64_t rowwg_lanes(int64_t M, int64_t nvec, int dtype, int64_t cus) {
    if ((dtype != RMSN_BF16 && dtype != RMSN_F16) || nvec <= kRowWGMinVecs || nvec >= kMaxVecLanes) return 0;
    const int64_t lanes = (nvec + 63) / 64 * 64;
    if ((lanes & (lanes - 1)) == 0) return 0;
    if (lanes <= 384) return lanes;
    if (lanes > 512 && lanes <= 768 && (lanes > 640 || M <= kShortWalk * cus)) return lanes;
    return 0;
}

// Forward two-pass rows: one row per 1024-lane workgroup, `ch` vectors per
// lane per chunk, `kv` of them kept in registers and, with `lds`, the next
// kLoopLdsVecs held in LDS (copy_mode 1; rmsn_fwd_loop.h).
void set_loop_shape(int ch, int kv, int lds, rmsnorm_config *c) {
    set_vector_shape(kMaxVecLanes, ch, rmsn::kWideLanes, 0, c);
    c->vector_path = kLoopPath;
    c->kept_vecs = kv;
    c->copy_mode = lds ? kCopyLds : 0;
}

// Split rows of two workgroups per CU: vectors per lane of the slices (their
// dW sums fill at most 64 KiB of LDS and the kernel 64 VGPRs); 16-bit
// activations only (fp32 rows measured faster on fewer, wider members).
constexpr int64_t kSplitTwoVecs = 2;

// Split-row backward: K workgroups of 1024 lanes per row, `vpt` vectors per
// lane of each member's slice (rmsn_bwd_split.h). The grid is set by
// ladder_grid (groups of K).
void set_split_shape(int64_t K, int64_t vpt, int pf, rmsnorm_config *c) {
    set_vector_shape(K * rmsn::kWideLanes, vpt, rmsn::kWideLanes, pf, c);
    c->vector_path = kSplitPath;
    c->rows_per_wg = 1;
}

int64_t split_members(const rmsnorm_config &c) {
    return c.vector_path == kSplitPath ? c.lanes_per_row / rmsn::kWideLanes : 1;
}

// Plain forward rows of exactly 1024 16-bit vectors (8192 columns, 16-bit
// weights) over many rows: one row per 1024-lane workgroup, each walking
// kFwdLongWalk rows with the next row's loads issued before the current
// row's arithmetic, instead of a row per 256-lane workgroup at 4 vectors per
// lane. Graph-timed, rotating inputs, three buffer placements each (us):
// bf16 32768 x 8192 176.9-178.4 -> 175.0-175.5, 65536 x 8192 362.0-373.4 ->
// 349.5-351.3, 131072 x 8192 752.3-785.4 -> 700.2-706.2; fp16 32768 x 8192
// 176.7-178.7 -> 175.7-176.2. At 24576 rows a tie (-0.2..-0.5%), at 16384
// 2.5% slower, so from kFwdLongRows. Walks of 3 or 4 rows were slower than 2
// (131072 x 8192: -8.1% and -5.5% against -9.6%); two rows of 512 lanes x 2
// per workgroup won at 32768-49152 rows and lost at 131072 (+4.5%); rows of
// 512 or 2048 vectors gained nothing consistent.
bool fwd_row_walk(int64_t M, int64_t nvec, int dtype, int res) {
    return !res && nvec == kMaxVecLanes && elem_size(dtype) == 2 && w_size(dtype) == 2 && M >= kFwdLongRows;
}

void ladder_shape(int64_t M, int64_t N, int dtype, int is_bwd, int res, const Align &a, int64_t cus,
                  rmsnorm_config *c) {
    const int64_t nvec = N * elem_size(dtype) / 16;
    // the forward holds very wide rows at up to 16 vectors per lane (8 with the residual add)
    const int64_t vmax = is_bwd ? wide_max_vecs(dtype) : res ? 2 * kFwdMaxVecs : kFwdXWideVecs;
    if (!vector_ok(N, dtype, a)) {
        // rows that are not a multiple of 16 bytes or not 16-byte aligned:
        // the element kernels (the row read once into registers) from 257
        // to 16384 columns, else the scalar kernel. At 16384 rows, against
        // the scalar kernel: bf16 4100 columns (4 elements per access) 130
        // -> 60 us forward and 459 -> 83 backward; bf16 4095 (one per
        // access) 129 -> 62 and 463 -> 79; fp32 4098 (two per access) 177
        // -> 102 and 491 -> 156 (see ladder_grid for the forward's grid).
        if (elem_ok(N)) {
            const int g = elem_group(N, dtype, a);
            set_elem_shape(N, g, elem_lanes(N, g, dtype, is_bwd), c);
        } else {
            set_scalar_shape(c);
        }
        return;
    }
    if (!is_bwd && nvec > kMaxVecLanes * vmax) {
        // the two-pass kernel addresses a row with 32-bit byte offsets (a 4
        // GiB fp32 row of 2^30 columns does not fit: the scalar kernel)
        if (nvec * 16 > (int64_t)UINT32_MAX) {
            set_scalar_shape(c);
        } else {
            int ch = 0, kv = 0, lds = 0;
            loop_choice(dtype, res, nvec, &ch, &kv, &lds);
            set_loop_shape(ch, kv, lds, c);
        }
        return;
    }
    if (nvec > kMaxVecLanes * vmax) {
        // backward: 16-bit activations, the fewest members of two per CU
        // (slices of 2 vectors per lane) up to kMaxSplit of them; else the
        // fewest of one per CU (up to 4 or 8 per lane, as the wide kernel)
        const int64_t K2 = (nvec + kMaxVecLanes * kSplitTwoVecs - 1) / (kMaxVecLanes * kSplitTwoVecs);
        const int64_t K1 = (nvec + kMaxVecLanes * vmax - 1) / (kMaxVecLanes * vmax);
        const int64_t K = dtype != RMSN_F32 && K2 <= rmsn::kMaxSplit ? K2 : K1;
        if (is_bwd && K <= rmsn::kMaxSplit) {
            const int64_t slice = (nvec + K - 1) / K;
            set_split_shape(K, (slice + kMaxVecLanes - 1) / kMaxVecLanes, 0, c);
        } else {
            set_scalar_shape(c);
        }
        return;
    }
    if (is_bwd && nvec > kMaxVecLanes && (dtype != RMSN_F32 || nvec > kMaxVecLanes * kBwdMaxVecs)) {
        const int64_t vpt = (nvec + kMaxVecLanes - 1) / kMaxVecLanes;
        const int pf = (dtype == RMSN_BF16 || dtype == RMSN_F16) ? 1 : 0;
        set_vector_shape(kMaxVecLanes, vpt, rmsn::kWideLanes, pf, c);
        c->vector_path = kWidePath;
        return;
    }
    int64_t lpr, vpt;
    if (nvec <= 32) {
        lpr = next_pow2(nvec);
    } else if (is_bwd) {
        lpr = nvec <= kMaxVecLanes ? next_pow2(nvec) : kMaxVecLanes;
        if (const int64_t l = rowwg_lanes(M, nvec, dtype, cus)) lpr = l;
    } else {
        lpr = next_pow2((nvec + kFwdMaxVecs - 1) / kFwdMaxVecs);
        if (lpr < 64) lpr = 64;
        if (lpr > kMaxVecLanes) lpr = kMaxVecLanes;
        // Rows of exactly 5 vectors on each of 128 or 256 lanes fill every
        // slot at 5 per lane, where the rule above leaves a fifth of them
        // idle at 3 per lane: bf16 16384 x 5120 56.0 -> 54.7 us, 32768 x 5120
        // 111.3 -> 108.2, 16384 x 10240 112.2 -> 110.8; fp32 16384 x 2560
        // 56.0 -> 54.3. At 512 lanes (20480 columns), at 64 (2560 bf16) and
        // at 7 per lane (896, 1792 vectors) it measured a tie (-0.7..+0.5%),
        // so only these.
        const int64_t l5 = nvec / kFwdExactVecs;
        if (nvec % kFwdExactVecs == 0 && l5 >= 128 && l5 <= 256 && (l5 & (l5 - 1)) == 0) lpr = l5;
    }
    vpt = (nvec + lpr - 1) / lpr;
    if (!is_bwd) {
        if (fwd_row_walk(M, nvec, dtype, res))
            set_vector_shape(kMaxVecLanes, 1, kMaxVecLanes, 1, c);
        else
            set_vector_shape(lpr, vpt, rmsn::wg_for_lpr((int)lpr), 0, c);
        return;
    }
    const int wg = (lpr >= 64 && lpr <= 256) ? kBwdGroupLanes : rmsn::wg_for_lpr((int)lpr);
    set_vector_shape(lpr, vpt, wg, lpr < kMaxVecLanes ? 1 : 0, c);
}

// Backward rows of 512 or 1024 lanes with one vector per lane and at least
// 3/4 of the lanes busy: two row blocks prefetched and one workgroup per
// compute unit (half the partial rows). Measured against two workgroups per
// CU with one block prefetched: 1.3-7.6% faster at 4096..65536 rows of
// 4096..8192 columns (16384 x 4096: 71.2 -> 69.3 us); at 5120 columns (5/8
// of 1024 lanes busy) 6.5% slower, hence the lane condition.
// Rows on whole wavefronts (row_is_wg) always prefetch two blocks: two
// workgroups per CU up to 384 lanes, one above (see rowwg_lanes).
// Returns the workgroups per compute unit of a depth-2 shape, 0 otherwise.
int deep_prefetch(int is_bwd, int64_t N, int dtype, const rmsnorm_config *c) {
    if (!is_bwd || c->vector_path != 1 || c->vecs_per_lane != 1) return 0;
    if (row_is_wg(*c)) return c->lanes_per_row <= 384 ? 2 : 1;
    const int64_t nvec = N * elem_size(dtype) / 16;
    return c->lanes_per_row >= 512 && 4 * nvec >= 3 * (int64_t)c->lanes_per_row ? 1 : 0;
}

// Wide rows (the wide-row kernel) with 16-bit activations and weights over
// walks of at least kWideLongWalk rows per compute unit: two workgroups per CU
// (past what stays resident at 3 or 4 vectors per lane, whose dW sums leave
// LDS for one: the second half of the grid then runs as the first drains),
// no prefetch at 2 or 3 vectors per lane. Measured (whole rmsnorm_bwd calls, graph-timed,
// rotating inputs; bf16): 16384 x 16384 286.1 -> 273.0 us, 32768 x 16384
// 577.6 -> 534.6, 32768 x 24576 844.0 -> 819.2, 16384 x 32768 593.2 -> 566.1,
// 32768 x 32768 1162.1 -> 1105.5; fp16 likewise. Shorter walks keep one
// prefetching workgroup per CU (1-2% faster there); fp32 activations or
// weights measured within 1.5% either way and keep it too.
constexpr int64_t kWideLongWalk = 64;

bool wide_long_walk(int64_t M, int dtype, int64_t cus, const rmsnorm_config *c) {
    return c->vector_path == kWidePath && (dtype == RMSN_BF16 || dtype == RMSN_F16) && M >= kWideLongWalk * cus;
}

// Backward prefetch depth. The deep shapes above: 2. Otherwise at 1024 lanes
// per row (one or two vectors per lane; the prefetching kernels with more
// vectors spill): 1 when each workgroup walks at most kShortWalk rows, else 0.
// Needs the grid, so it runs after ladder_grid.
// 16-bit rows of 64 or 128 lanes, several to a 1024-lane workgroup (plain
// call): no prefetch once each workgroup walks kNoPfMinBlocks row blocks or
// more, where the two resident workgroups per CU already keep enough loads in
// flight (bf16, graph-timed, against depth 1: 32768 x 512 22.4 -> 21.8 us,
// 65536 x 512 39.6 -> 37.4, 131072 x 512 75.8 -> 70.4, 16384 x 1024 23.2 ->
// 22.8, 65536 x 1024 71.6 -> 70.4, 131072 x 1024 141.5 -> 133.1; at a walk of
// 2 blocks depth 1 was 0.9% faster; fp32 rows measured within 0.6% and keep
// it).
constexpr int64_t kNoPfMinBlocks = 4;

void ladder_prefetch(int64_t M, int64_t N, int dtype, int is_bwd, int64_t cus, rmsnorm_config *c, int res = 0) {
    if (deep_prefetch(is_bwd, N, dtype, c))
        c->prefetch = 2;
    else if (is_bwd && c->vector_path == 1 && c->lanes_per_row == kMaxVecLanes && c->vecs_per_lane <= 2)
        c->prefetch = M <= kShortWalk * c->grid ? 1 : 0;
    else if (is_bwd && wide_long_walk(M, dtype, cus, c) && c->vecs_per_lane <= 3)
        c->prefetch = 0;
    else if (is_bwd && !res && c->vector_path == 1 && c->copy_mode == 0 && elem_size(dtype) == 2 &&
             c->wg_threads == kMaxVecLanes && c->vecs_per_lane == 1 && c->lanes_per_row >= 64 &&
             c->lanes_per_row <= 128 && c->grid > 0) {
        const int64_t blocks = (M + c->rows_per_wg - 1) / c->rows_per_wg;
        if ((blocks + c->grid - 1) / c->grid >= kNoPfMinBlocks) c->prefetch = 0;
    }
}

// Backward memory path. Rows of one vector per lane from 384 to 1024 vectors
// (at least 3/4 of 512 lanes busy) with each workgroup walking 8 to 64 rows
// take the LDS-staged kernel: the next two row blocks copied global->LDS
// (copy_mode 1, two stages), one workgroup per compute unit; rows of up to 512
// vectors on 512 lanes, wider ones on their whole wavefronts (16-bit
// activations) or on 1024 lanes (fp32 activations). Measured on MI355X against
// the register-ring rules above (whole rmsnorm_bwd calls, graph-timed, inputs
// rotating past the MALL; bf16 unless stated): 4096 x 4096 23.7 -> 22.6 us,
// 16384 x 4096 69.5 -> 68.6, 16384 x 5120 89.9 -> 83.3 (640 lanes), 8192 x
// 5120 51.9 -> 45.7, 16384 x 6144 104.8 -> 101.9, 16384 x 7168 121.8 -> 116.9
// (896 lanes), 4096 x 8192 41.0 -> 39.5, 16384 x 3072 59.0 -> 58.2; bf16 with
// fp32 weights 4096 x 5120 31.7 -> 27.2; fp32 4096 x 2560 28.0 -> 26.5,
// 16384 x 4096 133.5 -> 129.7. Deeper rings (3 to 8 stages) were never
// faster than two. Over longer walks the register ring wins (65536 x 4096:
// 264.6 against 278.3 us), as it does for walks of 1 to 4 rows (256 x 4096:
// 8.5 against 8.8 us) and for rows of 320 vectors (2560 bf16 columns); the
// residual-fused backward measured within noise either way and keeps it.
constexpr int64_t kLdsMinVecs = 384, kLdsMinWalk = 8, kLdsMaxWalk = 64;
// Rows of exactly 256 vectors (bf16 2048, fp32 1024 columns), four per
// 1024-lane workgroup, take the opposite turn: the LDS ring wins over long
// walks, from kLds256MinWalk rows per CU (two stages, one workgroup per CU,
// against the register ring's two per CU; bf16 32768 x 2048 71.2 -> 69.3 us,
// 65536 x 2048 139.7 -> 132.1, 131072 x 2048 280.6 -> 260.7, fp32 65536 x
// 1024 138.1 -> 131.1; at 64 rows per CU within 1.1% either way, at 32 1%
// slower).
constexpr int64_t kLds256MinWalk = 128;


void ladder_copy(int64_t M, int64_t N, int dtype, int is_bwd, int res, int64_t cus, rmsnorm_config *c) {
    if (!is_bwd || res || c->vector_path != 1 || cus < 1) return;
    const int64_t nvec = N * elem_size(dtype) / 16;
    if (nvec == 256 && M >= kLds256MinWalk * cus) {
        set_vector_shape(256, 1, kMaxVecLanes, kLdsStages, c);
        c->copy_mode = kCopyLds;
        c->grid = cus;
        c->partial_rows = c->grid;
        return;
    }
    if (nvec < kLdsMinVecs || nvec > kMaxVecLanes || M < kLdsMinWalk * cus || M > kLdsMaxWalk * cus) return;
    const int64_t lanes = nvec <= 512 ? 512 : dtype == RMSN_F32 ? kMaxVecLanes : (nvec + 63) / 64 * 64;
    set_vector_shape(lanes, 1, (int)lanes, kLdsStages, c);
    c->copy_mode = kCopyLds;
    c->grid = cus;
    c->partial_rows = c->grid;
}

// Grid. Forward: one row block per workgroup (capped at 2^20 workgroups,
// which then loop), except mid-size inputs of the plain call (res: the
// residual-fused kernel), which get a prefetching grid of three per CU, and
// the long walks of fwd_row_walk (half the rows).
// Backward (persistent, one partial dW row per workgroup): see the ladder
// comment; `blocks_per_cu` caps it at what stays resident.
// Mid-size plain forward inputs: 1024-lane workgroups (four 256-lane row
// blocks each), one per CU, each walking two with the second's loads issued
// first, instead of three prefetching 256-lane workgroups per CU. Taken where
// every workgroup walks exactly two blocks, and for 64-lane rows of one
// vector from more than 6 blocks of 256 lanes per CU. Graph-timed, rotating
// inputs, two buffer placements, us: walks of exactly two: bf16 8192 x 512
// 4.92-5.08 -> 4.16-4.20, 8192 x 1024 7.21 -> 6.62-6.66, 4096 x 3072 9.83 ->
// 8.70, 4096 x 4096 12.38-12.73 -> 11.10-11.18, 2048 x 6144 9.77-9.85 ->
// 8.78-8.84, 2048 x 8192 12.22 -> 11.46; fp32 8192 x 256 4.90 -> 4.00-4.06,
// 8192 x 512 7.15-7.24 -> 6.52, 4096 x 2048 12.13-12.21 -> 11.12-11.23, 2048
// x 4096 12.65 -> 11.33-11.44; fp16 8192 x 512 4.78-4.92 -> 4.16-4.19; bf16
// with fp32 weights 8192 x 512 4.85-4.92 -> 4.24. 64-lane rows of one vector
// with some walks of one: bf16 6400 x 512 4.60-4.66 -> 4.00-4.02, 7168 x 512
// 4.51 -> 3.98. Not taken: walks of one and two on wider rows (bf16 6656 x
// 1024 +5.5%, 3584 x 4096 -1.1%, 1792 x 8192 +1.9%; at 6 blocks per CU, half
// the workgroups walking one, +3-17%); 64-lane rows of more than two vectors
// (bf16 8192 x 2048 +10%, fp32 8192 x 1024 +15%); shapes whose 1024-lane
// kernel is not built for the format.
void fwd_mid_wide(int64_t M, int dtype, int64_t cus, rmsnorm_config *c, int64_t *grid) {
    if (c->lanes_per_row == 64 && c->vecs_per_lane > 2) return;
    const int64_t per = kMaxVecLanes / c->lanes_per_row;  // rows per 1024-lane workgroup
    const int64_t blocks = (M + per - 1) / per;
    const bool even = blocks == 2 * cus;
    const bool narrow = c->lanes_per_row == 64 && c->vecs_per_lane == 1 && 2 * blocks > 3 * cus && blocks <= 2 * cus;
    if (!even && !narrow) return;
    if (!rmsn::fwd_vec_kernel(dtype, 0, c->lanes_per_row, c->vecs_per_lane, (int)kMaxVecLanes, 1)) return;
    c->wg_threads = (int32_t)kMaxVecLanes;
    c->rows_per_wg = (int32_t)per;
    *grid = cus;
}

// 64-lane rows of one or two vectors just beyond the mid-size range: 512-lane
// workgroups (8 rows each), three per CU, each loading its next block ahead.
// Graph-timed, rotating inputs, two buffer placements, against one block per
// 256-lane workgroup (us; n blocks of 256 lanes per CU): bf16 x 512 at 10,
// 12, 14, 16: 5.46-5.49 -> 4.58-4.59, 6.40-6.43 -> 5.38-5.39, 7.31-7.36 ->
// 6.22-6.25, 7.81-7.82 -> 6.90-6.91; x 1024: 8.81-8.84 -> 7.87-7.91,
// 10.42-10.46 -> 9.58-9.64, 11.64-11.65 -> 10.92-10.99, 12.85-12.87 ->
// 12.01-12.05; fp32 x 256: -10% to -17%, x 512: -3% to -9%. One-vector rows
// at 18 and 20 against the 1024-lane grid of rows of 64 vectors: 5.6-7.7%
// faster; at 24 mixed (bf16 +1.2%, fp32 -4%). Two-vector rows from 18:
// within 1.4% either way. Rows of four vectors lose (bf16 8192 x 2048 +7%
// at two per CU). Only where the format has the kernel (bf16, fp32).
bool fwd_rows64_512(int dtype, int64_t cus, int64_t row_blocks, rmsnorm_config *c, int64_t *grid) {
    if (c->lanes_per_row != 64 || c->vecs_per_lane > 2 || c->wg_threads != 256) return false;
    const int64_t hi = c->vecs_per_lane == 1 ? kFwd512MaxBlocks1 : kFwd512MaxBlocks2;
    if (row_blocks <= kFwdMidHi * cus || row_blocks > hi * cus) return false;
    if (!rmsn::fwd_vec_kernel(dtype, 0, 64, c->vecs_per_lane, 512, 1)) return false;
    c->wg_threads = 512;
    c->rows_per_wg = 512 / 64;
    c->prefetch = 1;
    *grid = kFwdMidPerCU * cus;
    return true;
}

void ladder_grid(int64_t M, int64_t N, int dtype, int is_bwd, int res, int num_cus, int blocks_per_cu,
                 rmsnorm_config *c) {
    const int64_t row_blocks = (M + c->rows_per_wg - 1) / c->rows_per_wg;
    int64_t grid;
    if (!is_bwd) {
        grid = row_blocks < kMaxGrid ? row_blocks : kMaxGrid;
        // Mid-size inputs: 4 to 8 row blocks per compute unit of 256-lane
        // workgroups (e.g. 2048 x 4096 bf16) are dispatched nearly in one go,
        // and their time is the dispatch and the first loads. A grid of three
        // workgroups per CU, each loading its next block ahead (prefetch 1),
        // measured 3-18% faster for the plain forward in every format (2048 x
        // 4096 bf16: 7.8 -> 6.6 us; two buffer placements agree). At 2 blocks
        // per CU and from 16 up it was mixed or 1-3% slower; with the residual
        // add, mixed.
        const int64_t cus = num_cus > 0 ? num_cus : 1;
        if (!res && c->vector_path == 1 && c->lanes_per_row >= 64 && c->wg_threads <= 256 &&
            row_blocks >= kFwdMidLo * cus && row_blocks <= kFwdMidHi * cus) {
            grid = kFwdMidPerCU * cus;
            c->prefetch = 1;
            fwd_mid_wide(M, dtype, cus, c, &grid);
        }
        // non-temporal row loads for rows of a wavefront or more: measured with
        // inputs that are not cache-resident (the benchmark's regime), they are
        // 0-18% faster at every such shape; narrow rows lose 1.6% with them.
        // Inputs smaller than one XCD's L2 are likely still cache-resident (a
        // decode step's few rows): there they add latency (2.2 -> 2.5 us at
        // 1 x 4096), so they stay off.
        // 16-bit activations with fp32 weights: each one-block workgroup
        // re-reads the weights (twice the bytes of a 16-bit row) from cache.
        // A resident grid of two workgroups per CU keeps them in registers
        // over its rows (plain call, rows of 128 lanes or more, beyond the
        // mid-size range). bf16 weights fp32: 32768 x 8192 184 -> 175 us,
        // 8192 x 16384 92.9 -> 89.1, 4096 x 32768 93.6 -> 92.2, 16384 x 4096
        // 45.6 -> 44.6 (fp16 likewise). Narrower rows lose: 65536 x 2048
        // (64 lanes) 88.3 -> 89.5, 1M x 128 88 -> 129. With 16-bit weights
        // the same grid was 0-4% slower, and with the residual add 1-2%.
        if (!res && c->vector_path == 1 && elem_size(dtype) == 2 && w_size(dtype) == 4 &&
            c->lanes_per_row >= kFwdWideMinLanes && row_blocks > kFwdMidHi * cus) {
            int64_t resident = cus * (blocks_per_cu > 0 ? blocks_per_cu : 1);
            if (resident > kFwdWidePerCU * cus) resident = kFwdWidePerCU * cus;
            grid = row_blocks < resident ? row_blocks : resident;
            c->prefetch = 0;
        }
        if (!res && c->vector_path == 1) fwd_rows64_512(dtype, cus, row_blocks, c, &grid);
        // Rows narrower than a wavefront (one vector per lane, 8 to 32 lanes,
        // several rows per 256-lane workgroup) from 9 to 24 row blocks per CU:
        // four workgroups per CU, each loading its next block ahead. Graph-timed,
        // rotating inputs, two buffer placements, against one block per
        // workgroup: 4.5-10.5% faster at every one of 10, 12, 14, 16, 18, 20
        // and 24 blocks per CU for bf16 x 64, x 128, x 256 and fp32 x 64 (bf16
        // 65536 x 128 6.61-6.64 -> 6.18-6.21 us, 73728 x 128 7.45-7.50 ->
        // 6.71-6.72; fp32 73728 x 64 7.37-7.38 -> 6.65-6.66); at 32 and 64
        // blocks per CU within 2% either way, at 8 per CU 6-7% slower.
        // fp16 takes it unmeasured (the bf16 kernel with another conversion);
        // fp32 weights with 16-bit rows and the residual add keep their grids.
        if (!res && c->vector_path == 1 && c->lanes_per_row < 64 && c->wg_threads == 256 &&
            w_size(dtype) == elem_size(dtype) && row_blocks > kFwdMidHi * cus &&
            row_blocks <= kFwdNarrowMaxBlocks * cus) {
            grid = kFwdNarrowPerCU * cus;
            c->prefetch = 1;
        }
        // Rows of exactly 64 vectors (16-bit 512, fp32 256 columns) on 64 lanes,
        // beyond 16 row blocks of 256 lanes per CU: 16 rows per 1024-lane
        // workgroup, one block each. Graph-timed, rotating inputs, two buffer
        // placements, us: bf16 24576 x 512 10.88-10.95 -> 10.25-10.33, 32768 x
        // 512 13.97-14.01 -> 12.90-12.94, 65536 x 512 24.53-24.65 -> 23.91-23.99,
        // 131072 x 512 45.08-45.13 -> 44.38-44.51; fp32 32768 x 256 13.92 ->
        // 13.37-13.39, 65536 x 256 24.75 -> 23.98-24.15; fp16 32768 x 512 14.01-
        // 14.08 -> 12.98-13.03; bf16 with fp32 weights 13.27 against 14.10. At
        // 16384 rows and below within 2% either way; rows of 48 vectors (bf16
        // 384 columns, a quarter of the lanes idle) 2.5% slower. Where the
        // 512-lane grid above is built (bf16, fp32) it takes these rows up to 20
        // blocks per CU.
        if (!res && c->vector_path == 1 && c->lanes_per_row == 64 && c->vecs_per_lane == 1 &&
            c->wg_threads == 256 && N * elem_size(dtype) / 16 == 64 && row_blocks > kFwdRows64MinBlocks * cus) {
            c->wg_threads = (int32_t)kMaxVecLanes;
            c->rows_per_wg = (int32_t)(kMaxVecLanes / 64);
            const int64_t blocks = (M + c->rows_per_wg - 1) / c->rows_per_wg;
            grid = blocks < kMaxGrid ? blocks : kMaxGrid;
        }
        if (c->vector_path == 1 && fwd_row_walk(M, N * elem_size(dtype) / 16, dtype, res))
            grid = std::min<int64_t>(kMaxGrid, (row_blocks + kFwdLongWalk - 1) / kFwdLongWalk);
        // Element kernels keep a workgroup per row. On rows sized by
        // elem_lanes a resident grid walking the rows was as fast or slower
        // (bf16 16384 x 12002: 138 us against 148; 16384 x 4100: 52.5 against
        // 55.1); it had helped only with every row on 1024 lanes.
        const int64_t in_bytes = M * N * elem_size(dtype);
        c->stream_loads = (c->vector_path == 1 && c->lanes_per_row >= 64 && in_bytes >= kStreamMinBytes) ? 1 : 0;
    } else {
        const int64_t cus = num_cus > 0 ? num_cus : 1;
        const int deep = deep_prefetch(is_bwd, N, dtype, c);
        int64_t want = (c->vector_path == kWidePath ? 1 : deep ? deep : c->lanes_per_row < 64 ? 3 : 2) * cus;
        // element rows: about 1024 lanes per CU, 2 to 8 workgroups (bf16 16384
        // x 300 on 64 lanes: 16.7 us at 8 per CU, 19.0 at 2)
        if (c->vector_path == kElemPath)
            want = std::min<int64_t>(8, std::max<int64_t>(2, 1024 / c->lanes_per_row)) * cus;
        // partial rows are written once and read once (8 * N bytes each); at
        // most 1/kPartialShare of the 3 * M * N * elem algorithmic bytes, so
        // at most 3 * M * elem / (8 * kPartialShare) rows (N cancels)
        const int64_t cap = 3 * M * elem_size(dtype) / (8 * kPartialShare);
        if (want > cap) want = cap > cus ? cap : cus;
        const int64_t resident = cus * (blocks_per_cu > 0 ? blocks_per_cu : 1);
        if (want > resident) want = resident;
        if (wide_long_walk(M, dtype, cus, c)) want = 2 * cus;
        grid = row_blocks < want ? row_blocks : want;
        // Rows narrower than a wavefront take three workgroups per CU. When
        // the row blocks do not split evenly over them, some walk one block
        // more and finish alone, their CU half idle meanwhile; two per CU
        // then carry the same blocks per CU in fuller walks. Taken when it
        // cuts the largest blocks per CU (walk x workgroups per CU) by at
        // least 5%: bf16 16384 x 128 8.45 -> 7.14 us (6 -> 4 blocks per CU),
        // 65536 x 128 14.78 -> 14.11 (18 -> 16). 1M x 128 keeps three (258
        // against 256 blocks; two per CU measured 136.0 against 130.8 us).
        if (c->vector_path == 1 && c->lanes_per_row < 64 && grid == 3 * cus) {
            const int64_t load3 = (row_blocks + 3 * cus - 1) / (3 * cus) * 3;
            const int64_t load2 = (row_blocks + 2 * cus - 1) / (2 * cus) * 2;
            if (20 * load2 <= 19 * load3) grid = 2 * cus;
        }
        // 1024-lane workgroups at two per CU that would each walk a single
        // row block: one per CU walking two, the second block's loads issued
        // before the first's arithmetic, and half the partial rows (bf16 4096
        // x 1024 10.29 -> 9.55 us, 8192 x 512 10.11 -> 9.98; fp32 2048 x 1024
        // 10.36 -> 8.80, 4096 x 512 9.99 -> 9.27). Uneven walks of one or two
        // blocks went either way (bf16 6144 x 1024 2.6% slower at one per CU).
        if (c->vector_path == 1 && c->wg_threads == kMaxVecLanes && !deep && grid == 2 * cus &&
            row_blocks <= 2 * cus)
            grid = std::max<int64_t>(cus, (row_blocks + 1) / 2);
        // A few rows (a decode step's): one workgroup walks them all and
        // writes dW itself, with no combine launch. Faster while M * N is at
        // most kBwdSingleElems and the walk at most kBwdSinglePasses row
        // blocks (each pass costs a load latency): bf16 4096 columns 5.1 ->
        // 3.2 us at M = 2 and
        // 5.2 -> 4.6 at M = 4 (6 rows: 5.3 against 6.0), 8192 columns 6.0 ->
        // 4.8 at M = 2, 2048 columns 5.5 -> 4.3 at M = 8, fp32 4096 5.5 -> 3.3
        // at M = 2 (graph-timed rows + combine against the one kernel). Vector
        // rows only: the element and scalar kernels were not timed this way.
        if (c->vector_path == 1 && row_blocks <= kBwdSinglePasses && M * N <= kBwdSingleElems) grid = 1;
        // Split rows: groups of K members, as many as stay resident together
        // (every member of a group must run at once: they wait on each
        // other), at most one per row.
        if (c->vector_path == kSplitPath) {
            const int64_t K = split_members(*c);
            int64_t groups = resident / K;
            if (groups > M) groups = M;
            grid = (groups > 0 ? groups : 1) * K;
        }
    }
    c->grid = grid > 0 ? grid : 1;
    c->partial_rows = c->grid / split_members(*c);
    c->partial_stride = (N + rmsn::kPartialAlign - 1) / rmsn::kPartialAlign * rmsn::kPartialAlign;
}

// ---- per-device caches -----------------------------------------------------
//
// Device properties (compute units), kernel occupancy, and the resolved
// launch configuration of each (device, M, N, format, direction, residual,
// alignment class), so that a call does one device query and one locked
// lookup instead of re-running the ladder: a decode-sized backward kernel
// takes 2.5 us, and the host path must stay well below that. The
// configuration cache is cleared when it reaches kCacheMax entries (a caller
// cycling through many shapes still gets the same configurations, recomputed).

struct DeviceInfo {
    int num_cus = 0;
    std::unordered_map<const void *, int> occupancy;
};

struct CfgKey {
    int64_t M, N;
    int dev, dtype, is_bwd, res, act, w;
    bool operator==(const CfgKey &o) const {
        return M == o.M && N == o.N && dev == o.dev && dtype == o.dtype && is_bwd == o.is_bwd && res == o.res &&
               act == o.act && w == o.w;
    }
};

struct CfgKeyHash {
    size_t operator()(const CfgKey &k) const {
        uint64_t h = 1469598103934665603ull;  // FNV-1a over the fields
        for (int64_t v : {k.M, k.N, (int64_t)k.dev, (int64_t)k.dtype, (int64_t)k.is_bwd, (int64_t)k.res,
                          (int64_t)k.act, (int64_t)k.w}) {
            h ^= (uint64_t)v;
            h *= 1099511628211ull;
        }
        return (size_t)h;
    }
};

struct Resolved {
    rmsnorm_config c;
    const void *fn;
};

constexpr size_t kCacheMax = 4096;

std::mutex g_mu;
std::unordered_map<int, DeviceInfo> g_devices;
std::unordered_map<CfgKey, Resolved, CfgKeyHash> g_resolved;
std::unordered_map<CfgKey, int64_t, CfgKeyHash> g_workspace;  // key fields is_bwd..w unused (0)

int current_device(int *dev) { return hipGetDevice(dev) == hipSuccess ? RMSN_OK : RMSN_EHIP; }

int device_info(int dev, int *num_cus) {
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceInfo &d = g_devices[dev];
    if (d.num_cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return RMSN_EHIP;
        d.num_cus = n;
    }
    *num_cus = d.num_cus;
    return RMSN_OK;
}

int occupancy(int dev, const void *fn, int wg, int *blocks) {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto &occ = g_devices[dev].occupancy;
        auto it = occ.find(fn);
        if (it != occ.end()) {
            *blocks = it->second;
            return RMSN_OK;
        }
    }
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, wg, 0) != hipSuccess || b <= 0) return RMSN_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    g_devices[dev].occupancy[fn] = b;
    *blocks = b;
    return RMSN_OK;
}

const void *kernel_for(const rmsnorm_config &c, int64_t N, int dtype, int is_bwd, int res) {
    if (!c.vector_path) return rmsn::scalar_kernel(dtype, is_bwd, res, N <= rmsn::kScalarLdsCols ? 1 : 0);
    if (c.vector_path == kElemPath) return rmsn::elem_kernel(dtype, is_bwd, res, c.vecs_per_lane, c.elems_per_access, c.lanes_per_row);
    if (c.vector_path == kLoopPath) {
        if (is_bwd || (c.copy_mode != 0 && c.copy_mode != kCopyLds) || c.lanes_per_row != kMaxVecLanes ||
            c.wg_threads != rmsn::kWideLanes || c.prefetch != 0)
            return nullptr;
        const KernelEntry *e =
            rmsn::fwd_loop_kernel(dtype, res, c.vecs_per_lane, c.kept_vecs, c.copy_mode ? kLoopLdsVecs : 0);
        return e ? e->fn : nullptr;
    }
    if (c.vector_path == kSplitPath) {
        const int64_t K = split_members(c);
        if (!is_bwd || c.copy_mode != 0 || c.lanes_per_row != K * rmsn::kWideLanes || K < 2 || K > rmsn::kMaxSplit ||
            c.wg_threads != rmsn::kWideLanes)
            return nullptr;
        const KernelEntry *e = rmsn::bwd_split_kernel(dtype, res, c.vecs_per_lane, c.prefetch);
        return e ? e->fn : nullptr;
    }
    if (c.vector_path == kWidePath) {
        const KernelEntry *e = !is_bwd ? nullptr
                               : c.copy_mode == kCopyLds
                                   ? (res ? nullptr : rmsn::bwd_wide_lds_kernel(dtype, c.lanes_per_row, c.vecs_per_lane, c.prefetch))
                                   : rmsn::bwd_wide_kernel(dtype, res, c.vecs_per_lane, c.prefetch);
        return e ? e->fn : nullptr;
    }
    if (is_bwd && c.copy_mode == kCopyLds) {
        if (c.vector_path != 1 || c.vecs_per_lane != 1) return nullptr;
        const KernelEntry *e = row_is_wg(c) ? rmsn::bwd_lds_kernel(dtype, res, 0, (int)kMaxVecLanes, c.prefetch)
                                            : rmsn::bwd_lds_kernel(dtype, res, c.lanes_per_row, c.wg_threads, c.prefetch);
        return e ? e->fn : nullptr;
    }
    if (is_bwd && row_is_wg(c)) {
        const KernelEntry *e = rmsn::bwd_vec_kernel(dtype, res, 0, 1, (int)kMaxVecLanes, c.prefetch);
        return e ? e->fn : nullptr;
    }
    const KernelEntry *e =
        is_bwd ? rmsn::bwd_vec_kernel(dtype, res, c.lanes_per_row, c.vecs_per_lane, c.wg_threads, c.prefetch)
               : rmsn::fwd_vec_kernel(dtype, res, c.lanes_per_row, c.vecs_per_lane, c.wg_threads, c.prefetch);
    return e ? e->fn : nullptr;
}

// The ladder's full configuration on device `dev`, uncached.
int resolve_uncached(int dev, int64_t M, int64_t N, int dtype, int is_bwd, int res, const Align &a,
                     rmsnorm_config *c, const void **fn) {
    std::memset(c, 0, sizeof *c);
    int cus = 0, blocks = 0;
    int st = device_info(dev, &cus);
    if (st != RMSN_OK) return st;
    ladder_shape(M, N, dtype, is_bwd, res, a, cus, c);
    const void *k = kernel_for(*c, N, dtype, is_bwd, res);
    if (!k) return RMSN_ECONFIG;
    st = occupancy(dev, k, c->wg_threads, &blocks);
    if (st != RMSN_OK) return st;
    ladder_grid(M, N, dtype, is_bwd, res, cus, blocks, c);
    ladder_prefetch(M, N, dtype, is_bwd, cus, c, res);
    ladder_copy(M, N, dtype, is_bwd, res, cus, c);
    k = kernel_for(*c, N, dtype, is_bwd, res);
    if (!k) return RMSN_ECONFIG;
    *fn = k;
    return RMSN_OK;
}

// Full configuration on device `dev` (res: the residual-fused kernel), cached.
int resolve(int dev, int64_t M, int64_t N, int dtype, int is_bwd, int res, const Align &a, rmsnorm_config *c,
            const void **fn) {
    const CfgKey key{M, N, dev, dtype, is_bwd, res, a.act, a.w};
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_resolved.find(key);
        if (it != g_resolved.end()) {
            *c = it->second.c;
            if (fn) *fn = it->second.fn;
            return RMSN_OK;
        }
    }
    const void *k = nullptr;
    const int st = resolve_uncached(dev, M, N, dtype, is_bwd, res, a, c, &k);
    if (st != RMSN_OK) return st;
    if (fn) *fn = k;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_resolved.size() >= kCacheMax) g_resolved.clear();
    g_resolved.emplace(key, Resolved{*c, k});
    return RMSN_OK;
}

// Bytes of the partial rows at the start of the workspace.
int64_t partial_bytes(const rmsnorm_config &c) { return c.partial_rows * c.partial_stride * int64_t(sizeof(float)); }

// The backward's workspace: the partial rows, then (split rows) one exchange
// slot per workgroup, 256-byte aligned (partial_stride is a multiple of 64
// floats).
int64_t workspace_for(const rmsnorm_config &c) {
    const int64_t slots = c.vector_path == kSplitPath ? c.grid * rmsn::kSplitSlotBytes : 0;
    return partial_bytes(c) + (slots + 255) / 256 * 256;
}

// The documented workspace requirement of rmsnorm_bwd on device `dev`: enough
// for every row kernel the call may pick (plain or residual-fused, vector or
// scalar), so neither the caller's alignment nor the residual variant changes
// the answer. Cached per (device, M, N, format); *need receives the bytes.
int workspace_need(int dev, int64_t M, int64_t N, int dtype, int64_t *need) {
    const CfgKey key{M, N, dev, dtype, 0, 0, 0, 0};
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_workspace.find(key);
        if (it != g_workspace.end()) {
            *need = it->second;
            return RMSN_OK;
        }
    }
    int64_t most = 0;
    for (int fused = 0; fused <= 1; ++fused) {
        for (int v : {1, 4, 8, 16}) {  // every pointer alignment that selects a different kernel
            const Align a{v > elem_size(dtype) ? v : elem_size(dtype), v > w_size(dtype) ? v : w_size(dtype)};
            rmsnorm_config c;
            const int s = resolve(dev, M, N, dtype, 1, fused, a, &c, nullptr);
            if (s != RMSN_OK) return s;
            const int64_t b = workspace_for(c);
            if (b > most) most = b;
        }
    }
    *need = most;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_workspace.size() >= kCacheMax) g_workspace.clear();
    g_workspace.emplace(key, most);
    return RMSN_OK;
}

int launch(const void *fn, int64_t grid, int wg, void **args, hipStream_t stream) {
    if (grid <= 0) return RMSN_OK;
    if (grid > INT32_MAX) return RMSN_ECONFIG;
    if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)wg), args, 0, stream) != hipSuccess)
        return RMSN_EHIP;
    return RMSN_OK;
}

// An explicit configuration (config search, benchmarks) is checked against
// the shape: the kernel must exist, cover the row, and the grid must be
// positive. Shape fields derived from lanes_per_row are recomputed.
int explicit_config(const rmsnorm_config *req, int64_t M, int64_t N, int dtype, int is_bwd, int res,
                    const Align &a, rmsnorm_config *c, const void **fn) {
    std::memset(c, 0, sizeof *c);
    if (req->grid < 1 || req->grid > INT32_MAX) return RMSN_ECONFIG;
    if (req->vector_path < 0 || req->vector_path > kLoopPath) return RMSN_ECONFIG;
    if (req->kept_vecs != 0 && req->vector_path != kLoopPath) return RMSN_ECONFIG;
    if (req->vector_path == kElemPath) {
        const int64_t k = req->vecs_per_lane;
        const int64_t g = req->elems_per_access ? req->elems_per_access : elem_group(N, dtype, a);
        const int64_t lanes = req->lanes_per_row;
        if (!elem_lanes_ok(lanes) || (req->wg_threads != 0 && req->wg_threads != lanes) ||
            !elem_group_ok(N, dtype, a, g) || k < 1 || k * g > rmsn::kElemMaxK || lanes * k * g < N ||
            req->prefetch != 0 || req->stream_loads != 0 || req->copy_mode != 0)
            return RMSN_ECONFIG;
        set_elem_shape(N, (int)g, (int)lanes, c);
        c->vecs_per_lane = (int32_t)k;
    } else if (req->elems_per_access != 0) {
        return RMSN_ECONFIG;
    } else if (req->vector_path == kLoopPath) {
        // the forward's two-pass kernel: 1024 lanes, vecs_per_lane per chunk
        if (is_bwd || !vector_ok(N, dtype, a) || N * elem_size(dtype) > (int64_t)UINT32_MAX ||
            req->lanes_per_row != kMaxVecLanes ||
            (req->wg_threads != 0 && req->wg_threads != rmsn::kWideLanes) || req->prefetch != 0 ||
            (req->copy_mode != 0 && req->copy_mode != kCopyLds) || req->stream_loads < 0 || req->stream_loads > 1 ||
            req->kept_vecs < 0)
            return RMSN_ECONFIG;
        set_loop_shape(req->vecs_per_lane, req->kept_vecs, req->copy_mode, c);
    } else if (req->vector_path == kSplitPath) {
        // K = lanes_per_row / 1024 members per row; the grid whole groups,
        // all resident at once on the current device
        const int64_t nvec = N * elem_size(dtype) / 16;
        const int64_t K = req->lanes_per_row / rmsn::kWideLanes;
        if (!is_bwd || !vector_ok(N, dtype, a) || req->lanes_per_row % rmsn::kWideLanes != 0 || K < 2 ||
            K > rmsn::kMaxSplit || (req->wg_threads != 0 && req->wg_threads != rmsn::kWideLanes) ||
            (int64_t)req->lanes_per_row * req->vecs_per_lane < nvec || req->prefetch < 0 || req->prefetch > 1 ||
            req->copy_mode != 0 || req->stream_loads != 0 || req->grid % K != 0)
            return RMSN_ECONFIG;
        set_split_shape(K, req->vecs_per_lane, req->prefetch, c);
        const void *k = kernel_for(*c, N, dtype, is_bwd, res);
        if (!k) return RMSN_ECONFIG;
        int dev = 0, cus = 0, blocks = 0;
        int st = current_device(&dev);
        if (st == RMSN_OK) st = device_info(dev, &cus);
        if (st == RMSN_OK) st = occupancy(dev, k, rmsn::kWideLanes, &blocks);
        if (st != RMSN_OK) return st;
        if (req->grid > (int64_t)cus * blocks) return RMSN_ECONFIG;
    } else if (req->vector_path) {
        const int64_t nvec = N * elem_size(dtype) / 16;
        if (!vector_ok(N, dtype, a)) return RMSN_ECONFIG;
        if ((int64_t)req->lanes_per_row * req->vecs_per_lane < nvec) return RMSN_ECONFIG;
        if (req->copy_mode < 0 || req->copy_mode > kCopyLds) return RMSN_ECONFIG;
        const int max_pf = req->copy_mode == kCopyLds ? kMaxLdsStages : 2;
        // the LDS stages: at least two for rows of one vector per lane, one for wide rows
        if (req->copy_mode == kCopyLds &&
            (!is_bwd || req->prefetch < (req->vector_path == 1 ? 2 : req->vector_path == kWidePath ? 1 : 99)))
            return RMSN_ECONFIG;
        if (req->lanes_per_row < 1 || req->wg_threads < 0 || req->prefetch < 0 || req->prefetch > max_pf)
            return RMSN_ECONFIG;
        if (req->wg_threads > 0 && (req->wg_threads % req->lanes_per_row) != 0) return RMSN_ECONFIG;
        // wide rows: 1024 lanes, or 512 for the LDS-staged kernels; the workgroup is the row
        const int wide_lanes = req->lanes_per_row == 512 && req->copy_mode == kCopyLds ? 512 : rmsn::kWideLanes;
        if (req->vector_path == kWidePath &&
            (req->lanes_per_row != wide_lanes || (req->wg_threads != 0 && req->wg_threads != wide_lanes)))
            return RMSN_ECONFIG;
        if (req->stream_loads < 0 || req->stream_loads > 1) return RMSN_ECONFIG;
        set_vector_shape(req->lanes_per_row, req->vecs_per_lane, req->wg_threads, req->prefetch, c);
        c->vector_path = req->vector_path;
        c->copy_mode = req->copy_mode;
    } else if (req->copy_mode != 0) {
        return RMSN_ECONFIG;
    } else {
        set_scalar_shape(c);
    }
    const void *k = kernel_for(*c, N, dtype, is_bwd, res);
    if (!k) return RMSN_ECONFIG;
    // ladder_grid fills the derived fields; its rules may also reshape the
    // ladder's own choice (the workgroup of some forward rows), which an
    // explicit configuration does not take: the kernel above was chosen for
    // the requested workgroup, and launching it on another would be refused
    const int32_t wg = c->wg_threads, rows = c->rows_per_wg;
    ladder_grid(M, N, dtype, is_bwd, res, 1, 1, c);
    c->wg_threads = wg;
    c->rows_per_wg = rows;
    c->grid = req->grid;
    c->prefetch = req->vector_path ? req->prefetch : 0;  // as requested (the kernel above was chosen by it)
    c->partial_rows = req->grid / split_members(*c);
    c->stream_loads = req->vector_path ? req->stream_loads : 0;
    if (kernel_for(*c, N, dtype, is_bwd, res) != k) return RMSN_ECONFIG;
    *fn = k;
    return RMSN_OK;
}

int fwd_impl(const void *x, const void *res, const void *w, float eps, int64_t M, int64_t N, int dtype, void *h,
             void *y, float *rstd, void *stream, const rmsnorm_config *req) {
    int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!std::isfinite(eps) || eps < 0.f) return RMSN_EINVAL;
    if (M == 0) return RMSN_OK;
    if (!x || !w || !y || (res && !h)) return RMSN_EINVAL;
    const int fused = res ? 1 : 0;
    const Align a = fused ? align_of({x, y, res, h}, w) : align_of({x, y}, w);
    if (!natural(a, dtype) || !aligned4(rstd)) return RMSN_EINVAL;
    rmsnorm_config c;
    const void *fn = nullptr;
    if (req) {
        st = explicit_config(req, M, N, dtype, 0, fused, a, &c, &fn);
    } else {
        int dev = 0;
        st = current_device(&dev);
        if (st == RMSN_OK) st = resolve(dev, M, N, dtype, 0, fused, a, &c, &fn);
    }
    if (st != RMSN_OK) return st;
    int32_t n32 = (int32_t)N;
    int32_t nvec = (c.vector_path == 1 || c.vector_path == kLoopPath) ? (int32_t)(N * elem_size(dtype) / 16) : 0;
    int32_t stream_ld = c.stream_loads;
    void *args[] = {(void *)&x, (void *)&res, (void *)&w, (void *)&h, (void *)&y, (void *)&rstd,
                    (void *)&eps, (void *)&M, (void *)&n32, (void *)&nvec, (void *)&stream_ld};
    return launch(fn, c.grid, c.wg_threads, args, static_cast<hipStream_t>(stream));
}

// Partial rows the combine sums side by side: the fewest of 8, 16 and 32
// that launch at least 16 workgroups and leave each lane at most 8 partial
// rows (16 when they launch at least 256 workgroups); else 64. A lane adds its
// rows one after another and the S slice sums then go through a fixed tree
// of log2(S) levels in LDS (fp64, twice the bytes of fp32): fewer slices mean
// fewer, wider workgroups and a shallower tree, more slices shorter chains.
// Measured per launch with the fp64 sums (us, slices 8 / 16 / 32 / 64,
// graph-replayed): P = 256, N = 4096: 3.81 / 3.02 / 2.57 / 2.72; N = 2560:
// 3.78 / 2.98 / 2.56 / 2.70; N = 7168: 3.82 / 3.02 / 2.61 / 2.78; N = 8192:
// 3.82 / 3.02 / 2.61 / 2.79; N = 32768: 4.30 / 3.58 / 3.69 / 4.62; P = 512,
// N = 4100: 8.29 / 3.91 / 3.10 / 2.67; N = 8192: 5.63 / 3.97 / 3.13 / 2.79;
// P = 384, N = 4096: 4.74 / 3.39 / 3.12 / 2.97; P = 320, N = 4096: 4.18 /
// 3.58 / 2.86 / 2.84; P = 128, N = 4096: 2.93 / 2.49 / 2.62 / 2.49; P = 768,
// N = 128: 6.97 / 4.60 / 3.39 / 3.11; P = 64, N = 1024: 2.31 / 2.43 / 2.29 /
// 2.27. With fp32 sums (us, 64 / 32 / 16 / 8): P = 32, N = 262144: 12.65 /
// 7.10 / 4.75 / 3.67; P = 64, N = 131072: 7.45 / 4.95 / 3.84 / 4.01; P = 128,
// N = 65536: 5.08 / 3.83 / 3.59 / 3.41.
int combine_slices(int64_t P, int64_t N) {
    for (int S : {8, 16, 32}) {
        const int64_t cols = 4 * rmsn::kCombineWG / S;
        const int64_t wgs = (N + cols - 1) / cols;
        const int64_t rows = (P + S - 1) / S;
        if (wgs >= 16 && rows <= (wgs >= 256 ? 16 : 8)) return S;
    }
    return 64;
}

int combine_impl(const void *workspace, int64_t P, int64_t N, float *dw, hipStream_t s) {
    if (N < 1 || N > kMaxN || P < 0) return RMSN_EINVAL;
    if (!dw || !aligned4(dw)) return RMSN_EINVAL;
    if (P > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)) return RMSN_EWORKSPACE;
    const float *cpartial = static_cast<const float *>(workspace);
    int64_t ldp = (N + rmsn::kPartialAlign - 1) / rmsn::kPartialAlign * rmsn::kPartialAlign;
    int32_t n32 = (int32_t)N;
    void *cargs[] = {(void *)&cpartial, (void *)&ldp, (void *)&P, (void *)&n32, (void *)&dw};
    const int S = combine_slices(P, N);
    const int64_t cols = 4 * rmsn::kCombineWG / S;
    return launch(rmsn::dw_combine_kernel(S), (N + cols - 1) / cols, rmsn::kCombineWG, cargs, s);
}

// dw_direct: when not NULL and the grid writes a single partial row (one
// workgroup, or one group of a split row), that row is dW itself, written straight to dw_direct (16-byte aligned) instead of
// the workspace; *partial_rows is then 0 and there is nothing to combine.
// scratch: the workspace is the static device array of rmsnorm_bwd_noalloc
// (the ladder's configuration only); `workspace` is then set to its address
// on the current device, after every argument check, and the shape is refused
// (RMSN_ESCRATCH) when its partial rows do not fit.
int rows_impl(const void *x, const void *w, const void *dy, const void *dh, const float *rstd, int64_t M,
              int64_t N, int dtype, void *dx, void *&workspace, size_t workspace_bytes, int64_t *partial_rows,
              hipStream_t s, const rmsnorm_config *req, float *dw_direct = nullptr, bool scratch = false) {
    int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!partial_rows) return RMSN_EINVAL;
    *partial_rows = 0;
    if (M == 0) return RMSN_OK;
    if (!x || !w || !dy || !rstd || !dx) return RMSN_EINVAL;
    if (scratch && req) return RMSN_EINVAL;
    if (!scratch && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)) return RMSN_EWORKSPACE;
    const int fused = dh ? 1 : 0;
    const Align a = fused ? align_of({x, dy, dx, dh}, w) : align_of({x, dy, dx}, w);
    if (!natural(a, dtype) || !aligned4(rstd)) return RMSN_EINVAL;
    rmsnorm_config c;
    const void *fn = nullptr;
    if (req) {
        st = explicit_config(req, M, N, dtype, 1, fused, a, &c, &fn);
        if (st != RMSN_OK) return st;
        if (workspace_bytes < (size_t)workspace_for(c)) return RMSN_EWORKSPACE;
    } else {
        int dev = 0;
        st = current_device(&dev);
        if (st == RMSN_OK) st = resolve(dev, M, N, dtype, 1, fused, a, &c, &fn);
        if (st != RMSN_OK) return st;
        if (scratch) {
            // the static array: what this configuration writes must fit
            if ((uint64_t)workspace_for(c) > (uint64_t)RMSN_NOALLOC_SCRATCH_BYTES) return RMSN_ESCRATCH;
            st = rmsn::scratch_region(dev, &workspace);
            if (st != RMSN_OK) return st;
        } else {
            // the documented contract: at least what rmsnorm_bwd_workspace_bytes reports
            int64_t need = 0;
            st = workspace_need(dev, M, N, dtype, &need);
            if (st != RMSN_OK) return st;
            if (workspace_bytes < (size_t)need) return RMSN_EWORKSPACE;
        }
    }
    int32_t n32 = (int32_t)N;
    int32_t nvec = (c.vector_path == 1 || c.vector_path == kWidePath || c.vector_path == kSplitPath)
                       ? (int32_t)(N * elem_size(dtype) / 16)
                       : 0;
    const bool direct = dw_direct && c.partial_rows == 1 && aligned16(dw_direct);
    float *partial = direct ? dw_direct : static_cast<float *>(workspace);
    int64_t ldp = c.partial_stride;
    if (c.vector_path == kSplitPath) {
        // the exchange slots after the partial rows, zeroed by a kernel (so
        // that the call can be captured in a graph)
        void *xch = static_cast<char *>(workspace) + partial_bytes(c);
        int64_t words = c.grid * rmsn::kSplitSlotBytes / 4;
        void *zargs[] = {(void *)&xch, (void *)&words};
        st = launch(rmsn::fill_zero_kernel(), (words + 255) / 256, 256, zargs, s);
        if (st != RMSN_OK) return st;
        int32_t K = (int32_t)split_members(c);
        void *args[] = {(void *)&x, (void *)&w, (void *)&dy, (void *)&dh, (void *)&rstd, (void *)&dx,
                        (void *)&partial, (void *)&ldp, (void *)&M, (void *)&n32, (void *)&nvec, (void *)&K,
                        (void *)&xch};
        st = launch(fn, c.grid, c.wg_threads, args, s);
        if (st == RMSN_OK) *partial_rows = direct ? 0 : c.partial_rows;
        return st;
    }
    void *args[] = {(void *)&x, (void *)&w, (void *)&dy, (void *)&dh, (void *)&rstd, (void *)&dx,
                    (void *)&partial, (void *)&ldp, (void *)&M, (void *)&n32, (void *)&nvec};
    st = launch(fn, c.grid, c.wg_threads, args, s);
    if (st == RMSN_OK) *partial_rows = direct ? 0 : c.partial_rows;
    return st;
}

int bwd_impl(const void *x, const void *w, const void *dy, const void *dh, const float *rstd, int64_t M,
             int64_t N, int dtype, void *dx, float *dw, void *workspace, size_t workspace_bytes, void *stream,
             const rmsnorm_config *req, bool scratch = false) {
    int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!aligned4(dw)) return RMSN_EINVAL;
    if (M == 0) {
        if (!dw) return RMSN_OK;
        int64_t n = N;
        void *args[] = {(void *)&dw, (void *)&n};
        const int64_t grid = (N + 255) / 256 < 1024 ? (N + 255) / 256 : 1024;
        return launch(rmsn::fill_zero_kernel(), grid, 256, args, s);
    }
    if (!dw) return RMSN_EINVAL;
    int64_t P = 0;
    // A single workgroup (a few rows, e.g. one decode step's) writes dW
    // itself: no combine launch, about half of such a call's time.
    st = rows_impl(x, w, dy, dh, rstd, M, N, dtype, dx, workspace, workspace_bytes, &P, s, req, dw, scratch);
    if (st != RMSN_OK) return st;
    return P == 0 ? RMSN_OK : combine_impl(workspace, P, N, dw, s);
}

}  // namespace

extern "C" {

const char *rmsnorm_status_str(int status) {
    switch (status) {
    case RMSN_OK: return "ok";
    case RMSN_EINVAL: return "invalid argument";
    case RMSN_EDTYPE: return "unsupported dtype";
    case RMSN_EWORKSPACE: return "workspace missing, misaligned or too small";
    case RMSN_EHIP: return "HIP runtime error";
    case RMSN_ECONFIG: return "launch configuration does not fit the shape";
    case RMSN_ESCRATCH: return "shape needs more workspace than the static no-allocation scratch holds";
    default: return "unknown status";
    }
}

const char *rmsnorm_build_info(void) { return RMSN_BUILD_INFO; }

int rmsnorm_select_config(int64_t M, int64_t N, int dtype, int is_bwd, int aligned, int num_cus,
                          int blocks_per_cu, rmsnorm_config *out) {
    const int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!out || num_cus < 1 || blocks_per_cu < 1 || (is_bwd != 0 && is_bwd != 1)) return RMSN_EINVAL;
    if (aligned < 0 || aligned > 16 || (aligned > 1 && (aligned & (aligned - 1)) != 0)) return RMSN_EINVAL;
    // 0: every pointer only naturally aligned; 1: all 16-byte aligned; 2..16: that many bytes
    const int v = aligned == 1 ? 16 : aligned;
    const Align a{v > elem_size(dtype) ? v : elem_size(dtype), v > w_size(dtype) ? v : w_size(dtype)};
    std::memset(out, 0, sizeof *out);
    ladder_shape(M, N, dtype, is_bwd, 0, a, num_cus, out);
    ladder_grid(M, N, dtype, is_bwd, 0, num_cus, blocks_per_cu, out);
    ladder_prefetch(M, N, dtype, is_bwd, num_cus, out);
    ladder_copy(M, N, dtype, is_bwd, 0, num_cus, out);
    return RMSN_OK;
}

int rmsnorm_query_config(int64_t M, int64_t N, int dtype, int is_bwd, rmsnorm_config *out) {
    const int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!out || (is_bwd != 0 && is_bwd != 1)) return RMSN_EINVAL;
    int dev = 0;
    const int s = current_device(&dev);
    if (s != RMSN_OK) return s;
    return resolve(dev, M, N, dtype, is_bwd, 0, Align{16, 16}, out, nullptr);
}

int rmsnorm_fwd(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype, void *y,
                float *rstd, void *stream) {
    return fwd_impl(x, nullptr, w, eps, M, N, dtype, nullptr, y, rstd, stream, nullptr);
}

int rmsnorm_fwd_with_config(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype,
                            void *y, float *rstd, const rmsnorm_config *cfg, void *stream) {
    if (!cfg) return RMSN_EINVAL;
    return fwd_impl(x, nullptr, w, eps, M, N, dtype, nullptr, y, rstd, stream, cfg);
}

int rmsnorm_fwd_residual(const void *x, const void *res, const void *w, float eps, int64_t M, int64_t N,
                         int dtype, void *h, void *y, float *rstd, const rmsnorm_config *cfg, void *stream) {
    if (M > 0 && !res) return RMSN_EINVAL;
    if (M == 0) return check_shape(M, N, dtype);
    return fwd_impl(x, res, w, eps, M, N, dtype, h, y, rstd, stream, cfg);
}

int64_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype) {
    int st = check_shape(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (M == 0) return 0;
    int dev = 0;
    st = current_device(&dev);
    if (st != RMSN_OK) return st;
    int64_t need = 0;
    st = workspace_need(dev, M, N, dtype, &need);
    return st != RMSN_OK ? st : need;
}

int rmsnorm_bwd(const void *x, const void *w, const void *dy, const float *rstd, int64_t M, int64_t N,
                int dtype, void *dx, float *dw, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_impl(x, w, dy, nullptr, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, stream, nullptr);
}

int rmsnorm_bwd_with_config(const void *x, const void *w, const void *dy, const float *rstd, int64_t M,
                            int64_t N, int dtype, void *dx, float *dw, void *workspace,
                            size_t workspace_bytes, const rmsnorm_config *cfg, void *stream) {
    if (!cfg) return RMSN_EINVAL;
    return bwd_impl(x, w, dy, nullptr, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, stream, cfg);
}

int rmsnorm_bwd_residual(const void *h, const void *w, const void *dy, const void *dh, const float *rstd,
                         int64_t M, int64_t N, int dtype, void *dx, float *dw, void *workspace,
                         size_t workspace_bytes, const rmsnorm_config *cfg, void *stream) {
    if (M > 0 && !dh) return RMSN_EINVAL;
    return bwd_impl(h, w, dy, dh, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, stream, cfg);
}

int rmsnorm_bwd_noalloc(const void *x, const void *w, const void *dy, const float *rstd, int64_t M, int64_t N,
                        int dtype, void *dx, float *dw, void *stream) {
    return bwd_impl(x, w, dy, nullptr, rstd, M, N, dtype, dx, dw, nullptr, 0, stream, nullptr, true);
}

int rmsnorm_bwd_rows(const void *x, const void *w, const void *dy, const float *rstd, int64_t M, int64_t N,
                     int dtype, void *dx, void *workspace, size_t workspace_bytes, int64_t *partial_rows,
                     void *stream) {
    return rows_impl(x, w, dy, nullptr, rstd, M, N, dtype, dx, workspace, workspace_bytes, partial_rows,
                     static_cast<hipStream_t>(stream), nullptr);
}

int rmsnorm_bwd_combine(const void *workspace, int64_t partial_rows, int64_t N, float *dw, void *stream) {
    return combine_impl(workspace, partial_rows, N, dw, static_cast<hipStream_t>(stream));
}

}  // extern "C"
