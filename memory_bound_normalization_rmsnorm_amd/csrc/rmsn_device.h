// rmsn_device.h -- device helpers shared by the RMSNorm kernels (gfx950).
//
// * buffer-resource loads/stores: an access whose byte offset is at or past
//   the resource's record count reads 0 and writes nothing, which masks row
//   tails and missing rows without branches;
// * 16-byte vector loads/stores and their unpacking into fp32 lanes;
// * bf16 <-> fp32 conversion (bf16 stores round to nearest even with the
//   hardware v_cvt_pk_bf16_f32);
// * sums over a group of lanes that share one row: DPP within 16 lanes,
//   ds_swizzle across 32, v_readlane across the 64-lane wavefront, and LDS
//   across the wavefronts of a workgroup. Every sum has a fixed order, so
//   results are bit-identical from run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t g32x4 __attribute__((vector_size(16)));  // the buffer builtins' vector type
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Bit reinterpretation goes through these by-value helpers. Applied directly
// to an ext_vector element (`__builtin_bit_cast(float, v.y)`), clang reads
// element 0 whatever the element named, so vector components are always
// copied into a scalar first.
__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Storage types: fp32 is `float`; bf16 and fp16 are carried as their 16-bit
// patterns.
struct bf16_t {
    uint16_t bits;
};
struct f16_t {
    uint16_t bits;
};

// registers a lane's NV dW sums take, for occupancy estimates (with F64, the
// fp32 block sums, the fp64 totals, the fold's conversions and the fp64
// pairs' alignment)
constexpr int dw_sum_regs(int nv, bool f64) { return f64 ? 3 * nv + 8 : nv; }

constexpr int kDwBlockRows = 8;  // rows (row blocks) summed in fp32 before each fp64 fold

// One lane's dW running sums over the rows a workgroup walks, for NV columns.
// With F64, each row's term dy * x * rstd is added with an fp32 fma into a
// block sum, and every kDwBlockRows rows the block sums are added into fp64
// totals. Summed in fp32 alone over a walk of tens of rows, a column's
// rounding error grows with the walk and shows on columns whose total nearly
// cancels; the fp32 blocks keep the per-row cost to one fma (an fp64 fma per
// row measured 2-8% slower on several shapes). The workgroup's rows are the
// same for all its lanes, so the fold is taken uniformly. With F64 false the
// lane keeps plain fp32 sums (for kernels where the fp64 totals would cost
// resident workgroups).
template <int NV, bool F64>
struct DwSums {
    static constexpr bool kF64 = F64;
    float blk[NV];
    double tot[F64 ? NV : 1];
    int in_blk;

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < NV; ++i) blk[i] = 0.f;
#pragma unroll
        for (int i = 0; i < (F64 ? NV : 1); ++i) tot[i] = 0.0;
        in_blk = 0;
    }
    // term i of the current row: (dy * x) * rstd, gx = dy * x (exact for 16-bit inputs)
    __device__ __forceinline__ void add(int i, float gx, float r) { blk[i] = __builtin_fmaf(gx, r, blk[i]); }
    __device__ __forceinline__ void fold() {
        if constexpr (F64) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                tot[i] += (double)blk[i];
                blk[i] = 0.f;
            }
        }
        in_blk = 0;
    }
    // after each row (block of rows) the workgroup has added
    __device__ __forceinline__ void end_row() {
        if constexpr (F64) {
            if (++in_blk == kDwBlockRows) fold();
        }
    }
    // the sums, rounded to fp32 (call fold() first)
    __device__ __forceinline__ float get(int i) const {
        if constexpr (F64) return (float)tot[i];
        else return blk[i];
    }
};

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;  // elements per 16-byte vector
    static __device__ __forceinline__ float load(const float *p) { return *p; }
    static __device__ __forceinline__ void store(float *p, float v) { *p = v; }
    // the value store() writes, read back (the storage rounding, in registers)
    static __device__ __forceinline__ float rounded(float v) { return v; }
    static __device__ __forceinline__ void unpack(const u32x4 &v, float (&f)[4]) {
        f[0] = as_float(v.x);
        f[1] = as_float(v.y);
        f[2] = as_float(v.z);
        f[3] = as_float(v.w);
    }
    // acc + sum of the squares of the vector's elements, in element order
    static __device__ __forceinline__ float sumsq(const u32x4 &v, float acc) {
        float f[4];
        unpack(v, f);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(f[k], f[k], acc);
        return acc;
    }
    static __device__ __forceinline__ u32x4 pack(const float (&f)[4]) {
        u32x4 v;
        v.x = as_u32(f[0]);
        v.y = as_u32(f[1]);
        v.z = as_u32(f[2]);
        v.w = as_u32(f[3]);
        return v;
    }
};

__device__ __forceinline__ float bf16_lo(uint32_t d) { return as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return as_float(d & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <>
struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ float load(const bf16_t *p) {
        return __builtin_bit_cast(float, (uint32_t)p->bits << 16);
    }
    static __device__ __forceinline__ void store(bf16_t *p, float v) {
        p->bits = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
    static __device__ __forceinline__ float rounded(float v) {
        return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v) << 16);
    }
    static __device__ __forceinline__ void unpack(const u32x4 &v, float (&f)[8]) {
        f[0] = bf16_lo(v.x);
        f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y);
        f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z);
        f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w);
        f[7] = bf16_hi(v.w);
    }
    // acc + sum of squares with v_dot2_f32_bf16: each bf16 product is exact in
    // fp32; pairs are added in element order.
    static __device__ __forceinline__ float sumsq(const u32x4 &v, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), acc, false);
        return acc;
    }
    static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
        u32x4 v;
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
        return v;
    }
};

__device__ __forceinline__ float f16_lo(uint32_t d) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(d & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t d) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> 16)); }
// The fp32 values are rounded once, to nearest even, to fp16. The empty asm
// makes them opaque fp32 registers first: otherwise the compiler may fold the
// conversion into the fma that produced them (v_fma_mixlo/mixhi_f16, which
// rounds the exact fma result to fp16), and whether it does depends on the
// code around the call, so two kernels computing the same fp32 value could
// store different fp16 bits.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    asm("" : "+v"(lo), "+v"(hi));
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <>
struct Elem<f16_t> {
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ float load(const f16_t *p) { return (float)__builtin_bit_cast(_Float16, p->bits); }
    static __device__ __forceinline__ void store(f16_t *p, float v) {
        asm("" : "+v"(v));  // one rounding of the fp32 value, as in pack_f16x2
        p->bits = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
    static __device__ __forceinline__ float rounded(float v) {
        asm("" : "+v"(v));
        return (float)(_Float16)v;
    }
    static __device__ __forceinline__ void unpack(const u32x4 &v, float (&f)[8]) {
        f[0] = f16_lo(v.x);
        f[1] = f16_hi(v.x);
        f[2] = f16_lo(v.y);
        f[3] = f16_hi(v.y);
        f[4] = f16_lo(v.z);
        f[5] = f16_hi(v.z);
        f[6] = f16_lo(v.w);
        f[7] = f16_hi(v.w);
    }
    // acc + sum of squares with v_dot2_f32_f16: each fp16 product is exact in
    // fp32; pairs are added in element order.
    static __device__ __forceinline__ float sumsq(const u32x4 &v, float acc) {
        acc = __builtin_amdgcn_fdot2(as_f16x2(v.x), as_f16x2(v.x), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(v.y), as_f16x2(v.y), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(v.z), as_f16x2(v.z), acc, false);
        acc = __builtin_amdgcn_fdot2(as_f16x2(v.w), as_f16x2(v.w), acc, false);
        return acc;
    }
    static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
        u32x4 v;
        v.x = pack_f16x2(f[0], f[1]);
        v.y = pack_f16x2(f[2], f[3]);
        v.z = pack_f16x2(f[4], f[5]);
        v.w = pack_f16x2(f[6], f[7]);
        return v;
    }
};

// Raw buffer resource (stride 0): `bytes` is the record count. Word 3 of the
// descriptor selects 32-bit data format, the value used for raw (untyped)
// buffer access on CDNA. The base pointer must be wave-uniform.
constexpr int kBufWord3 = 0x00020000;
// Cache-policy bits of the buffer accesses (CDNA3/4: bit 0 sc0, bit 1 nt,
// bit 4 sc1). Rows are streamed exactly once; measured on MI355X (HIP-graph
// timed, inputs rotating past the 256 MB MALL), the non-temporal hint pays on
// the forward's stores, on the forward's loads of wavefront-wide rows (0-18%
// from 1024 x 1024 to 65536 x 4096; the host passes that choice as
// `stream_ld`, so a caller whose input is still cache-resident can turn it
// off: there it cost 7% at 4096 x 4096), and on both the backward's loads and
// stores. It costs 1.6% on the loads of narrow rows (QK-norm's 128). The
// defaults below are those measurements; -D overrides exist to re-measure.
constexpr int kNonTemporal = 2;
#ifndef RMSN_FWD_LOAD_AUX
#define RMSN_FWD_LOAD_AUX 2         // streaming forward loads
#endif
#ifndef RMSN_FWD_NARROW_LOAD_AUX
#define RMSN_FWD_NARROW_LOAD_AUX 0  // the other forward loads
#endif
#ifndef RMSN_FWD_STORE_AUX
#define RMSN_FWD_STORE_AUX 2
#endif
#ifndef RMSN_BWD_LOAD_AUX
#define RMSN_BWD_LOAD_AUX 2
#endif
#ifndef RMSN_BWD_STORE_AUX
#define RMSN_BWD_STORE_AUX 2
#endif
#ifndef RMSN_BWD_PARTIAL_AUX
#define RMSN_BWD_PARTIAL_AUX 0  // the backward's partial dW rows (read back by the combine)
#endif
constexpr uint32_t kOff = 0x80000000u;  // an offset past every record count used here

struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void *base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufWord3)) {}
    template <int AUX = 0>
    __device__ __forceinline__ u32x4 load16(uint32_t off) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
    template <int AUX = 0>
    __device__ __forceinline__ void store16(uint32_t off, const u32x4 &v) const {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(g32x4, v), r, off, 0, AUX);
    }
    __device__ __forceinline__ float load4(uint32_t off) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    __device__ __forceinline__ void store4(uint32_t off, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    }
};

// Hide a packed vector's value from the optimiser. Used so the compiler keeps
// rows and weights packed in registers (4 VGPRs per 16 bytes) and unpacks
// them where they are used, instead of hoisting or keeping the unpacked fp32
// copies alive (twice the registers for bf16), which would cut occupancy.
__device__ __forceinline__ void keep_packed(u32x4 &v) { asm volatile("" : "+v"(v)); }

// The weights that pair with one 16-byte activation vector of format T, in
// format TW: one 16-byte vector when TW is T, two when 16-bit activations
// meet fp32 (master) weights. Weight element e of the group belongs to the
// same column as activation element e.
template <typename T, typename TW>
struct WeightVec {
    static constexpr int kPerVec = Elem<T>::kPerVec;
    static constexpr int kVecs = kPerVec * (int)sizeof(TW) / 16;
    static_assert(kVecs == 1 || kVecs == 2, "weights pair with one activation vector");
    u32x4 v[kVecs];

    // idx: the activation vector's index in its row (kOff-style masking by `in`)
    __device__ __forceinline__ void load(const Buf &wb, int idx, bool in) {
#pragma unroll
        for (int q = 0; q < kVecs; ++q) v[q] = wb.load16(in ? (uint32_t)(idx * kVecs + q) * 16u : kOff);
    }
    __device__ __forceinline__ void keep() {
#pragma unroll
        for (int q = 0; q < kVecs; ++q) keep_packed(v[q]);
    }
    __device__ __forceinline__ void unpack(float (&f)[kPerVec]) const {
        if constexpr (kVecs == 1) {
            Elem<TW>::unpack(v[0], f);
        } else {
            float a[4], b[4];
            Elem<float>::unpack(v[0], a);
            Elem<float>::unpack(v[1], b);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = a[e];
                f[4 + e] = b[e];
            }
        }
    }
};

// ---- lane-group sums ------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// DPP controls (GCN/CDNA encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// ds_swizzle bit-mask mode: and 0x1F, or 0, xor 0x10 -> partner lane ^ 16 (within 32).
constexpr int kSwizzleXor16 = 0x401F;

// Sum over aligned groups of G lanes (G a power of two, 1..64); every lane of
// a group receives the group's sum. After each step all lanes of the merged
// group hold the same value (a + b == b + a in IEEE arithmetic), so the
// result is uniform and its rounding does not depend on the lane.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group must be a power of two <= 64");
    if constexpr (G >= 2) v += dpp<kQuadXor1>(v);
    if constexpr (G >= 4) v += dpp<kQuadXor2>(v);
    // After the quad steps every lane of a quad holds the quad sum, so the
    // mirror permutations pair each lane with a lane of the neighbouring quad
    // (half-row) or half-row (row).
    if constexpr (G >= 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (G >= 16) v += dpp<kRowMirror>(v);
    if constexpr (G >= 32)
        v += __builtin_bit_cast(float,
                                __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16));
    if constexpr (G >= 64) {
        float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        v = lo + hi;
    }
    return v;
}

// Sum over a row group of LPR lanes. For LPR <= 64 the group lives inside one
// wavefront. For LPR > 64 the group is LPR/64 whole wavefronts: each wave
// reduces itself, writes one value to LDS, and after a barrier every lane adds
// the wave partials in wave order. `slots` must hold 2 * (WG / 64) floats;
// `parity` alternates between consecutive calls so one barrier per call
// suffices (a slot is rewritten only after every wave has passed the barrier
// of the following call, which comes after its reads of this one).
template <int LPR, int WG>
__device__ __forceinline__ float row_sum(float v, float *slots, int parity) {
    if constexpr (LPR <= 64) {
        return group_sum<LPR>(v);
    } else {
        constexpr int kWaves = WG / 64;
        constexpr int kWavesPerRow = LPR / 64;
        v = group_sum<64>(v);
        const int wave = threadIdx.x >> 6;
        float *buf = slots + parity * kWaves;
        if ((threadIdx.x & 63) == 0) buf[wave] = v;
        __syncthreads();
        const int first = wave - (wave % kWavesPerRow);
        float s = buf[first];
#pragma unroll
        for (int k = 1; k < kWavesPerRow; ++k) s += buf[first + k];
        return s;
    }
}

// Sum over the whole workgroup, whose size (a multiple of 64, at most WG) is
// set at launch: as row_sum with one row per workgroup, the wave partials
// added in wave order. `slots` must hold 2 * (WG / 64) floats; `parity` as in
// row_sum.
template <int WG>
__device__ __forceinline__ float wg_sum(float v, float *slots, int parity) {
    v = group_sum<64>(v);
    const int waves = (int)(blockDim.x >> 6);
    float *buf = slots + parity * (WG / 64);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = buf[0];
    for (int k = 1; k < waves; ++k) s += buf[k];
    return s;
}

}  // namespace rmsn
