// common.h -- device helpers shared by the library's HIP kernels (gfx950 only).
// Internal to the library; nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tl {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// tile record fields
constexpr int kRecSlot = 0, kRecPos = 1, kRecRows = 2, kRecSegRows = 3, kRecSeg = 4, kRecSegTile = 5,
              kRecRowIds = 8;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------- bf16
// bf16 is the top half of a binary32: widening is a shift (low element of a
// packed pair) or a mask (high element).
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_round(float v) { return (float)(__bf16)v; }

// acc + a.lo*b.lo + a.hi*b.hi over packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float dot8(const u32x4_t a, const u32x4_t b, float acc) {
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    acc = dot2(a.w, b.w, acc);
    return acc;
}

// ---------------------------------------------------------------- MFMA
// D[16x16] += A[16x32] * B[32x16] in bf16 with fp32 accumulation.
// Operand layout used throughout: lane l feeds row (A) / column (B) l % 16
// with the 8 consecutive k values 8*(l/16) .. +8 of the 32-wide k block; the
// same k assignment on both operands makes the product independent of how
// the hardware orders k inside a lane group.  Result: lane l holds column
// l % 16, rows 4*(l/16) + i for i = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t a, const u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4_t ld16(const void *p) {
    return *reinterpret_cast<const u32x4_t *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4_t v) { *reinterpret_cast<u32x4_t *>(p) = v; }
__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }
// Cache policy.  Bytes a kernel touches once -- A rows, output rows, the B
// rows of adapters that serve few rows -- are loaded and stored with the
// nontemporal hint, so they do not push out of L2 what is read again: x rows
// gathered by the experts of a token, B rows shared by the tiles of a long
// segment.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4_t ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
__device__ __forceinline__ uint32_t ld4_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint2 ld8_stream(const void *p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st4_stream(void *p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
}
__device__ __forceinline__ void st8_stream(void *p, uint2 v) {
    __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t *>(p));
}
__device__ __forceinline__ void st16_stream(void *p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}
// A B row load: streamed (S) or kept in the caches for later tiles.
template <bool S>
__device__ __forceinline__ u32x4_t ld16_b(const void *p) {
    return S ? ld16_stream(p) : ld16(p);
}

// ---------------------------------------------------------------- buffer addressing
// A buffer resource spans [base, base + bytes), bytes < 2^31.  A buffer load
// at an offset outside it returns zero and a store there is dropped, so a
// masked access is a select of its offset rather than a branch around it
// (which would also keep the compiler from counting the loads in flight).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;   // descriptor word 3 on gfx9: 32-bit data format
constexpr uint32_t kOob = 0x80000000u;  // an offset past the end of every resource made here
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufWord3);
}
// (cache-policy operand: 0 default, kNt the nontemporal hint)
constexpr int kNt = 2;
template <int CP = 0>
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP));
}
template <int CP = 0>
__device__ __forceinline__ uint2 buf_ld8(rsrc_t r, uint32_t off) {
    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP));
    return make_uint2(v.x, v.y);
}
template <int CP = 0>
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, off, 0, CP);
}

// ---------------------------------------------------------------- DPP lane sums
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of 2^lg lanes (lg <= 4); every lane of a group gets
// the group's total.  quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at xor 1
// and xor 2; row_half_mirror (i <-> 7-i) and row_mirror (i <-> 15-i) then
// join quads into 8 and 16 lanes.
__device__ __forceinline__ float group_sum(float v, int lg) {
    if (lg >= 1) v += dpp_mov<0xB1>(v);
    if (lg >= 2) v += dpp_mov<0x4E>(v);
    if (lg >= 3) v += dpp_mov<0x141>(v);
    if (lg >= 4) v += dpp_mov<0x140>(v);
    return v;
}

// ---------------------------------------------------------------- wave/block scans
// Inclusive scans over the 64 lanes of a wave with DPP moves, no LDS
// traffic: shifts by 1, 2, 4 and 8 lanes within each row of 16 lanes (a
// lane whose source lies outside its row adds 0), then lane 15 of each row
// added to the next row (rows 1 and 3) and lane 31 added to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_in(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, true);
}
constexpr int kDppRowShr = 0x110, kDppBcast15 = 0x142, kDppBcast31 = 0x143;

__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_in<kDppRowShr + 1, 0xf>(v);
    v += dpp_in<kDppRowShr + 2, 0xf>(v);
    v += dpp_in<kDppRowShr + 4, 0xf>(v);
    v += dpp_in<kDppRowShr + 8, 0xf>(v);
    v += dpp_in<kDppBcast15, 0xa>(v);
    v += dpp_in<kDppBcast31, 0xc>(v);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

struct Int3 {
    int a, b, c;
};
__device__ __forceinline__ Int3 operator+(Int3 x, Int3 y) { return {x.a + y.a, x.b + y.b, x.c + y.c}; }

__device__ __forceinline__ Int3 wave_incl_scan3(Int3 v) {
    return {wave_incl_scan(v.a), wave_incl_scan(v.b), wave_incl_scan(v.c)};
}

// Exclusive scan over the NT threads of a block; every thread must call it.
// `scratch` holds NT/64 + 1 entries.  Returns the exclusive prefix and the
// block total.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int &total) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = wave_id();
    int inc = wave_incl_scan(v);
    if (lane == kWave - 1) scratch[w] = inc;
    __syncthreads();
    if (w == 0) {
        int s = lane < NW ? scratch[lane] : 0;
        int si = wave_incl_scan(s);
        if (lane < NW) scratch[lane] = si - s;
        if (lane == NW - 1) scratch[NW] = si;
    }
    __syncthreads();
    int r = scratch[w] + inc - v;
    total = scratch[NW];
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ Int3 block_excl_scan3(Int3 v, Int3 *scratch, Int3 &total) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = wave_id();
    Int3 inc = wave_incl_scan3(v);
    if (lane == kWave - 1) scratch[w] = inc;
    __syncthreads();
    if (w == 0) {
        Int3 s = lane < NW ? scratch[lane] : Int3{0, 0, 0};
        Int3 si = wave_incl_scan3(s);
        if (lane < NW) scratch[lane] = Int3{si.a - s.a, si.b - s.b, si.c - s.c};
        if (lane == NW - 1) scratch[NW] = si;
    }
    __syncthreads();
    Int3 p = scratch[w];
    Int3 r = {p.a + inc.a - v.a, p.b + inc.b - v.b, p.c + inc.c - v.c};
    total = scratch[NW];
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------- workspace control line
constexpr int kCtlError = 0;  // set when a bounded wait gave up
constexpr int kCtlGen = 1;    // tag of the last completed call on this workspace (0: none yet)
constexpr int kCtlDone = 2;   // finished tiles of the running call

// Call tags have the top bit set and never equal 0xFFFFFFFF: they run
// 0x80000001, 0x80000002, ... 0xFFFFFFFE and start over.  Whatever else a
// workspace may hold where a later call keeps its flags and partials -- zero
// fill, or the int32 metadata a MoE call builds in the same workspace (row
// ids, positions, slots, counts: all in [0, 2^31)) -- can therefore never
// read as the current call's tag, and neither can an earlier call's tag.
__device__ __forceinline__ uint32_t next_tag(uint32_t last) {
    return (last >= 0x80000001u && last < 0xFFFFFFFEu) ? last + 1u : 0x80000001u;
}

// ---------------------------------------------------------------- device-scope sync
__device__ __forceinline__ int atomic_add_release(int *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_acqrel(int *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_acquire(const int *p) {
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_relaxed(const int *p) {
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_relaxed(int *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int xchg_relaxed(int *p, int v) {
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 64-bit words read and written as single atomic units: a value with the
// tag of the call that wrote it travels in one word, so a reader that sees
// the tag also sees the value, with no fence on either side.
__device__ __forceinline__ void store_word64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_word64(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
    return ((uint64_t)tag << 32) | __float_as_uint(v);
}

}  // namespace tl
