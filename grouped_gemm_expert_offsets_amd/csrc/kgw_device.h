// Device-side building blocks shared by the bf16 and fp8 K-grouped kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kgw {

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

typedef __attribute__((address_space(3))) char lds_char;
// Global-memory views: loads and stores through these are `global_*`, not
// `flat_*`, instructions (flat ones also count on the LDS counter).
typedef __attribute__((address_space(1))) char gbl_char;
typedef __attribute__((address_space(1))) i32x4 gbl_i32x4;
typedef __attribute__((address_space(1))) f32x4 gbl_f32x4;

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, kBufferWord3);
}

__device__ __forceinline__ i32x4 buffer_load_16B(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

__device__ __forceinline__ uint8_t buffer_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
}

// Buffer resource of a raw byte buffer as four SGPR words (for inline asm).
// Loads at byte offsets >= num_bytes return zero without touching memory.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t num_bytes = 0xFFFFFFFFu) {
    const uint64_t a = (uint64_t)base;
    i32x4 r = {(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)num_bytes, kBufferWord3};
    r[0] = __builtin_amdgcn_readfirstlane(r[0]);
    r[1] = __builtin_amdgcn_readfirstlane(r[1]);
    r[2] = __builtin_amdgcn_readfirstlane(r[2]);
    return r;
}

// LDS byte address of a __shared__ location (wave-uniform callers only).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Direct global -> LDS load (buffer_load_dwordx4 ... lds): every lane fetches 16
// bytes at byte offset `voff` of the buffer and the wave's 64 results land
// contiguously in LDS at byte address `lds_dst` + 16 * lane (`lds_dst` is
// wave-uniform and travels in M0).  Issued as inline asm so the compiler does
// not track it: otherwise it must assume the write may alias any LDS read and
// waits for all such loads (vmcnt(0)) before every read, which would collapse
// the multi-stage ring.  Callers order these loads with wait_vmcnt + barrier.
__device__ __forceinline__ void dma_16B(i32x4 rsrc, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_dst) : "memory");
}

// Narrow direct loads to LDS: every lane fetches the byte (dma_1B, zero-extended)
// or the dword (dma_4B) at `voff` of the buffer, and lane L's value lands as the
// dword at `lds_dst` + 4 * L.  Same ordering rules as dma_16B.
__device__ __forceinline__ void dma_1B(i32x4 rsrc, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_ubyte %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_dst) : "memory");
}
__device__ __forceinline__ void dma_4B(i32x4 rsrc, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(lds_dst) : "memory");
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left unconstrained); gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// s_waitcnt lgkmcnt(N) alone: at most N of this wave's LDS / scalar reads are still
// outstanding.  LDS reads return in issue order, so every LDS read issued before the
// last N has returned.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// Workgroup barrier without the memory fence __syncthreads() adds: the fence
// would wait for every outstanding direct-to-LDS load, collapsing the pipeline.
// Callers order their own memory with wait_vmcnt / lgkmcnt waits.  The empty
// asm statements keep the compiler from moving memory accesses across the
// barrier (the barrier intrinsic itself does not order memory).
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS accessors on explicit address-space-3 pointers (ds_read / ds_write).
__device__ __forceinline__ void lds_store_16B(lds_char* base, uint32_t off, i32x4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) i32x4*>(base + off) = v;
}
__device__ __forceinline__ i32x4 lds_load_16B(const lds_char* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(base + off);
}
__device__ __forceinline__ i32x2 lds_load_8B(const lds_char* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) i32x2*>(base + off);
}
__device__ __forceinline__ int lds_load_4B(const lds_char* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) int*>(base + off);
}

// Transposing LDS reads (gfx950).  Within each group of 16 lanes, lane 4b+c
// (tr16) or 2b+c (tr8) names one 8-byte piece of row b of a 4x16 (16-bit) or
// 8x16 (8-bit) block; lane i receives column i of that block, rows in order.
__device__ __forceinline__ i16x4 lds_read_tr16(const lds_char* base, uint32_t off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(base + off));
}
__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char* base, uint32_t off) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(base + off));
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// e4m3 x e4m3 -> f32 with one E8M0 scale byte per lane for each operand (byte 0 of sa/sb).
__device__ __forceinline__ f32x16 mfma_scale_e4m3_32x32x64(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// UE8M0 scale byte -> the fp32 value 2^(s - 127): exponent field s for 1..254,
// the subnormal 2^-127 for 0, NaN for 0xFF.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    const uint32_t bits = s == 0u ? 0x00400000u : (s == 255u ? 0x7FC00000u : (s << 23));
    return __builtin_bit_cast(float, bits);
}

// UE8M0 scale byte -> the scale operand of the v_cvt_scalef32_* conversions.  Those
// instructions take only the exponent field of their fp32 scale operand as the scale (a
// GPU probe over all 256 field values and a few mantissas: the mantissa bits change
// nothing, field 0 scales by 2^-127 and field 255 gives NaN, exactly as e8m0_to_f32's
// value does), so the byte moved into that field is the operand: one shift instead of
// the two special cases.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t s) { return __builtin_bit_cast(float, s << 23); }

// Two e4m3 bytes (bytes 2*HI and 2*HI+1 of `packed`) -> two bf16 (low half = lower
// byte) multiplied by `scale`.  For a power-of-two scale the result is exact:
// every e4m3 value times 2^k is a bf16 number while it stays in range.
template <bool HI>
__device__ __forceinline__ int cvt_e4m3x2_bf16(int packed, float scale) {
    return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, scale, HI));
}

// Eight e4m3 values (k order in byte order) -> eight bf16 in MFMA operand order.
__device__ __forceinline__ i32x4 cvt_e4m3x8_bf16(i32x2 v, float scale) {
    const i32x4 r = {cvt_e4m3x2_bf16<false>(v[0], scale), cvt_e4m3x2_bf16<true>(v[0], scale),
                     cvt_e4m3x2_bf16<false>(v[1], scale), cvt_e4m3x2_bf16<true>(v[1], scale)};
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 l = (__bf16)lo;   // round to nearest even (v_cvt_pk_bf16_f32)
    __bf16 h = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// IEEE binary16, round to nearest even (v_cvt_f16_f32; overflow gives infinity).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const _Float16 l = (_Float16)lo, h = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Output element kinds (the values of kgw_out_dtype_t).
constexpr int kOutF32 = 0, kOutBf16 = 1, kOutF16 = 2;

// Pack / unpack two values of a 16-bit output kind.
template <int OUT>
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    static_assert(OUT == kOutBf16 || OUT == kOutF16, "16-bit output kinds only");
    if constexpr (OUT == kOutBf16) return pack_bf16x2(lo, hi);
    else return pack_f16x2(lo, hi);
}
template <int OUT>
__device__ __forceinline__ float half_lo(uint32_t w) {
    if constexpr (OUT == kOutBf16) return bf16_lo(w);
    else return f16_lo(w);
}
template <int OUT>
__device__ __forceinline__ float half_hi(uint32_t w) {
    if constexpr (OUT == kOutBf16) return bf16_hi(w);
    else return f16_hi(w);
}

// Workgroups are dealt round-robin over the XCDs; give the workgroups of one
// XCD a contiguous run of logical slots so that concurrently running tiles on
// one XCD share operand panels in that XCD's L2.
__device__ __forceinline__ int xcd_slot(int bid, int grid, int num_xcds) {
    if (num_xcds <= 1 || grid % num_xcds != 0) return bid;
    return (bid % num_xcds) * (grid / num_xcds) + bid / num_xcds;
}

// Tile order inside one expert: columns of `group_m` M-tiles, walking M first,
// so a run of consecutive items covers a compact block of the output.
__device__ __forceinline__ void tile_coords(int local, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int per_group = group_m * tiles_n;
    const int grp = local / per_group;
    const int first = grp * group_m;
    const int gm = min(group_m, tiles_m - first);
    const int in = local - grp * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

}  // namespace kgw
