// pkv_device.h -- device-side building blocks for the gfx950 attention kernels.
//
// Lane layouts (verified on gfx950 with an in-bounds probe of each builtin):
//  v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16]
//      (e = 0..7) and C[4*(l/16)+i][l%16] (i = 0..3).
//  v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32)+e], B[8*(l/32)+e][l%32]
//      and C[8*(i/4) + 4*(l/32) + i%4][l%32] (i = 0..15).
//  ds_read_b64_tr_b16: inside each group of 16 lanes, output lane i, element e is
//      element i%4 of the 8-byte chunk addressed by lane 4e + i/4 of the group;
//      i.e. lanes 4e..4e+3 address row e of a 4 x 16 block and lane i receives
//      column i.
//  v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3): lane l holds A row l%32 and B
//      column l%32, 32 bytes each whose k index depends only on (l/32, byte),
//      the same for A and B; C as for the 32x32 bf16 MFMA.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// S += A B on e4m3fn operands (32 bytes per lane each, k layout as noted at
// the top), fp32 accumulation; no block scaling.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
    const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Transposed 4 x b16 read from LDS (see the layout note at the top).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Transposed 8-bit LDS read: in each group of 16 lanes, byte j of lane l's
// result is byte l % 8 of the 8 bytes that lane 2 j + (l % 16) / 8 of the
// group addresses.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four e4m3fn bytes (one dword) -> four bf16 packed in two dwords, with
// gfx950's direct fp8 -> bf16 conversion (scale 1): one instruction per two
// values. Exact: every e4m3fn value is representable in bf16.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    return r;
}

// Eight e4m3fn bytes -> eight bf16 (one 16-byte MFMA operand).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
    u32x2 a = fp8x4_to_bf16x4(w.x), b = fp8x4_to_bf16x4(w.y);
    return u32x4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Keep LDS traffic of one wave in program order and visible to its own later
// reads: wait for outstanding LDS operations and stop the compiler moving
// memory operations across this point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Logical position -> (logical block, offset in block). Page sizes that are
// powers of two (bs_shift >= 0) use a shift and a mask; others divide.
__device__ __forceinline__ int32_t page_index(int32_t pos, int32_t bs, int32_t bs_shift) {
    return bs_shift >= 0 ? pos >> bs_shift : pos / bs;
}
__device__ __forceinline__ int32_t page_offset(int32_t pos, int32_t bs, int32_t bs_shift) {
    return bs_shift >= 0 ? pos & (bs - 1) : pos % bs;
}

// Physical cache row (block * block_size + offset) of logical key `pos`
// (the host guarantees num_blocks * block_size < 2^31).
// block_table == nullptr means the flat layout: row = flat_base + pos.
__device__ __forceinline__ int32_t kv_row(const int32_t* __restrict__ bt_row, int32_t pos, int32_t bs,
                                          int32_t bs_shift, int32_t flat_base) {
    if (bt_row == nullptr) return flat_base + pos;
    return bt_row[page_index(pos, bs, bs_shift)] * bs + page_offset(pos, bs, bs_shift);
}

}  // namespace pkv
