// pkv_cache.hip -- KV-cache write by slot_mapping for gfx950.
//
// The "FlashAttention deep dive" page's KV-cache update scatters this step's
// keys and values into the paged cache before attention runs: token t goes to
// slot slot_mapping[t], i.e. block slot / block_size, row slot % block_size of
// the [num_blocks, block_size, num_kv_heads, head_size] cache. Because the
// cache rows of consecutive blocks are contiguous, that row is simply row
// `slot` of the cache seen as [num_blocks * block_size, num_kv_heads * head_size].
//
// One thread moves 8 consecutive elements (16 bytes of bf16); a token's K and V
// rows are read and written with full, coalesced 16-byte accesses.
//
// FP8 (OCP e4m3fn) encoding: y = x / scale (correctly rounded binary32
// division), saturated to +-448 (the hardware conversion would produce NaN
// above 464), NaN kept as 0x7F with the sign of y, then the hardware
// round-to-nearest-even conversion.
#include "pkv_device.h"
#include "pkv_kernels.h"

namespace pkv {

enum CacheKind { kCopy = 0, kToBf16 = 1, kToFp8 = 2 };

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN stays a quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, float sc) {
    float y[4] = {__fdiv_rn(a, sc), __fdiv_rn(b, sc), __fdiv_rn(c, sc), __fdiv_rn(d, sc)};
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = __builtin_isnan(y[i]) ? 0.f : fminf(fmaxf(y[i], -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], w, true);
    uint32_t r = (uint32_t)w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (__builtin_isnan(y[i])) {
            const uint32_t code = 0x7Fu | ((__float_as_uint(y[i]) >> 24) & 0x80u);
            r = (r & ~(0xFFu << (8 * i))) | (code << (8 * i));
        }
    }
    return r;
}

// src: 8 elements as floats
template <int SRC_F32>
__device__ __forceinline__ void load8(const void* src, int64_t e, float* v) {
    if constexpr (SRC_F32) {
        const f32x4 a = *(const f32x4*)((const float*)src + e);
        const f32x4 b = *(const f32x4*)((const float*)src + e + 4);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
        const u32x4 w = *(const u32x4*)((const uint16_t*)src + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    }
}

template <int SRC_F32, int KIND>
__global__ __launch_bounds__(256) void cache_write_kernel(const void* key, const void* value, void* kc, void* vc,
                                                          const int64_t* slots, int64_t T, int64_t row_elems,
                                                          const float* ks, const float* vs) {
    const int64_t cpr = row_elems / 8;  // chunks of 8 elements per token row
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= 2 * T * cpr) return;
    const int which = (int)(idx / (T * cpr));  // 0 = key, 1 = value
    const int64_t rem = idx - which * T * cpr;
    const int64_t t = rem / cpr;
    const int64_t c = rem - t * cpr;
    const int64_t slot = slots[t];
    if (slot < 0) return;
    const void* src = which ? value : key;
    void* dst = which ? vc : kc;
    const int64_t se = t * row_elems + c * 8;
    const int64_t de = slot * row_elems + c * 8;
    if constexpr (KIND == kCopy) {
        if constexpr (SRC_F32) {
            *(f32x4*)((float*)dst + de) = *(const f32x4*)((const float*)src + se);
            *(f32x4*)((float*)dst + de + 4) = *(const f32x4*)((const float*)src + se + 4);
        } else {
            *(u32x4*)((uint16_t*)dst + de) = *(const u32x4*)((const uint16_t*)src + se);
        }
    } else if constexpr (KIND == kToBf16) {
        float v[8];
        load8<SRC_F32>(src, se, v);
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
        *(u32x4*)((uint16_t*)dst + de) = w;
    } else {
        float v[8];
        load8<SRC_F32>(src, se, v);
        const float sc = which ? *vs : *ks;
        const u32x2 w = {fp8x4(v[0], v[1], v[2], v[3], sc), fp8x4(v[4], v[5], v[6], v[7], sc)};
        *(u32x2*)((uint8_t*)dst + de) = w;
    }
}

hipError_t launch_cache_write(const void* key, const void* value, int src_f32, void* kc, void* vc, int cache_kind,
                              const int64_t* slots, int64_t T, int32_t Hkv, int32_t hd, const float* ks,
                              const float* vs, hipStream_t s) {
    const int64_t row = (int64_t)Hkv * hd;
    const int64_t n = 2 * T * (row / 8);
    dim3 grid((unsigned)((n + 255) / 256));
#define PKV_CW(SF, K) hipLaunchKernelGGL((cache_write_kernel<SF, K>), grid, dim3(256), 0, s, key, value, kc, vc, slots, T, row, ks, vs)
    if (src_f32) {
        if (cache_kind == kCopy) PKV_CW(1, kCopy);
        else if (cache_kind == kToBf16) PKV_CW(1, kToBf16);
        else PKV_CW(1, kToFp8);
    } else {
        if (cache_kind == kCopy) PKV_CW(0, kCopy);
        else PKV_CW(0, kToFp8);
    }
#undef PKV_CW
    return hipGetLastError();
}

}  // namespace pkv
