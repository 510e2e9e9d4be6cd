// pkv_common.h -- device helpers shared by the attention kernel sources
// (pkv_attn.hip, pkv_prefill_wide.hip).
#pragma once
#include <type_traits>

#include "pkv_device.h"
#include "pkv_kernels.h"

namespace pkv {

// ----------------------------------------------------------------- helpers

template <int N>
__device__ __forceinline__ void store_bf16(uint16_t* dst, const float* v) {
    static_assert(N % 2 == 0, "");
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            u32x4 w = {pack_bf16x2(v[i], v[i + 1]), pack_bf16x2(v[i + 2], v[i + 3]), pack_bf16x2(v[i + 4], v[i + 5]),
                       pack_bf16x2(v[i + 6], v[i + 7])};
            *(u32x4*)(dst + i) = w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            u32x2 w = {pack_bf16x2(v[i], v[i + 1]), pack_bf16x2(v[i + 2], v[i + 3])};
            *(u32x2*)(dst + i) = w;
        }
    }
}

template <int N>
__device__ __forceinline__ void store_f32(float* dst, const float* v) {
#pragma unroll
    for (int i = 0; i < N; i += 4) *(f32x4*)(dst + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
}

// 8 elements of K or V as stored: 16 bytes of bf16 or 8 bytes of fp8.
template <bool FP8>
using raw8_t = typename std::conditional<FP8, u32x2, u32x4>::type;

template <bool FP8>
__device__ __forceinline__ raw8_t<FP8> load_raw8(const void* base, int64_t elem) {
    if constexpr (FP8) return *(const u32x2*)((const uint8_t*)base + elem);
    else return *(const u32x4*)((const uint16_t*)base + elem);
}

// Widen stored elements to 8 bf16 (exact for e4m3fn).
template <bool FP8>
__device__ __forceinline__ u32x4 to_bf16x8(raw8_t<FP8> r) {
    if constexpr (FP8) return fp8x8_to_bf16x8(r);
    else return r;
}

template <bool FP8>
__device__ __forceinline__ u32x4 load_kv8(const void* base, int64_t elem) {
    return to_bf16x8<FP8>(load_raw8<FP8>(base, elem));
}

// Request owning packed token `tok` (binary search over query_start_loc).
__device__ __forceinline__ int request_of(const FwdParams& p, int64_t tok) {
    if (p.single_len > 0) return 0;
    const int32_t* qsl = p.qsl;
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Sliding window: the first key query position `pos` (its index among the
// request's keys) may see.
__device__ __forceinline__ int window_lo(const FwdParams& p, int pos) {
    return p.window_left < 0 ? 0 : max(0, pos - p.window_left);
}

// Where a request's KV ranges start: the window start of its first query
// token (no later token sees an earlier key), rounded down to 64 keys; 0
// without a window. Split s of a request covers keys
// [base + s * split_len, base + (s+1) * split_len), and the balanced decode
// list holds the request's 32-key tiles from base on.
__device__ __forceinline__ int window_base(const FwdParams& p, int q_len, int L) {
    return window_lo(p, L - q_len) & ~63;
}

// Logits soft cap in the log2 domain: x = s * log2(e) becomes
// cap_l2 * tanh(x / cap_l2) with cap_l2 = softcap * log2(e), computed as
// cap_l2 * (1 - 2 / (e^{2 s / softcap} + 1)) and e^{2 s / softcap} =
// exp2(x * cap_inv2), cap_inv2 = 2 / softcap. Saturates to +-cap_l2.
__device__ __forceinline__ float softcap_l2(float x, float cap_l2, float cap_inv2) {
    const float e = fast_exp2(x * cap_inv2);
    return cap_l2 * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
}

// ALiBi slope of query head h in the log2 domain (0 without ALiBi): the
// score of query position i and key j gets -slope * |i - j| added.
__device__ __forceinline__ float alibi_l2(const FwdParams& p, int h) { return p.alibi ? p.alibi[h] * kLog2e : 0.f; }

// Sink logit of query head h in the log2 domain (-inf without sinks).
__device__ __forceinline__ float sink_l2(const FwdParams& p, int h) {
    return p.sinks ? p.sinks[h] * kLog2e : -INFINITY;
}

// Final normalisation of one row: m is the log2-domain maximum the running
// sum l and the accumulator are taken against, vsc the value scale. Returns
// the factor that turns the accumulator into the output, and the row's lse
// (natural log). A sink logit (log2 domain; -inf: none) joins the normaliser
// and adds no value: factor = vsc / (l + 2^(sink - m)), with both terms taken
// against max(m, sink) so neither can overflow.
//
// lc is the sum the accumulator's own weights add up to: where the
// probabilities are rounded to bf16 for the P V product, the sum of those
// rounded values, so that the output is a weighted mean of value rows whose
// weights add up to one (for a row dominated by one key the output is then
// that key's value row, however its weight was rounded). lse comes from the
// sum of the unrounded probabilities, l.
__device__ __forceinline__ void finalize_row(float m, float l, float lc, float sink2, float vsc, float& factor,
                                             float& lse) {
    if (sink2 == -INFINITY) {
        factor = lc > 0.f ? vsc / lc : 0.f;
        const float mu = m == -INFINITY ? 0.f : m;
        lse = l > 0.f ? (mu + fast_log2(l)) * kLn2 : -INFINITY;
    } else {
        const float mu = fmaxf(m, sink2);
        const float a = l > 0.f ? fast_exp2(m - mu) : 0.f;
        const float es = fast_exp2(sink2 - mu);
        factor = vsc * a / (lc * a + es);
        lse = (mu + fast_log2(l * a + es)) * kLn2;
    }
}
__device__ __forceinline__ void finalize_row(float m, float l, float sink2, float vsc, float& factor, float& lse) {
    finalize_row(m, l, l, sink2, vsc, factor, lse);
}

// acc + the two bf16 values of a packed pair (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                           acc, false);
}

// One 16-byte global -> LDS copy per lane, written by the load unit straight
// into LDS at lds_base + 16 * lane (lds_base must be wave-uniform); `off` is
// added to the global address.
template <int OFF>
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, OFF, 0);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt == 0 and leaves
// the other counters alone.
constexpr int kWaitVmcnt0 = 0x0F70;

// Rescale of the running output is skipped until a row's running maximum
// grows by more than this (log2 units): probabilities are then formed against
// a stale maximum and stay below 2^8, and the final normalisation by the same
// stale maximum keeps the result exact.
constexpr float kLazyRescale = 8.f;


// K/V tiles of 64 keys live in LDS row-major (a key's head_size bf16
// elements contiguous). A 64-lane tile copy moves whole cache rows: each group
// of head_size / 8 lanes reads one row, 16 bytes per lane, and the load unit
// writes them at 16 * lane, so one copy fills 1 KB of consecutive rows (a
// "copy group"). The layout then adds PAD bytes after each copy group and
// permutes the 16-byte chunks of row r: chunk c sits at position c ^ sw(r).
// PAD and sw are chosen per head size so that, with the 64 four-byte LDS banks
// of gfx950 (16 lanes per clock for 16-byte reads, 32 for 8-byte reads), the
// K fragment reads and the transposed V reads of the MFMA loop hit every bank
// at most once. (Copying one 16-byte column of 64 rows per instruction
// instead, as a chunk-major layout requires, moves the same bytes far more
// slowly.)
template <int HD>
struct PfLayout;
template <>
struct PfLayout<64> {
    static constexpr int PAD = 16, A0 = 0, A1 = 4, A2 = 2, A3 = 0;
};
template <>
struct PfLayout<128> {
    static constexpr int PAD = 16, A0 = 4, A1 = 8, A2 = 0, A3 = 0;
};
template <>
struct PfLayout<256> {
    static constexpr int PAD = 64, A0 = 8, A1 = 0, A2 = 1, A3 = 2;
};
template <int HD>
struct PfTile {
    using L = PfLayout<HD>;
    static constexpr int CPR = HD / 8;                 // 16-byte chunks per row
    static constexpr int RP = CPR * 16;                // bytes per row
    static constexpr int KPI = 64 / CPR;               // rows per copy group
    static constexpr int GP = 1024 + L::PAD;           // bytes per copy group
    static constexpr int SWMASK = L::A0 | L::A1 | L::A2 | L::A3;
    static_assert(SWMASK < CPR && KPI * RP == 1024, "");
    static __device__ __forceinline__ int sw(int r) {
        return (L::A0 * (r & 1)) ^ (L::A1 * ((r >> 1) & 1)) ^ (L::A2 * ((r >> 2) & 1)) ^ (L::A3 * ((r >> 3) & 1));
    }
    // byte offset of row r's first position
    static __device__ __forceinline__ int row_base(int r) { return (r / KPI) * GP + (r % KPI) * RP; }
};
// Index of the bits of x selected by mask, packed (a compile-time pext).
constexpr int pext(int x, int mask) {
    int r = 0, k = 0;
    for (int b = 0; b < 16; ++b)
        if (mask & (1 << b)) r |= ((x >> b) & 1) << k++;
    return r;
}
constexpr int popcount(int x) { return x ? (x & 1) + popcount(x >> 1) : 0; }
constexpr int kTileRows = 64;

// How a prefill workgroup finds the cache rows of a tile's keys.
//  kPgAny:  any page size; every key is translated through the block table.
//  kPgWide: the page size is a power of two of at least 16. The 16 keys a
//           wave copies in a tile start 16-aligned, so they share one page:
//           one (wave-uniform) block-table entry per wave and tile.
//  kPgFlat: no block table; K/V rows are packed like q.
constexpr int kPgAny = 0, kPgWide = 1, kPgFlat = 2;

}  // namespace pkv
